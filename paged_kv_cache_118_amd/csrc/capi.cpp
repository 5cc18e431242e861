// libpa C ABI: argument checks, launch configuration and dispatch.
// The operations themselves are defined in include/pa.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <unordered_set>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

using namespace pa;

int pa::device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 256;
  return cus;
}

namespace {

constexpr int kPartGranule = 256;  // fixed chunks are a multiple of this many tokens
// Every GQA group (G >= 2) goes to the matrix cores where they support the
// shape: the MFMA kernel reads each K/V token once per kv head, the VALU
// kernel once per q head, and at G = 2 and 3 the MFMA kernel ran 1.9-2.8x
// faster (bf16, D 128, block sizes 16 and 32, contexts 1-8K).
constexpr int kMfmaMinGroup = 2;
// The token-balanced split keeps per-sequence prefix sums in LDS.
constexpr int kMaxSplitSeqs = 8192;
// Workers per CU: the decode kernel's occupancy with the launch's dynamic LDS
// (one round of workers fills the chip), capped for the VALU kernel at
// kValuWorkersPerCu.  Every worker boundary inside an item costs one more
// fp32 partial written and merged, so fewer, longer shares pay off once the
// CU is kept busy: 8 VALU workers per CU measured about 1% faster than 16 on
// the OPT-13B-shaped workload.
constexpr int kValuWorkersPerCu = 8;
constexpr int kWavesPerWorkgroup = 4;  // both split kernels launch 4-wavefront workgroups

int device_lds_per_cu() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 64 * 1024;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
          hipSuccess ||
      v <= 0)
    return 64 * 1024;
  return v;
}

int waves_per_cu(bool mfma, pa_dtype dt, int head_dim, size_t lds_bytes) {
  static int cache[2][3][5] = {};
  int dsel = head_dim == 64 ? 0 : head_dim == 128 ? 1 : head_dim == 256 ? 2 : 3;
  if (dsel > 2) dsel = 3;
  int& x = cache[mfma ? 1 : 0][(int)dt][dsel];
  if (x == 0)
    x = mfma ? decode_mfma_waves_per_cu(dt, head_dim)
             : std::min(kValuWorkersPerCu, decode_valu_waves_per_cu(dt, head_dim));
  // resident workgroups are also bounded by the LDS the split keeps per workgroup
  static const int lds_cu = device_lds_per_cu();
  const int by_lds = (int)(lds_cu / std::max<size_t>(lds_bytes, 1)) * kWavesPerWorkgroup;
  return std::max(kWavesPerWorkgroup, std::min(x, by_lds));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(pa_dtype d) { return d == PA_F32 ? 4 : 2; }

bool dtype_ok(pa_dtype d) { return d == PA_F32 || d == PA_F16 || d == PA_BF16; }

bool block_size_ok(int bs) {
  return bs == 1 || bs == 2 || bs == 4 || bs == 8 || (bs >= 16 && bs % 16 == 0);
}

bool validate_enabled() {
  static int v = -1;
  if (v < 0) {
    const char* e = std::getenv("PA_VALIDATE");
    v = (e && e[0] && e[0] != '0') ? 1 : 0;
  }
  return v == 1;
}

enum class Path { kValu, kMfma, kGeneric };

Path choose_path(pa_dtype dt, int head_dim, int block_size, int group) {
  if (group >= kMfmaMinGroup && decode_mfma_supported(dt, head_dim, block_size, group))
    return Path::kMfma;
  if (decode_valu_supported(dt, head_dim, block_size)) return Path::kValu;
  return Path::kGeneric;
}

// How one pa_decode call divides its work (decode_split.h).
struct Plan {
  Path path;
  int split;        // 0: one worker per item, 1: token-balanced split
  int step;         // tokens per worker step
  int items_per_seq;
  int rows_per_item;
  int part_steps;   // split 1: steps per partition (shares are whole partitions), 0 = none
  int num_workers;
  size_t ws_bytes;
  size_t pre_off, ppre_off;
};

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

Plan make_plan(int num_seqs, int hq, int hkv, int head_dim, int block_size, int len_cap,
               int partition_size, pa_dtype dt) {
  Plan p{};
  const int group = hkv > 0 ? hq / hkv : 1;
  p.path = choose_path(dt, head_dim, block_size, group);
  p.step = p.path == Path::kMfma ? 32 : 16;
  p.items_per_seq = p.path == Path::kMfma ? hkv : hq;
  p.rows_per_item = p.path == Path::kMfma ? group : 1;
  const int64_t items = (int64_t)num_seqs * p.items_per_seq;
  const int64_t item_steps = ((int64_t)len_cap + p.step - 1) / p.step;
  p.split = (p.path != Path::kGeneric && partition_size >= 0 && len_cap > 0 &&
             num_seqs <= kMaxSplitSeqs && items * item_steps < (int64_t)1 << 30)
                ? 1
                : 0;
  if (!p.split) {
    p.num_workers = (int)items;
    return p;
  }
  p.part_steps = partition_size > 0 ? std::max(1, partition_size / p.step) : 0;
  p.num_workers =
      device_cus() * waves_per_cu(p.path == Path::kMfma, dt, head_dim, split_lds_bytes(num_seqs));
  const size_t slots = (size_t)(items + p.num_workers);  // partial of item i by worker w: i + w
  p.pre_off = round_up(slots * part_record(p.rows_per_item, head_dim) * 4, 256);
  p.ppre_off = p.pre_off + round_up(((size_t)num_seqs + 1) * 4, 256);
  p.ws_bytes = p.ppre_off + round_up(((size_t)num_seqs + 1) * 4, 256);
  return p;
}

// ----------------------------------------------------- shared-prefix plan --
// pa_decode_shared: the tail pass uses the token-balanced split of a plain
// decode (with the larger LDS of its scan), the prefix pass its own split
// over (group, kv head) items with 16-row records; the workspace holds the
// tail split's, then the prefix records, the prefix step prefixes and the
// group of each sequence.
struct CascadePlan {
  bool ok;  // false: the plain decode runs instead
  Plan tail;
  int p_workers;
  size_t p_off, p_pre_off, grp_off, ws_bytes;
};

bool prefix_pass_supported(pa_dtype dt, int head_dim, int block_size, int group) {
  return (dt == PA_F16 || dt == PA_BF16) && (head_dim == 64 || head_dim == 128) &&
         (block_size == 8 || block_size == 16 || block_size % 32 == 0) && group <= kPrefixRows;
}

CascadePlan make_cascade_plan(int num_seqs, int num_groups, int hq, int hkv, int head_dim,
                              int block_size, int len_cap, pa_dtype dt) {
  CascadePlan c{};
  c.tail = make_plan(num_seqs, hq, hkv, head_dim, block_size, len_cap, 0, dt);
  c.ok = num_groups > 0 && c.tail.split && num_groups <= num_seqs &&
         prefix_pass_supported(dt, head_dim, block_size, hq / hkv);
  if (!c.ok) {
    c.ws_bytes = c.tail.ws_bytes;
    return c;
  }
  // the tail pass's workers, sized with its larger LDS
  c.tail.num_workers = device_cus() * waves_per_cu(c.tail.path == Path::kMfma, dt, head_dim,
                                                   cascade_lds_bytes(num_seqs, num_groups));
  const size_t slots = (size_t)num_seqs * c.tail.items_per_seq + c.tail.num_workers;
  c.tail.pre_off = round_up(slots * part_record(c.tail.rows_per_item, head_dim) * 4, 256);
  c.tail.ppre_off = c.tail.pre_off + round_up(((size_t)num_seqs + 1) * 4, 256);
  c.tail.ws_bytes = c.tail.ppre_off + round_up(((size_t)num_seqs + 1) * 4, 256);
  const size_t p_lds = split_lds_bytes(num_groups) + sizeof(int) * (2 * (size_t)num_groups + 1);
  c.p_workers = device_cus() * waves_per_cu(true, dt, head_dim, p_lds);
  const size_t p_slots = (size_t)num_groups * hkv + c.p_workers;
  c.p_off = c.tail.ws_bytes;
  c.p_pre_off = c.p_off + round_up(p_slots * part_record(kPrefixRows, head_dim) * 4, 256);
  c.grp_off = c.p_pre_off + round_up(((size_t)num_groups + 1) * 4, 256);
  c.ws_bytes = c.grp_off + round_up((size_t)num_seqs * 16, 256);  // int4 per sequence
  return c;
}

// True when a kernel may dereference p: device memory, or pinned host memory
// mapped at the same address (pageable host memory is refused).
bool device_accessible(const void* p) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  const bool kind = at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeHost ||
                    at.type == hipMemoryTypeManaged || at.type == hipMemoryTypeUnified;
  return kind && at.devicePointer == p;
}

pa_status hip_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_EHIP; }

template <typename T>
bool copy_to_host(std::vector<T>& dst, const T* src, size_t n, hipStream_t s) {
  dst.resize(n);
  if (n == 0) return true;
  if (hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, s) != hipSuccess)
    return false;
  return hipStreamSynchronize(s) == hipSuccess;
}

}  // namespace

namespace pa {

// pa_decode and pa_decode_write: k_new / v_new null for a plain decode.
pa_status decode_impl(void* out, const void* q, const void* k_new, const void* v_new,
                      int64_t new_stride, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, float scale,
                      int32_t block_size, int32_t num_kv_heads, int32_t num_seqs,
                      int32_t num_q_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                      int32_t max_context_len, int64_t num_blocks, pa_dtype dtype,
                      int32_t partition_size, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || max_blocks_per_seq < 0 || max_context_len < 0 || num_blocks <= 0)
    return PA_EINVAL;
  if (!dtype_ok(dtype)) return PA_ENOTSUP;
  if (num_q_heads % num_kv_heads != 0) return PA_EINVAL;
  if (!std::isfinite(scale)) return PA_EINVAL;
  if (!(head_dim == 16 || head_dim == 32 || head_dim == 64 || head_dim == 128 || head_dim == 256))
    return PA_ENOTSUP;
  if (!block_size_ok(block_size)) return PA_ENOTSUP;
  if (partition_size > 0 && partition_size % kPartGranule != 0) return PA_EINVAL;
  const bool write = k_new != nullptr || v_new != nullptr;
  if (write) {
    const int es = elem_bytes(dtype);
    if (!k_new || !v_new || new_stride < (int64_t)num_kv_heads * head_dim ||
        (new_stride * es) % 16 != 0)
      return PA_EINVAL;
  }
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_EINVAL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_EINVAL;
  if (write) {
    if (!aligned16(k_new) || !aligned16(v_new)) return PA_EINVAL;
    // the new rows come straight from a caller's tensors: a host pointer
    // would fault the kernel
    if (!device_accessible(k_new) || !device_accessible(v_new)) return PA_EINVAL;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  const int64_t cap64 = std::min<int64_t>((int64_t)max_context_len,
                                          (int64_t)max_blocks_per_seq * block_size);
  const int len_cap = (int)cap64;
  // the workspace size depends on max_context_len only (what the caller sized it with)
  const Plan sized = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                               max_context_len, partition_size, dtype);
  Plan p = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, len_cap,
                     partition_size, dtype);

  DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.scale_log2e = scale * 1.4426950408889634f;
  a.block_size = block_size;
  a.num_kv_heads = num_kv_heads;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.head_dim = head_dim;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.len_cap = len_cap;
  a.num_blocks = num_blocks;
  a.split = p.split;
  a.part_steps = p.part_steps;
  a.num_workers = p.num_workers;
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_stride = new_stride;
  a.fold_in_merge = p.path == Path::kMfma ? 1 : 0;
  if (p.split) {
    if (p.ws_bytes > sized.ws_bytes) return PA_EINVAL;  // cannot happen: len_cap <= max
    if (!workspace || workspace_bytes < p.ws_bytes || !aligned16(workspace)) return PA_EINVAL;
    char* base = static_cast<char*>(workspace);
    a.ws_part = reinterpret_cast<float*>(base);
    a.ws_pre = reinterpret_cast<int32_t*>(base + p.pre_off);
    a.ws_ppre = reinterpret_cast<int32_t*>(base + p.ppre_off);
  }

  if (validate_enabled()) {
    std::vector<int32_t> lens, tab;
    if (!copy_to_host(lens, context_lens, (size_t)num_seqs, s)) return PA_EHIP;
    if (!copy_to_host(tab, block_tables, (size_t)num_seqs * max_blocks_per_seq, s))
      return PA_EHIP;
    for (int b = 0; b < num_seqs; ++b) {
      if (lens[b] < 0 || lens[b] > len_cap) return PA_EVALIDATE;
      const int nb = (lens[b] + block_size - 1) / block_size;
      for (int j = 0; j < nb; ++j) {
        const int32_t e = tab[(size_t)b * max_blocks_per_seq + j];
        if (e < 0 || e >= num_blocks) return PA_EVALIDATE;
      }
    }
    if (write) {
      // every new token's slot is its sequence's alone: no other sequence
      // writes it or reads it as one of its positions in this call
      std::unordered_set<int64_t> written;
      for (int b = 0; b < num_seqs; ++b) {
        if (lens[b] == 0) continue;
        const int pos = lens[b] - 1;
        const int64_t slot =
            (int64_t)tab[(size_t)b * max_blocks_per_seq + pos / block_size] * block_size +
            pos % block_size;
        if (!written.insert(slot).second) return PA_EVALIDATE;
      }
      for (int b = 0; b < num_seqs; ++b)
        for (int u = 0; u + 1 < lens[b]; ++u) {
          const int64_t slot =
              (int64_t)tab[(size_t)b * max_blocks_per_seq + u / block_size] * block_size +
              u % block_size;
          if (written.count(slot)) return PA_EVALIDATE;
        }
    }
  }

  hipError_t e = hipSuccess;
  if (write && p.path != Path::kGeneric && !p.split) {
    // an unsplit decode has no merge to fold the new token in: store the
    // tokens first and decode the pools plainly
    e = launch_store_new_tokens(a, dtype, s);
    if (e != hipSuccess) return PA_EHIP;
    a.k_new = a.v_new = nullptr;
  }
  switch (p.path) {
    case Path::kMfma: e = launch_decode_mfma(a, dtype, s); break;
    case Path::kValu: e = launch_decode_valu(a, dtype, s); break;
    case Path::kGeneric: e = launch_decode_generic(a, dtype, s); break;
  }
  if (e != hipSuccess) return PA_EHIP;
  if (p.split) e = launch_decode_merge(a, dtype, p.items_per_seq, s);
  return hip_status(e);
}

}  // namespace pa

extern "C" {

const char* pa_strerror(pa_status s) {
  switch (s) {
    case PA_OK: return "success";
    case PA_EINVAL: return "invalid argument";
    case PA_ENOTSUP: return "unsupported dtype / head_dim / block_size";
    case PA_ENOMEM: return "not enough free KV blocks";
    case PA_EHIP: return "HIP runtime or launch failure";
    case PA_EVALIDATE: return "device index data failed validation";
    case PA_ENOENT: return "unknown or duplicate sequence id";
    case PA_ESCRATCH: return "the call needs more scratch than pa_decode_noalloc's static array";
  }
  return "unknown status";
}

int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                 int32_t partition_size, pa_dtype dtype) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len <= 0) return -1;
  const Plan p = make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                           max_context_len, partition_size, dtype);
  if (!p.split) return -1;
  return p.part_steps * p.step;
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                 int32_t partition_size, pa_dtype dtype) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_context_len <= 0)
    return 0;
  return make_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len,
                   partition_size, dtype)
      .ws_bytes;
}

pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens, float scale,
                    int32_t block_size, int32_t num_kv_heads, int32_t num_seqs,
                    int32_t num_q_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                    int32_t max_context_len, int64_t num_blocks, pa_dtype dtype,
                    int32_t partition_size, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return decode_impl(out, q, nullptr, nullptr, 0, k_cache, v_cache, block_tables, context_lens,
                     scale, block_size, num_kv_heads, num_seqs, num_q_heads, head_dim,
                     max_blocks_per_seq, max_context_len, num_blocks, dtype, partition_size,
                     workspace, workspace_bytes, stream);
}

pa_status pa_decode_write(void* out, const void* q, const void* k_new, const void* v_new,
                          int64_t new_token_stride, void* k_cache, void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens, float scale,
                          int32_t block_size, int32_t num_kv_heads, int32_t num_seqs,
                          int32_t num_q_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                          int32_t max_context_len, int64_t num_blocks, pa_dtype dtype,
                          int32_t partition_size, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (!k_new || !v_new) return PA_EINVAL;
  return decode_impl(out, q, k_new, v_new, new_token_stride, k_cache, v_cache, block_tables,
                     context_lens, scale, block_size, num_kv_heads, num_seqs, num_q_heads,
                     head_dim, max_blocks_per_seq, max_context_len, num_blocks, dtype,
                     partition_size, workspace, workspace_bytes, stream);
}

size_t pa_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_groups,
                                        int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size,
                                        int32_t max_context_len, pa_dtype dtype) {
  if (num_seqs <= 0 || num_groups < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || max_context_len <= 0)
    return 0;
  return make_cascade_plan(num_seqs, num_groups, num_q_heads, num_kv_heads, head_dim, block_size,
                           max_context_len, dtype)
      .ws_bytes;
}

pa_status pa_decode_shared(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens, float scale,
                           int32_t block_size, int32_t num_kv_heads, int32_t num_seqs,
                           int32_t num_q_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                           int32_t max_context_len, int64_t num_blocks, pa_dtype dtype,
                           const int32_t* group_start, const int32_t* group_prefix_len,
                           int32_t num_groups, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (num_groups < 0 || num_seqs < 0 || num_kv_heads <= 0 || num_q_heads <= 0 ||
      block_size <= 0 || max_blocks_per_seq < 0 || max_context_len < 0)
    return PA_EINVAL;
  if (num_groups > 0 && (!group_start || !group_prefix_len)) return PA_EINVAL;
  const int len_cap = (int)std::min<int64_t>((int64_t)max_context_len,
                                             (int64_t)max_blocks_per_seq * block_size);
  const CascadePlan sized =
      make_cascade_plan(std::max(num_seqs, 1), num_groups, num_q_heads, num_kv_heads, head_dim,
                        block_size, max_context_len, dtype);
  const CascadePlan c = make_cascade_plan(std::max(num_seqs, 1), num_groups, num_q_heads,
                                          num_kv_heads, head_dim, block_size, len_cap, dtype);
  if (num_seqs == 0 || !c.ok || num_groups > num_seqs)  // no prefix pass: a plain decode
    return pa::decode_impl(out, q, nullptr, nullptr, 0, k_cache, v_cache, block_tables,
                           context_lens, scale, block_size, num_kv_heads, num_seqs, num_q_heads,
                           head_dim, max_blocks_per_seq, max_context_len, num_blocks, dtype, 0,
                           workspace, workspace_bytes, stream);
  // the checks of pa_decode, then the groups'
  if (!dtype_ok(dtype)) return PA_ENOTSUP;
  if (num_q_heads % num_kv_heads != 0 || !std::isfinite(scale) || num_blocks <= 0)
    return PA_EINVAL;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_EINVAL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_EINVAL;
  if (c.ws_bytes > sized.ws_bytes) return PA_EINVAL;  // cannot happen: len_cap <= max
  if (!workspace || workspace_bytes < c.ws_bytes || !aligned16(workspace)) return PA_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int group = num_q_heads / num_kv_heads;
  if (validate_enabled()) {
    std::vector<int32_t> lens, tab, gs, gp;
    if (!copy_to_host(lens, context_lens, (size_t)num_seqs, s) ||
        !copy_to_host(tab, block_tables, (size_t)num_seqs * max_blocks_per_seq, s) ||
        !copy_to_host(gs, group_start, (size_t)num_groups + 1, s) ||
        !copy_to_host(gp, group_prefix_len, (size_t)num_groups, s))
      return PA_EHIP;
    for (int b = 0; b < num_seqs; ++b) {
      if (lens[b] < 0 || lens[b] > len_cap) return PA_EVALIDATE;
      const int nb = (lens[b] + block_size - 1) / block_size;
      for (int j = 0; j < nb; ++j) {
        const int32_t e = tab[(size_t)b * max_blocks_per_seq + j];
        if (e < 0 || e >= num_blocks) return PA_EVALIDATE;
      }
    }
    if (gs[0] != 0 || gs[num_groups] != num_seqs) return PA_EVALIDATE;
    for (int g = 0; g < num_groups; ++g) {
      const int m = gs[g + 1] - gs[g];
      if (m < 1 || m * group > kPrefixRows) return PA_EVALIDATE;
      if (gp[g] < 0 || gp[g] % block_size != 0) return PA_EVALIDATE;
      const int nb = gp[g] / block_size;
      for (int b = gs[g]; b < gs[g + 1]; ++b) {
        if (lens[b] < gp[g]) return PA_EVALIDATE;
        for (int j = 0; j < nb; ++j)
          if (tab[(size_t)b * max_blocks_per_seq + j] != tab[(size_t)gs[g] * max_blocks_per_seq + j])
            return PA_EVALIDATE;
      }
    }
  }
  DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.scale_log2e = scale * 1.4426950408889634f;
  a.block_size = block_size;
  a.num_kv_heads = num_kv_heads;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.head_dim = head_dim;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.len_cap = len_cap;
  a.num_blocks = num_blocks;
  a.split = 1;
  a.part_steps = 0;
  a.num_workers = c.tail.num_workers;
  char* base = static_cast<char*>(workspace);
  a.ws_part = reinterpret_cast<float*>(base);
  a.ws_pre = reinterpret_cast<int32_t*>(base + c.tail.pre_off);
  a.ws_ppre = reinterpret_cast<int32_t*>(base + c.tail.ppre_off);
  a.group_start = group_start;
  a.group_prefix = group_prefix_len;
  a.num_groups = num_groups;
  a.ws_grp = reinterpret_cast<int32_t*>(base + c.grp_off);
  a.pws_part = reinterpret_cast<float*>(base + c.p_off);
  a.pws_pre = reinterpret_cast<int32_t*>(base + c.p_pre_off);
  a.p_num_workers = c.p_workers;
  // prefix pass: its own split and records
  DecodeArgs pa_ = a;
  pa_.num_workers = c.p_workers;
  pa_.ws_part = a.pws_part;
  pa_.ws_pre = a.pws_pre;
  pa_.ws_ppre = a.pws_pre;  // unused (no partitions)
  hipError_t e = launch_decode_prefix(pa_, dtype, s);
  if (e != hipSuccess) return PA_EHIP;
  e = c.tail.path == Path::kMfma ? launch_decode_mfma(a, dtype, s) : launch_decode_valu(a, dtype, s);
  if (e != hipSuccess) return PA_EHIP;
  return hip_status(launch_cascade_merge(a, dtype, c.tail.items_per_seq, s));
}

pa_status pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, const int32_t* context_lens,
                     const int32_t* query_start, float scale, int32_t block_size,
                     int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads,
                     int32_t head_dim, int32_t max_blocks_per_seq, int32_t max_query_len,
                     int32_t max_context_len, int64_t num_blocks, pa_dtype dtype, void* stream) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || max_blocks_per_seq < 0 || max_query_len < 0 || max_context_len < 0 ||
      num_blocks <= 0)
    return PA_EINVAL;
  if (!dtype_ok(dtype)) return PA_ENOTSUP;
  if (num_q_heads % num_kv_heads != 0 || !std::isfinite(scale)) return PA_EINVAL;
  if (!prefill_supported(dtype, head_dim, block_size)) return PA_ENOTSUP;
  if (num_seqs == 0 || max_query_len == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
    return PA_EINVAL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int len_cap = (int)std::min<int64_t>((int64_t)max_context_len,
                                             (int64_t)max_blocks_per_seq * block_size);
  if (validate_enabled()) {
    std::vector<int32_t> lens, tab, qs;
    if (!copy_to_host(lens, context_lens, (size_t)num_seqs, s)) return PA_EHIP;
    if (!copy_to_host(qs, query_start, (size_t)num_seqs + 1, s)) return PA_EHIP;
    if (!copy_to_host(tab, block_tables, (size_t)num_seqs * max_blocks_per_seq, s))
      return PA_EHIP;
    if (qs[0] != 0) return PA_EVALIDATE;
    for (int b = 0; b < num_seqs; ++b) {
      const int ql = qs[b + 1] - qs[b];
      if (ql < 0 || ql > max_query_len || lens[b] < ql || lens[b] > len_cap) return PA_EVALIDATE;
      const int nb = (lens[b] + block_size - 1) / block_size;
      for (int j = 0; j < nb; ++j) {
        const int32_t e = tab[(size_t)b * max_blocks_per_seq + j];
        if (e < 0 || e >= num_blocks) return PA_EVALIDATE;
      }
    }
  }
  PrefillArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.scale_log2e = scale * 1.4426950408889634f;
  a.block_size = block_size;
  a.num_kv_heads = num_kv_heads;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.head_dim = head_dim;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_query_len = max_query_len;
  a.len_cap = len_cap;
  a.num_blocks = num_blocks;
  return hip_status(launch_prefill(a, dtype, s));
}

pa_status pa_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                               const int64_t* slot_mapping, int32_t num_tokens,
                               int64_t k_token_stride, int64_t v_token_stride,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int64_t num_blocks, pa_dtype dtype, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PA_EINVAL;
  if (!dtype_ok(dtype)) return PA_ENOTSUP;
  if (!block_size_ok(block_size) || head_dim > 256) return PA_ENOTSUP;
  const int es = elem_bytes(dtype);
  if ((head_dim * es) % 16 != 0) return PA_ENOTSUP;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PA_EINVAL;
  if (k_token_stride < (int64_t)num_kv_heads * head_dim ||
      v_token_stride < (int64_t)num_kv_heads * head_dim)
    return PA_EINVAL;
  if ((k_token_stride * es) % 16 != 0 || (v_token_stride * es) % 16 != 0) return PA_EINVAL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_EINVAL;
  // the token rows often come straight from a caller's tensors: a host
  // pointer here would fault the kernel
  if (!device_accessible(k) || !device_accessible(v)) return PA_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (validate_enabled()) {
    std::vector<int64_t> slots;
    if (!copy_to_host(slots, slot_mapping, (size_t)num_tokens, s)) return PA_EHIP;
    std::unordered_set<int64_t> seen;
    for (int64_t x : slots) {
      if (x < 0) continue;
      if (x >= num_blocks * block_size || !seen.insert(x).second) return PA_EVALIDATE;
    }
  }
  return hip_status(launch_reshape_and_cache(k, v, k_cache, v_cache, slot_mapping, num_tokens,
                                             k_token_stride, v_token_stride, num_kv_heads,
                                             head_dim, block_size, num_blocks, es, s));
}

pa_status pa_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                         const int64_t* src_dst_pairs, int32_t num_pairs, int64_t src_num_blocks,
                         int64_t dst_num_blocks, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, pa_dtype dtype, void* stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      src_num_blocks <= 0 || dst_num_blocks <= 0)
    return PA_EINVAL;
  if (!dtype_ok(dtype)) return PA_ENOTSUP;
  const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * elem_bytes(dtype);
  if (block_bytes % 16 != 0) return PA_ENOTSUP;
  if (num_pairs == 0) return PA_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !src_dst_pairs) return PA_EINVAL;
  if (!aligned16(src_k) || !aligned16(src_v) || !aligned16(dst_k) || !aligned16(dst_v))
    return PA_EINVAL;
  // every pointer the kernel reads or writes must be mapped for the device
  if (!device_accessible(src_k) || !device_accessible(src_v) || !device_accessible(dst_k) ||
      !device_accessible(dst_v) || !device_accessible(src_dst_pairs))
    return PA_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (validate_enabled()) {
    std::vector<int64_t> pr;
    if (!copy_to_host(pr, src_dst_pairs, (size_t)num_pairs * 2, s)) return PA_EHIP;
    std::unordered_set<int64_t> dsts;
    for (int i = 0; i < num_pairs; ++i) {
      const int64_t a = pr[2 * i], b = pr[2 * i + 1];
      if (a < 0 || b < 0 || a >= src_num_blocks || b >= dst_num_blocks) return PA_EVALIDATE;
      if (!dsts.insert(b).second) return PA_EVALIDATE;
    }
  }
  return hip_status(launch_swap_blocks(src_k, src_v, dst_k, dst_v, src_dst_pairs, num_pairs,
                                       block_bytes, src_num_blocks, dst_num_blocks, s));
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* src_dst_pairs,
                         int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int64_t num_blocks, pa_dtype dtype, void* stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PA_EINVAL;
  if (!dtype_ok(dtype)) return PA_ENOTSUP;
  const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * elem_bytes(dtype);
  if (block_bytes % 16 != 0) return PA_ENOTSUP;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !src_dst_pairs) return PA_EINVAL;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PA_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (validate_enabled()) {
    std::vector<int64_t> pr;
    if (!copy_to_host(pr, src_dst_pairs, (size_t)num_pairs * 2, s)) return PA_EHIP;
    std::unordered_set<int64_t> dsts, srcs;
    for (int i = 0; i < num_pairs; ++i) {
      const int64_t a = pr[2 * i], b = pr[2 * i + 1];
      if (a < 0 || b < 0 || a >= num_blocks || b >= num_blocks) return PA_EVALIDATE;
      if (!dsts.insert(b).second) return PA_EVALIDATE;
      srcs.insert(a);
    }
    for (int64_t d : dsts)
      if (srcs.count(d)) return PA_EVALIDATE;
  }
  return hip_status(
      launch_copy_blocks(k_cache, v_cache, src_dst_pairs, num_pairs, block_bytes, num_blocks, s));
}

}  // extern "C"
