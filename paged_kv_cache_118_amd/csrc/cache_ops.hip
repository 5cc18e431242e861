// KV-cache write (reshape_and_cache) and copy-on-write block copy for gfx950.
//
// Both are pure bit moves.  The write puts token t's K/V rows into slot
// slot_mapping[t] = block * BS + offset (flat slot numbering of the kernel
// pseudocode on vkads.cloudxian.cn "vLLM PagedAttention源码：KV Cache"); the
// copy duplicates whole blocks before a write into a shared tail block
// (wq-win.github.io "079 | vLLM 与 PagedAttention", section 二, part
// "共享与写时复制").
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kThreads = 256;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Stores that go around the L2's normal allocation: every written byte is
// new to the pool and the kernel never reads it back.
__device__ inline void store16_nt(char* dst, const char* lds_src) {
  const uint4 x = *reinterpret_cast<const uint4*>(lds_src);
  __builtin_nontemporal_store(u32x4_t{x.x, x.y, x.z, x.w}, reinterpret_cast<u32x4_t*>(dst));
}

// Large writes (prompt chunks): one workgroup = about TT consecutive tokens
// of one kv head, 8*TT threads.  Workgroups go through the kv heads fastest
// and through the token blocks from the last one back: neighbouring
// workgroups read neighbouring pieces of the same token rows and write
// neighbouring parts of the same pool blocks, and the batch's last tokens --
// in a mixed batch the scattered decode tokens, whose one-token V slabs are
// written element by element and take longest -- start first instead of
// forming the kernel's tail.  (On the OPT-66B-shaped chunk write, 64 tokens
// per workgroup in this order took 55-56 us against 65-68 us for 32 tokens
// in token-block-major order.)
//
// Boundaries.  Workgroup boundary i sits at token i*TT, moved forward (at most
// 7 tokens) past tokens whose slot continues the previous token's slot inside
// one 8-slot run.  With a block size that is a multiple of 8, slots 8k .. 8k+7
// of a block are one 128-byte line of each K piece run and one V slab, so a
// run of consecutive slots is never split between two workgroups (which, on
// different XCDs, would each write part of the same lines).  Any placement
// would be correct; this one only saves partial-line writes.  So that no
// load waits for the boundaries, a workgroup loads its whole window -- the
// TT + 7 tokens from i*TT, and the slot before it -- at once and finds both
// boundaries in LDS; rows past its end are read twice (the next workgroup
// owns them), at most 7 of TT + 7.
//
// The K and V rows are staged in LDS by 16-byte loads running along each row
// (a wavefront reads whole cache lines), then:
//  K: the pool stores 16-byte pieces [D/X][BS][X]; piece c of a token row is
//     one 16-byte store, threads taking tokens fastest, so consecutive slots
//     of one block fill one contiguous run per piece.
//  V: the pool stores 8-token slabs [D][VS].  Where the call writes all eight
//     slots of a slab (consecutive tokens at slots 8k .. 8k+7, the common case
//     for prompt chunks), each slab row -- the 8 tokens' element d -- is
//     gathered from LDS and written as whole 16-byte pieces; the tokens of
//     partly written slabs store their elements one by one, lanes taking
//     tokens fastest.
// The 16-byte stores are non-temporal: every byte is new to the pool and
// the kernel never reads it back.
template <int ES, int TT>
__global__ __launch_bounds__(8 * TT) void reshape_and_cache_kernel(
    const char* __restrict__ k, const char* __restrict__ v, char* __restrict__ k_cache,
    char* __restrict__ v_cache, const int64_t* __restrict__ slots, int32_t num_tokens,
    int64_t k_stride, int64_t v_stride, int32_t hkv, int32_t D, int32_t bs, int64_t num_blocks) {
  using E = typename std::conditional<ES == 4, uint32_t, uint16_t>::type;
  constexpr int NT = 8 * TT;
  constexpr int TW = TT + 7;  // window: the tokens a workgroup may own
  static_assert(TW < NT && (NT & (NT - 1)) == 0, "a thread per window token");
  extern __shared__ __align__(16) char smem[];
  const int row_bytes = D * ES;            // a multiple of 16
  const int pitch = row_bytes + 16;        // LDS row pitch (16-byte aligned, skewed banks)
  char* sk = smem;
  char* sv = smem + TW * pitch;
  int64_t* swin = reinterpret_cast<int64_t*>(smem + 2 * TW * pitch);  // slots w0-1 .. w0+TW-1
  int* slead = reinterpret_cast<int*>(swin + TW + 1);  // token leads a fully written slab
  int* scov = slead + TW;                              // token lies in such a slab
  __shared__ int s_leaders[TW / 8 + 1];
  __shared__ int s_nlead, s_t0, s_t1;
  const int h = blockIdx.x % hkv;
  const int w0 = ((int)gridDim.x / hkv - 1 - (int)blockIdx.x / hkv) * TT;
  const int wn = min(TW, num_tokens - w0);  // window tokens present
  const int64_t max_slot = num_blocks * (int64_t)bs;
  const int vs = v_slab(bs);
  const int chunks = row_bytes / 16;

  if (threadIdx.x <= TW) {
    const int t = w0 - 1 + (int)threadIdx.x;
    swin[threadIdx.x] = (t >= 0 && t < num_tokens) ? slots[t] : -1;
  }
  for (int i = threadIdx.x; i < wn * chunks; i += NT) {  // lanes along a row
    const int tt = i / chunks, c = i - tt * chunks;
    const int64_t t = w0 + tt;
    const uint4 kv = *reinterpret_cast<const uint4*>(k + (t * k_stride + (int64_t)h * D) * ES +
                                                      c * 16);
    const uint4 vv = *reinterpret_cast<const uint4*>(v + (t * v_stride + (int64_t)h * D) * ES +
                                                      c * 16);
    *reinterpret_cast<uint4*>(sk + tt * pitch + c * 16) = kv;
    *reinterpret_cast<uint4*>(sv + tt * pitch + c * 16) = vv;
  }
  __syncthreads();
  if (threadIdx.x < 64) {  // both boundaries: lanes 0-6 after w0, 8-14 after w0 + TT
    const int lane = threadIdx.x;
    const int j = lane & 7;
    const int base = (lane >> 3) == 1 ? min(TT, num_tokens - w0) : 0;  // relative to w0
    bool cont = false;
    if (lane < 16 && j < 7 && w0 + base + j > 0 && base + j < wn) {
      const int64_t cur = swin[base + j + 1];
      cont = cur > 0 && cur == swin[base + j] + 1 && (cur & 7) != 0;
    }
    const uint64_t m = __ballot(cont);
    if (lane == 0) {
      s_t0 = __builtin_ctzll(~(m & 0x7f));
      s_t1 = min(TT, num_tokens - w0) + __builtin_ctzll(~((m >> 8) & 0x7f));
      s_nlead = 0;
    }
  }
  __syncthreads();
  const int r0 = s_t0;              // first owned window row
  const int nt = s_t1 - r0;         // owned tokens
  const int64_t* sslot = swin + 1 + r0;
  const char* kr = sk + r0 * pitch;
  const char* vr = sv + r0 * pitch;
  if (threadIdx.x < nt) {
    const int tt = threadIdx.x;
    const int64_t s0 = sslot[tt];
    bool lead = vs == 8 && s0 >= 0 && s0 + 7 < max_slot && (s0 & 7) == 0 && tt + 8 <= nt;
    for (int j = 1; lead && j < 8; ++j) lead = sslot[tt + j] == s0 + j;
    slead[tt] = lead;
    if (lead) s_leaders[atomicAdd(&s_nlead, 1)] = tt;
  }
  __syncthreads();
  if (threadIdx.x < nt) {
    const int tt = threadIdx.x;
    int cov = 0;
    for (int j = 0; j < 8 && j <= tt; ++j) cov |= slead[tt - j] && sslot[tt] == sslot[tt - j] + j;
    scov[tt] = cov;
  }

  // K pieces: tokens fastest.
  for (int i = threadIdx.x; i < nt * chunks; i += NT) {
    const int c = i / nt, tt = i - c * nt;
    const int64_t slot = sslot[tt];
    if (slot >= 0 && slot < max_slot) {
      const int64_t blk = slot / bs;
      const int off = (int)(slot - blk * bs);
      store16_nt(k_cache + (((blk * hkv + h) * chunks + c) * bs + off) * 16, kr + tt * pitch + c * 16);
    }
  }
  __syncthreads();

  // V, fully written slabs: one 16-byte piece (8 tokens x 16 / (8 ES) dims)
  // per thread, dims fastest so a wavefront writes one contiguous run.
  constexpr int PPR = 8 * ES / 16;  // 16-byte pieces per slab row
  const int nl = s_nlead;
  for (int i = threadIdx.x; i < nl * D * PPR; i += NT) {
    const int li = i / (D * PPR), r = i - li * (D * PPR);
    const int d = r / PPR, half = r - d * PPR;  // pieces of a row: tokens 0-3 / 4-7 for fp32
    const int tt = s_leaders[li];
    const int64_t slot = sslot[tt];
    const int64_t blk = slot / bs;
    const int off = (int)(slot - blk * bs);
    __align__(16) E e[16 / ES];
#pragma unroll
    for (int u = 0; u < 16 / ES; ++u)
      e[u] = *reinterpret_cast<const E*>(vr + (tt + half * (16 / ES) + u) * pitch + d * ES);
    store16_nt(v_cache + ((((blk * hkv + h) * (bs / 8) + off / 8) * D + d) * 8) * ES + half * 16,
               reinterpret_cast<const char*>(e));
  }

  // V, tokens of partly written slabs: element by element, lanes taking
  // tokens (groups of TL >= nt lanes, a power of two), the NT / TL groups
  // taking every (NT / TL)-th element.
  const int lg = nt <= 1 ? 0 : 32 - __builtin_clz(nt - 1);  // log2 TL
  const int tt = threadIdx.x & ((1 << lg) - 1);
  if (tt >= nt || scov[tt]) return;
  const int64_t slot = sslot[tt];
  if (slot < 0 || slot >= max_slot) return;
  const int64_t blk = slot / bs;
  const int off = (int)(slot - blk * bs);
  E* vdst = reinterpret_cast<E*>(v_cache) +
            ((blk * hkv + h) * (bs / vs) + off / vs) * (int64_t)D * vs + off % vs;
  const E* src = reinterpret_cast<const E*>(vr + tt * pitch);
  for (int d = threadIdx.x >> lg; d < D; d += NT >> lg) vdst[(int64_t)d * vs] = src[d];
}

// Decode-sized writes (a token or a few per sequence, scattered slots, no
// slab ever filled whole): 8 tokens of one kv head per workgroup, K pieces
// straight from the token rows to the pool (tokens fastest), V through LDS so
// that lanes with consecutive slots write consecutive slab elements; one
// barrier instead of the staged kernel's three.  Every store is non-temporal:
// a token touches 16-byte pieces of many lines it does not fill, and plain
// stores cost the OPT-13B-shaped decode step about 9 us more.
template <int ES>
__global__ __launch_bounds__(64) void reshape_and_cache_small_kernel(
    const char* __restrict__ k, const char* __restrict__ v, char* __restrict__ k_cache,
    char* __restrict__ v_cache, const int64_t* __restrict__ slots, int32_t num_tokens,
    int64_t k_stride, int64_t v_stride, int32_t hkv, int32_t D, int32_t bs, int64_t num_blocks) {
  using E = typename std::conditional<ES == 4, uint32_t, uint16_t>::type;
  constexpr int TT = 8, NT = 64;
  extern __shared__ __align__(16) char smem[];
  const int row_bytes = D * ES;
  const int lds_stride = row_bytes + 4;  // pad: consecutive tokens hit different banks
  const int h = blockIdx.y;
  const int t0 = blockIdx.x * TT;
  const int nt = min(TT, num_tokens - t0);
  const int64_t max_slot = num_blocks * (int64_t)bs;
  const int vs = v_slab(bs);
  const int chunks = row_bytes / 16;
  for (int i = threadIdx.x; i < nt * chunks; i += NT) {
    const int c = i / nt, tt = i - c * nt;
    const int64_t t = t0 + tt;
    const int64_t slot = slots[t];
    const uint4 kv = *reinterpret_cast<const uint4*>(k + (t * k_stride + (int64_t)h * D) * ES +
                                                      c * 16);
    const uint4 vv = *reinterpret_cast<const uint4*>(v + (t * v_stride + (int64_t)h * D) * ES +
                                                      c * 16);
    uint32_t* dst = reinterpret_cast<uint32_t*>(smem + tt * lds_stride + c * 16);
    dst[0] = vv.x;
    dst[1] = vv.y;
    dst[2] = vv.z;
    dst[3] = vv.w;
    if (slot >= 0 && slot < max_slot) {
      const int64_t blk = slot / bs;
      const int off = (int)(slot - blk * bs);
      __builtin_nontemporal_store(u32x4_t{kv.x, kv.y, kv.z, kv.w},
          reinterpret_cast<u32x4_t*>(k_cache + (((blk * hkv + h) * chunks + c) * bs + off) * 16));
    }
  }
  __syncthreads();
  const int tt = threadIdx.x % TT;
  const int dgrp = threadIdx.x / TT;
  if (tt >= nt) return;
  const int64_t slot = slots[t0 + tt];
  if (slot < 0 || slot >= max_slot) return;
  const int64_t blk = slot / bs;
  const int off = (int)(slot - blk * bs);
  E* vdst = reinterpret_cast<E*>(v_cache) + ((blk * hkv + h) * (bs / vs) + off / vs) * (int64_t)D * vs +
            off % vs;
  const E* src = reinterpret_cast<const E*>(smem + tt * lds_stride);
  for (int d = dgrp; d < D; d += NT / TT) __builtin_nontemporal_store(src[d], vdst + (int64_t)d * vs);
}

// Whole-block copies: block b of either pool is one contiguous run of
// block_bytes bytes (all heads, all slots), so each pair is two memcpys.
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(char* __restrict__ k_cache,
                                                               char* __restrict__ v_cache,
                                                               const int64_t* __restrict__ pairs,
                                                               int64_t block_bytes,
                                                               int64_t num_blocks) {
  const int64_t src = pairs[2 * blockIdx.y], dst = pairs[2 * blockIdx.y + 1];
  if (src < 0 || dst < 0 || src >= num_blocks || dst >= num_blocks) return;
  const int64_t n16 = block_bytes / 16;
  const uint4* ks = reinterpret_cast<const uint4*>(k_cache + src * block_bytes);
  const uint4* vs = reinterpret_cast<const uint4*>(v_cache + src * block_bytes);
  uint4* kd = reinterpret_cast<uint4*>(k_cache + dst * block_bytes);
  uint4* vd = reinterpret_cast<uint4*>(v_cache + dst * block_bytes);
  for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * kThreads) {
    const uint4 a = ks[i];
    const uint4 b = vs[i];
    kd[i] = a;
    vd[i] = b;
  }
}

// Whole-block copies between two pools of the same layout (the swap of
// blocks between device memory and pinned host memory): block src of the
// source pools to block dst of the destination pools, K and V.  Ids outside
// either pool skip the pair.
__global__ __launch_bounds__(kThreads) void swap_blocks_kernel(
    const char* __restrict__ src_k, const char* __restrict__ src_v, char* __restrict__ dst_k,
    char* __restrict__ dst_v, const int64_t* __restrict__ pairs, int64_t block_bytes,
    int64_t src_blocks, int64_t dst_blocks) {
  const int64_t src = pairs[2 * blockIdx.y], dst = pairs[2 * blockIdx.y + 1];
  if (src < 0 || dst < 0 || src >= src_blocks || dst >= dst_blocks) return;
  const int64_t n16 = block_bytes / 16;
  const uint4* ks = reinterpret_cast<const uint4*>(src_k + src * block_bytes);
  const uint4* vs = reinterpret_cast<const uint4*>(src_v + src * block_bytes);
  uint4* kd = reinterpret_cast<uint4*>(dst_k + dst * block_bytes);
  uint4* vd = reinterpret_cast<uint4*>(dst_v + dst * block_bytes);
  for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * kThreads) {
    const uint4 a = ks[i];
    const uint4 b = vs[i];
    kd[i] = a;
    vd[i] = b;
  }
}

// LDS of one large-write workgroup: K and V rows, slots (and the one
// before), two flags per window token.
size_t rc_lds_bytes(int tt, int D, int es) {
  return (size_t)(tt + 7) * (2 * (D * es + 16) + 8 + 8) + 8;
}

// The largest LDS one workgroup may take on the current device.
size_t max_lds_per_workgroup() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
      v <= 0)
    return 64 * 1024;
  return (size_t)v;
}

template <int TT>
void launch_rc(const void* k, const void* v, void* k_cache, void* v_cache, const int64_t* slots,
               int32_t num_tokens, int64_t k_stride, int64_t v_stride, int32_t hkv, int32_t D,
               int32_t bs, int64_t num_blocks, int es, hipStream_t s) {
  dim3 grid((num_tokens + TT - 1) / TT * hkv);
  const size_t lds = rc_lds_bytes(TT, D, es);
  if (es == 4)
    hipLaunchKernelGGL((reshape_and_cache_kernel<4, TT>), grid, dim3(8 * TT), lds, s,
                       (const char*)k, (const char*)v, (char*)k_cache, (char*)v_cache, slots,
                       num_tokens, k_stride, v_stride, hkv, D, bs, num_blocks);
  else
    hipLaunchKernelGGL((reshape_and_cache_kernel<2, TT>), grid, dim3(8 * TT), lds, s,
                       (const char*)k, (const char*)v, (char*)k_cache, (char*)v_cache, slots,
                       num_tokens, k_stride, v_stride, hkv, D, bs, num_blocks);
}

}  // namespace

hipError_t launch_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                                    const int64_t* slots, int32_t num_tokens, int64_t k_stride,
                                    int64_t v_stride, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int64_t num_blocks, int elem_bytes,
                                    hipStream_t s) {
  if (num_tokens == 0) return hipSuccess;
  if (num_tokens >= 1024) {
    // 64 tokens per workgroup where the LDS allows (16-bit rows, and fp32 up
    // to D 128), else fewer
    const size_t cap = max_lds_per_workgroup();
    if (rc_lds_bytes(64, head_dim, elem_bytes) <= cap)
      launch_rc<64>(k, v, k_cache, v_cache, slots, num_tokens, k_stride, v_stride, num_kv_heads,
                    head_dim, block_size, num_blocks, elem_bytes, s);
    else if (rc_lds_bytes(32, head_dim, elem_bytes) <= cap)
      launch_rc<32>(k, v, k_cache, v_cache, slots, num_tokens, k_stride, v_stride, num_kv_heads,
                    head_dim, block_size, num_blocks, elem_bytes, s);
    else
      launch_rc<16>(k, v, k_cache, v_cache, slots, num_tokens, k_stride, v_stride, num_kv_heads,
                    head_dim, block_size, num_blocks, elem_bytes, s);
  } else {
    dim3 grid((num_tokens + 7) / 8, num_kv_heads);
    const size_t lds = (size_t)8 * (head_dim * elem_bytes + 4);
    if (elem_bytes == 4)
      hipLaunchKernelGGL(reshape_and_cache_small_kernel<4>, grid, dim3(64), lds, s,
                         (const char*)k, (const char*)v, (char*)k_cache, (char*)v_cache, slots,
                         num_tokens, k_stride, v_stride, num_kv_heads, head_dim, block_size,
                         num_blocks);
    else
      hipLaunchKernelGGL(reshape_and_cache_small_kernel<2>, grid, dim3(64), lds, s,
                         (const char*)k, (const char*)v, (char*)k_cache, (char*)v_cache, slots,
                         num_tokens, k_stride, v_stride, num_kv_heads, head_dim, block_size,
                         num_blocks);
  }
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs,
                              int32_t num_pairs, int64_t block_bytes, int64_t num_blocks,
                              hipStream_t s) {
  if (num_pairs == 0) return hipSuccess;
  const int64_t n16 = block_bytes / 16;
  int gx = (int)((n16 + kThreads * 4 - 1) / (kThreads * 4));
  if (gx < 1) gx = 1;
  dim3 grid(gx, num_pairs);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kThreads), 0, s, (char*)k_cache,
                     (char*)v_cache, pairs, block_bytes, num_blocks);
  return hipGetLastError();
}

hipError_t launch_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                              const int64_t* pairs, int32_t num_pairs, int64_t block_bytes,
                              int64_t src_blocks, int64_t dst_blocks, hipStream_t s) {
  if (num_pairs == 0) return hipSuccess;
  const int64_t n16 = block_bytes / 16;
  int gx = (int)((n16 + kThreads * 4 - 1) / (kThreads * 4));
  if (gx < 1) gx = 1;
  dim3 grid(gx, num_pairs);
  hipLaunchKernelGGL(swap_blocks_kernel, grid, dim3(kThreads), 0, s, (const char*)src_k,
                     (const char*)src_v, (char*)dst_k, (char*)dst_v, pairs, block_bytes,
                     src_blocks, dst_blocks);
  return hipGetLastError();
}

}  // namespace pa
