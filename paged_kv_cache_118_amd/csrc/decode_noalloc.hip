// pa_decode_noalloc: pa_decode with its split workspace in a static device
// array of this library instead of a caller-supplied buffer, for callers that
// cannot allocate device memory (code under graph capture, tight serving
// loops, harnesses that forbid allocation).  Nothing here allocates: the
// array is part of the code object, loaded once per device with the library.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pa.h"
#include "pa_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;  // the largest workspace served
constexpr int kMaxDevices = 64;

// The split's partial records and prefix sums.  In host code this name only
// stands for the symbol: its device address comes from hipGetSymbolAddress,
// once per device (each device holds its own copy of the array).
__device__ __align__(256) char scratch[kScratchBytes];

struct DeviceScratch {
  std::once_flag once;
  hipError_t err = hipSuccess;
  void* ptr = nullptr;
};
DeviceScratch g_scratch[kMaxDevices];

// The array's address on device `dev` (looked up with that device current,
// then the caller's device restored), or null on a HIP error.
void* scratch_on(int dev) {
  DeviceScratch& d = g_scratch[dev];
  std::call_once(d.once, [&] {
    int cur = -1;
    d.err = hipGetDevice(&cur);
    if (d.err != hipSuccess) return;
    if (cur != dev && (d.err = hipSetDevice(dev)) != hipSuccess) return;
    void* p = nullptr;
    d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (d.err == hipSuccess) d.ptr = p;
    if (cur != dev) {
      const hipError_t e = hipSetDevice(cur);
      if (d.err == hipSuccess) d.err = e;
    }
  });
  return d.err == hipSuccess ? d.ptr : nullptr;
}

}  // namespace

extern "C" {

size_t pa_decode_noalloc_scratch_bytes(void) { return kScratchBytes; }

pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            float scale, int32_t block_size, int32_t num_kv_heads,
                            int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                            int32_t max_blocks_per_seq, int32_t max_context_len,
                            int64_t num_blocks, pa_dtype dtype, int32_t partition_size,
                            void* stream) {
  const size_t need = pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                block_size, max_context_len, partition_size,
                                                dtype);
  if (need > kScratchBytes) return PA_ESCRATCH;
  if (need == 0)  // nothing splits: no scratch (pa_decode checks the rest)
    return pa::decode_impl(out, q, nullptr, nullptr, 0, k_cache, v_cache, block_tables,
                           context_lens, scale, block_size, num_kv_heads, num_seqs, num_q_heads,
                           head_dim, max_blocks_per_seq, max_context_len, num_blocks, dtype,
                           partition_size, nullptr, 0, stream);
  int dev = -1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if ((s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess) return PA_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return PA_EHIP;
  void* ws = scratch_on(dev);
  if (!ws) return PA_EHIP;
  return pa::decode_impl(out, q, nullptr, nullptr, 0, k_cache, v_cache, block_tables,
                         context_lens, scale, block_size, num_kv_heads, num_seqs, num_q_heads,
                         head_dim, max_blocks_per_seq, max_context_len, num_blocks, dtype,
                         partition_size, ws, kScratchBytes, stream);
}

}  // extern "C"
