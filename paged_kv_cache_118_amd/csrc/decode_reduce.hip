// Merge of split-context partitions.
//
// A sequence longer than one partition is processed as P-token pieces, each
// leaving fp32 (m_p, l_p, o_p): its running max (base-2 domain), the sum of
// exp2(s - m_p) and the unnormalised output.  Because every block shares one
// softmax denominator (wq-win.github.io "079 | vLLM 与 PagedAttention",
// section 二, the Z / o equations), the exact result is recovered by
// rescaling to the global max M:
//   out = sum_p 2^(m_p - M) o_p  /  sum_p 2^(m_p - M) l_p.
#include <math.h>

#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kThreads = 128;
constexpr int kMaxLdsParts = 1024;

template <typename TT>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float x) {
  if constexpr (TT::bytes == 4)
    reinterpret_cast<float*>(out)[idx] = x;
  else
    reinterpret_cast<uint16_t*>(out)[idx] = to_bits(TT{}, x);
}

// One workgroup per (q head, sequence); threads over head_dim.
template <typename TT>
__global__ __launch_bounds__(kThreads) void decode_reduce_kernel(DecodeArgs a) {
  __shared__ float s_f[kMaxLdsParts];
  __shared__ float s_red[kThreads / 64];
  const int h = blockIdx.x, b = blockIdx.y;
  int L = a.context_lens[b];
  L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
  const int np = (L + a.part - 1) / a.part;
  if (np <= 1) return;  // written directly by the partition kernel
  const int64_t row = (int64_t)b * a.num_q_heads + h;
  const float* m = a.ws_m + row * a.max_parts;
  const float* l = a.ws_l + row * a.max_parts;
  const float* o = a.ws_o + row * a.max_parts * a.head_dim;

  // global max over partitions
  float M = -INFINITY;
  for (int i = threadIdx.x; i < np; i += kThreads) M = fmaxf(M, m[i]);
  for (int k = 1; k < 64; k <<= 1) M = fmaxf(M, __shfl_xor(M, k));
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = M;
  __syncthreads();
  M = s_red[0];
  for (int i = 1; i < kThreads / 64; ++i) M = fmaxf(M, s_red[i]);
  __syncthreads();

  // rescale factors (kept in LDS for the first kMaxLdsParts partitions)
  float lsum = 0.f;
  for (int i = threadIdx.x; i < np; i += kThreads) {
    const float f = __builtin_amdgcn_exp2f(m[i] - M);
    if (i < kMaxLdsParts) s_f[i] = f;
    lsum += f * l[i];
  }
  for (int k = 1; k < 64; k <<= 1) lsum += __shfl_xor(lsum, k);
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = lsum;
  __syncthreads();
  float Lt = 0.f;
  for (int i = 0; i < kThreads / 64; ++i) Lt += s_red[i];

  const int D = a.head_dim;
  for (int d = threadIdx.x; d < D; d += kThreads) {
    float acc = 0.f;
    for (int i = 0; i < np; ++i) {
      const float f = i < kMaxLdsParts ? s_f[i] : __builtin_amdgcn_exp2f(m[i] - M);
      acc += f * o[(int64_t)i * D + d];
    }
    store_out<TT>(a.out, row * D + d, acc / Lt);
  }
}

}  // namespace

hipError_t launch_decode_reduce(const DecodeArgs& a, pa_dtype dt, hipStream_t s) {
  if (a.num_seqs == 0 || a.max_parts <= 1) return hipSuccess;
  dim3 grid(a.num_q_heads, a.num_seqs);
  switch (dt) {
    case PA_F32:
      hipLaunchKernelGGL(decode_reduce_kernel<F32>, grid, dim3(kThreads), 0, s, a);
      break;
    case PA_F16:
      hipLaunchKernelGGL(decode_reduce_kernel<F16>, grid, dim3(kThreads), 0, s, a);
      break;
    case PA_BF16:
      hipLaunchKernelGGL(decode_reduce_kernel<BF16>, grid, dim3(kThreads), 0, s, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace pa
