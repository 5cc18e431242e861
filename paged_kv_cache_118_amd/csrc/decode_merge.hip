// Merge of items that several workers split between them (decode_split.h).
//
// Each worker leaves, per q row of the item, fp32 (m_w, l_w, o_w): its running
// max (base-2 domain), the sum of exp2(s - m_w) and the unnormalised output.
// Because every block shares one softmax denominator (wq-win.github.io "079 |
// vLLM 与 PagedAttention", section 二, the Z / o equations), the exact result is
// recovered by rescaling to the global max M:
//   out = sum_w 2^(m_w - M) o_w  /  sum_w 2^(m_w - M) l_w.
// This kernel also writes the zero rows of empty sequences.
#include <math.h>

#include "decode_split.h"
#include "pa_internal.h"

namespace pa {

namespace {


template <typename TT>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float x) {
  if constexpr (TT::bytes == 4)
    reinterpret_cast<float*>(out)[idx] = x;
  else
    reinterpret_cast<uint16_t*>(out)[idx] = to_bits(TT{}, x);
}

// One workgroup per item, one thread per output (q row r, dim d); rows x
// head_dim <= 2048, so a thread takes at most two outputs.  The item's length
// and descriptor (first worker F, number of workers cnt -- written by worker
// F) are read together: an empty item gets zero rows, an item one worker
// covered is already done.  Otherwise each thread loads (m, l, o) of up to
// kBatch partials back to back and folds them in with an online rescale, so a
// merge costs one memory round trip per kBatch partials.
constexpr int kBatch = 16;

__device__ __forceinline__ void merge_output(const DecodeArgs& a, int64_t slot0, int cnt, int R,
                                             int r, int d, float& out) {
  const int D = a.head_dim;
  float M = -INFINITY, Lt = 0.f, acc = 0.f;
  for (int w0 = 0; w0 < cnt; w0 += kBatch) {
    float m[kBatch], l[kBatch], o[kBatch];
#pragma unroll
    for (int w = 0; w < kBatch; ++w) {
      const bool ok = w0 + w < cnt;
      const int64_t row = (slot0 + w0 + (ok ? w : 0)) * R + r;
      m[w] = ok ? a.ws_m[row] : -INFINITY;
      l[w] = ok ? a.ws_l[row] : 0.f;
      o[w] = ok ? a.ws_o[row * D + d] : 0.f;
    }
    float Mn = M;
#pragma unroll
    for (int w = 0; w < kBatch; ++w) Mn = fmaxf(Mn, m[w]);
    const float sc = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
    Lt *= sc;
    acc *= sc;
#pragma unroll
    for (int w = 0; w < kBatch; ++w) {
      const float f = m[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[w] - Mn);
      Lt += f * l[w];
      acc += f * o[w];
    }
    M = Mn;
  }
  out = acc / Lt;
}

template <typename TT>
__global__ __launch_bounds__(1024) void decode_merge_kernel(DecodeArgs a, int H,
                                                           int rows_per_item) {
  const int D = a.head_dim;
  const int t = threadIdx.x;
  const int item = blockIdx.x;
  const int b = item / H, h = item - b * H;
  const int L = clamp_len(a.context_lens[b], a.len_cap);
  const int2 desc = a.ws_desc[item];
  const int64_t orow0 = ((int64_t)b * a.num_q_heads + (int64_t)h * rows_per_item) * D;
  const int R = rows_per_item, total = R * D;
  for (int i = t; i < total; i += blockDim.x) {
    float x = 0.f;
    if (L > 0) {
      if (desc.y <= 1) continue;  // one worker saw the whole item and wrote it
      const int r = i / D, d = i - r * D;
      merge_output(a, (int64_t)item + desc.x, desc.y, R, r, d, x);
    }
    store_out<TT>(a.out, orow0 + i, x);
  }
}

}  // namespace

hipError_t launch_decode_merge(const DecodeArgs& a, pa_dtype dt, int items_per_seq,
                              hipStream_t s) {
  if (a.num_seqs == 0 || !a.split) return hipSuccess;
  const int rpi = a.num_q_heads / items_per_seq;
  const int outputs = rpi * a.head_dim;
  const int threads = outputs >= 1024 ? 1024 : (outputs + 63) / 64 * 64;
  dim3 grid(a.num_seqs * items_per_seq);
  switch (dt) {
    case PA_F32:
      hipLaunchKernelGGL(decode_merge_kernel<F32>, grid, dim3(threads), 0, s, a, items_per_seq,
                         rpi);
      break;
    case PA_F16:
      hipLaunchKernelGGL(decode_merge_kernel<F16>, grid, dim3(threads), 0, s, a, items_per_seq,
                         rpi);
      break;
    case PA_BF16:
      hipLaunchKernelGGL(decode_merge_kernel<BF16>, grid, dim3(threads), 0, s, a, items_per_seq,
                         rpi);
      break;
  }
  return hipGetLastError();
}

}  // namespace pa
