// Merge of the partials of items that the decode kernels split (decode_split.h).
//
// Each worker's piece of a split item left fp32 (m, l, o) per q row
// of the item: its running max (base-2 domain), the sum of exp2(s - m) and the
// unnormalised output.  Because every block shares one softmax denominator
// (wq-win.github.io "079 | vLLM 与 PagedAttention", section 二, the Z / o
// equations), the exact row is recovered by rescaling to the global max M:
//   out = sum_i 2^(m_i - M) o_i  /  sum_i 2^(m_i - M) l_i.
// The pieces an item has follow from the split arithmetic alone (the step
// and partition prefixes the decode kernel exported, the worker count, the
// partition size), so nothing but the partials themselves has to be
// communicated.  This kernel also writes the zero rows of empty sequences.
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

// Partials folded per memory round trip: each thread loads (m, l, o) of up to
// kBatch pieces back to back, then folds them in with one rescale.
constexpr int kBatch = 16;

// slot_of(k) = slot of the item's k-th piece, k < K.
template <typename SlotOf>
__device__ __forceinline__ float merge_output(const DecodeArgs& a, SlotOf slot_of, int K, int R,
                                              int r, int d) {
  const int D = a.head_dim;
  const int od = ((d >> 4) * 4 + ((d & 15) >> 2)) * R * 4 + r * 4 + (d & 3);  // within a record
  const int RS = part_record(R, D);
  float M = -INFINITY, Lt = 0.f, acc = 0.f;
  for (int k0 = 0; k0 < K; k0 += kBatch) {
    float m[kBatch], l[kBatch], o[kBatch];
#pragma unroll
    for (int w = 0; w < kBatch; ++w) {
      const bool ok = k0 + w < K;
      const float* rec = a.ws_part + (int64_t)slot_of(ok ? k0 + w : k0) * RS;
      m[w] = ok ? rec[R * D + r] : -INFINITY;
      l[w] = ok ? rec[R * D + 16 + r] : 0.f;
      o[w] = ok ? rec[od] : 0.f;
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
  return acc / Lt;
}

// One workgroup per item (b, h), one thread per output (q row r, dim d).
template <typename TT>
__global__ __launch_bounds__(1024) void decode_merge_kernel(DecodeArgs a, int H, int R) {
  const int D = a.head_dim, B = a.num_seqs;
  const int item = blockIdx.x;
  const int b = item / H, h = item - b * H;
  const int* pre = a.ws_pre;
  const int n = (pre[b + 1] - pre[b]) / H;
  const int64_t orow0 = ((int64_t)b * a.num_q_heads + (int64_t)h * R) * D;
  const int total = R * D;
  if (n == 0) {  // empty sequence: zero rows
    for (int t = threadIdx.x; t < total; t += blockDim.x) store_out<TT>(a.out, orow0 + t, 0.f);
    return;
  }
  const Split sp = make_split(a.num_workers, pre[B], a.part_steps, H, B, pre, a.ws_ppre);
  const int64_t S = pre[b] + (int64_t)h * n, E = S + n;
  const int F = sp.worker_of(S), Lw = sp.worker_of(E - 1);
  if (F == Lw) return;  // one piece: the decode kernel wrote the row
  // one piece per worker F .. Lw, in slots item + F .. item + Lw
  const int base = item + F;
  for (int t = threadIdx.x; t < total; t += blockDim.x) {
    const int r = t / D, d = t - r * D;
    store_out<TT>(a.out, orow0 + t,
                  merge_output(a, [base](int k) { return base + k; }, Lw - F + 1, R, r, d));
  }
}

}  // namespace

hipError_t launch_decode_merge(const DecodeArgs& a, pa_dtype dt, int items_per_seq,
                               hipStream_t s) {
  if (a.num_seqs == 0 || !a.split) return hipSuccess;
  const int R = a.num_q_heads / items_per_seq;
  const int outputs = R * a.head_dim;
  const int threads = outputs >= 1024 ? 1024 : (outputs + 63) / 64 * 64;
  dim3 grid(a.num_seqs * items_per_seq);
  switch (dt) {
    case PA_F32:
      hipLaunchKernelGGL(decode_merge_kernel<F32>, grid, dim3(threads), 0, s, a, items_per_seq,
                         R);
      break;
    case PA_F16:
      hipLaunchKernelGGL(decode_merge_kernel<F16>, grid, dim3(threads), 0, s, a, items_per_seq,
                         R);
      break;
    case PA_BF16:
      hipLaunchKernelGGL(decode_merge_kernel<BF16>, grid, dim3(threads), 0, s, a, items_per_seq,
                         R);
      break;
  }
  return hipGetLastError();
}

}  // namespace pa
