// Paged decode attention for grouped-query heads on the gfx950 matrix cores.
//
// Same definition as decode_valu.hip (global softmax over all blocks, tail
// masked, stable online reduction: wq-win.github.io "079 | vLLM 与
// PagedAttention", section 二, the Z / o equations), for G = Hq / Hkv q heads
// sharing one kv head (the GQA storage the same page's section 二 mentions).
// The G q rows of one kv head form a real, if small, dense contraction, so
// each K and V element is read from HBM once per kv head and used G times.
//
// Work item = (partition, kv head, sequence); four wavefronts per workgroup,
// each streaming 32-token groups.  With lane = 16*kb + n (n = lane % 16,
// kb = lane / 16) and v_mfma_f32_16x16x32 (A: row n, k-slots of group kb;
// B: column n, same k-slots; C: column n, rows 4*kb .. 4*kb+3):
//   S^T = K Q^T  : A = K rows (tokens), B = Q^T (heads, zero past G), two
//                  16-token tiles x D/32 k-steps.  Tile j's row r holds
//                  token 8*(r/4) + 4*j + r%4, so lane (n, kb) ends up with
//                  the scores of head n for the 8 tokens 8*kb .. 8*kb+7.
//   O^T += V^T P^T : A = V^T (16 d rows, 8 tokens per k-group, read as one
//                  16-byte run of a [D][16] V slab), B = P^T, which is
//                  exactly the lane's 8 weights; C = O^T keeps head n in lane
//                  n for every d tile, so the online-softmax rescale of the
//                  accumulators needs no data exchange.
// Only the max / sum over the 4 k-groups of a head crosses lanes (xor 16, 32).
#include <math.h>

#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kGroup = 32;  // tokens per wave step

__device__ __forceinline__ uint4 ld16(const char* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ float4_t mfma(F16, const uint4& a, const uint4& b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ float4_t mfma(BF16, const uint4& a, const uint4& b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf168_t, a),
                                                 __builtin_bit_cast(bf168_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(F16, float lo, float hi) {
  return (uint32_t)to_bits(F16{}, lo) | ((uint32_t)to_bits(F16{}, hi) << 16);
}
__device__ __forceinline__ uint32_t pack2(BF16, float lo, float hi) {
  return (uint32_t)to_bits(BF16{}, lo) | ((uint32_t)to_bits(BF16{}, hi) << 16);
}

template <typename TT>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float x) {
  reinterpret_cast<uint16_t*>(out)[idx] = to_bits(TT{}, x);
}

struct TableWindow {
  int base;
  int entry;
  __device__ __forceinline__ void ensure(const int32_t* row, int nblk, int64_t num_blocks, int lb,
                                         int n, int lane) {
    if (lb < base || lb + n - base > 64) {
      base = lb;
      const int idx = lb + lane;
      const int e = idx < nblk ? row[idx] : 0;
      entry = (e < 0 || (int64_t)e >= num_blocks) ? 0 : e;
    }
  }
  __device__ __forceinline__ int get(int lb) const {
    return __builtin_amdgcn_readlane(entry, lb - base);
  }
};

template <typename TT, int D, int VS>
__global__ __launch_bounds__(kThreads) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int EB = 2;
  constexpr int KN = D / 32;  // uint4 per lane per K tile (= QK k-steps)
  constexpr int MT = D / 16;  // d tiles of O^T
  constexpr int OST = D + 4;  // LDS row pitch of the merge buffer (floats)

  __shared__ float s_m[kWaves][16], s_l[kWaves][16];
  __shared__ float s_o[kWaves][16][OST];

  const int p = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, kb = lane >> 4;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int bs = a.block_size;
  int L = a.context_lens[b];
  L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
  const int t0 = p * a.part;
  const int64_t head0 = (int64_t)b * a.num_q_heads + (int64_t)g * G;  // first q row
  if (t0 >= L) {
    if (p == 0)
      for (int i = threadIdx.x; i < G * D; i += kThreads) store_out<TT>(a.out, head0 * D + i, 0.f);
    return;
  }
  const int t1 = min(t0 + a.part, L);
  const int nblk = (L + bs - 1) / bs;
  const int32_t* trow = a.block_tables + (int64_t)b * a.max_blocks_per_seq;
  const int ngroups = (t1 - t0 + kGroup - 1) / kGroup;
  const int s_begin = ngroups * w / kWaves, s_end = ngroups * (w + 1) / kWaves;
  const int nb_grp = bs >= kGroup ? 1 : kGroup / bs;  // blocks touched by one group

  const char* kbase = reinterpret_cast<const char*>(a.k_cache);
  const char* vbase = reinterpret_cast<const char*>(a.v_cache);
  const int64_t hkv = a.num_kv_heads;

  // Q^T operand: head n, d = kb*D/4 + 8*s + e for k-step s.
  uint4 qv[KN];
  {
    const char* qp = reinterpret_cast<const char*>(a.q) + ((head0 + n) * D + kb * (D / 4)) * EB;
#pragma unroll
    for (int s = 0; s < KN; ++s) qv[s] = n < G ? ld16(qp + 16 * s) : make_uint4(0, 0, 0, 0);
  }

  TableWindow tw;
  tw.base = 0x7fffffff;
  tw.entry = 0;

  // K row of tile j for this lane, and the V token run of k-group kb.
  const int kt_off0 = (n >> 2) * 8 + (n & 3);  // token of tile 0 row n (tile 1: +4)
  auto issue = [&](int s, uint4 (&kr)[2][KN], uint4 (&vr)[MT]) {
    const int tok = t0 + s * kGroup;
    const int lb0 = tok / bs;
    tw.ensure(trow, nblk, a.num_blocks, lb0, nb_grp, lane);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int t = tok + kt_off0 + 4 * j;
      const int lb = t / bs;
      int64_t phys = tw.get(lb0);
      for (int q = 1; q < nb_grp; ++q)
        if (lb == lb0 + q) phys = tw.get(lb0 + q);
      const char* kp = kbase + (((phys * hkv + g) * bs + (t - lb * bs)) * D + kb * (D / 4)) * EB;
#pragma unroll
      for (int i = 0; i < KN; ++i) kr[j][i] = ld16(kp + 16 * i);
    }
    {
      const int t = tok + kb * 8;
      const int lb = t / bs;
      int64_t phys = tw.get(lb0);
      for (int q = 1; q < nb_grp; ++q)
        if (lb == lb0 + q) phys = tw.get(lb0 + q);
      const int off = t - lb * bs;
      const char* vp =
          vbase + ((((phys * hkv + g) * (bs / VS) + off / VS) * D + n) * VS + off % VS) * EB;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) vr[mt] = ld16(vp + (int64_t)mt * 16 * VS * EB);
    }
  };

  float m_run = -INFINITY, l_lane = 0.f;
  float4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = float4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int s, const uint4 (&kr)[2][KN], uint4 (&vr)[MT]) {
    const int tok = t0 + s * kGroup;
    const int nvalid = min(kGroup, t1 - tok);
    float4_t st[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      st[j] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < KN; ++i) st[j] = mfma(TT{}, kr[j][i], qv[i], st[j]);
    }
    float sc[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sc[e] = st[0][e] * a.scale_log2e;
      sc[4 + e] = st[1][e] * a.scale_log2e;
    }
    if (nvalid < kGroup) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (kb * 8 + e >= nvalid) sc[e] = -INFINITY;  // select: masked K may be NaN
    }
    float mx = sc[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sc[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float pw[8], psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pw[e] = __builtin_amdgcn_exp2f(sc[e] - m_new);
      psum += pw[e];
    }
    l_lane = l_lane * alpha + psum;
    m_run = m_new;
    const uint4 pb = make_uint4(pack2(TT{}, pw[0], pw[1]), pack2(TT{}, pw[2], pw[3]),
                                pack2(TT{}, pw[4], pw[5]), pack2(TT{}, pw[6], pw[7]));
    if (nvalid < kGroup) {  // zero V of masked tokens (their bits may be NaN)
      const int keep = min(max(nvalid - kb * 8, 0), 8);  // valid tokens of this k-group
      uint32_t m4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = (2 * i < keep) ? 0xffffu : 0u;
        const uint32_t hi = (2 * i + 1 < keep) ? 0xffff0000u : 0u;
        m4[i] = lo | hi;
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        vr[mt].x &= m4[0];
        vr[mt].y &= m4[1];
        vr[mt].z &= m4[2];
        vr[mt].w &= m4[3];
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc[mt] *= alpha;
      acc[mt] = mfma(TT{}, vr[mt], pb, acc[mt]);
    }
  };

  {
    uint4 ka[2][KN], va[MT], kb2[2][KN], vb2[MT];
    int s = s_begin;
    if (s < s_end) issue(s, ka, va);
    while (s < s_end) {
      if (s + 1 < s_end) issue(s + 1, kb2, vb2);
      compute(s, ka, va);
      ++s;
      if (s >= s_end) break;
      if (s + 1 < s_end) issue(s + 1, ka, va);
      compute(s, kb2, vb2);
      ++s;
    }
  }

  // per-head sum over the 4 k-groups, then merge the waves through LDS
  l_lane += __shfl_xor(l_lane, 16);
  l_lane += __shfl_xor(l_lane, 32);
  if (kb == 0) {
    s_m[w][n] = m_run;
    s_l[w][n] = l_lane;
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) s_o[w][n][mt * 16 + 4 * kb + e] = acc[mt][e];
  __syncthreads();

  const bool split = (L + a.part - 1) / a.part > 1;
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int hn = i / D, d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, s_m[ww][hn]);
    float o = 0.f, Lt = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = s_m[ww][hn] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s_m[ww][hn] - M);
      o += f * s_o[ww][hn][d];
      Lt += f * s_l[ww][hn];
    }
    if (!split) {
      store_out<TT>(a.out, (head0 + hn) * D + d, o / Lt);
    } else {
      const int64_t pi = (head0 + hn) * a.max_parts + p;
      a.ws_o[pi * D + d] = o;
      if (d == 0) {
        a.ws_m[pi] = M;
        a.ws_l[pi] = Lt;
      }
    }
  }
}

template <typename TT, int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.max_parts, a.num_kv_heads, a.num_seqs);
  if (a.block_size >= 16)
    hipLaunchKernelGGL((decode_mfma_kernel<TT, D, 16>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<TT, D, 8>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <typename TT>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
  switch (a.head_dim) {
    case 64: return launch_d<TT, 64>(a, s);
    case 128: return launch_d<TT, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool decode_mfma_supported(pa_dtype dt, int head_dim, int block_size, int group) {
  const bool dt_ok = dt == PA_F16 || dt == PA_BF16;
  const bool d_ok = head_dim == 64 || head_dim == 128;
  const bool bs_ok = block_size == 8 || block_size == 16 || (block_size % 32 == 0);
  return dt_ok && d_ok && bs_ok && group >= 2 && group <= 16;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, pa_dtype dt, hipStream_t s) {
  if (a.num_seqs == 0) return hipSuccess;
  if (dt == PA_F16) return launch_t<F16>(a, s);
  if (dt == PA_BF16) return launch_t<BF16>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace pa
