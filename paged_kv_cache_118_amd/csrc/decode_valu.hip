// Paged single-query decode attention on the vector ALUs (gfx950).
//
// Computes, per (sequence, q head), the global-softmax attention of the Z / o
// equations in wq-win.github.io "079 | vLLM 与 PagedAttention", section 二,
// part "分块以后，注意力仍需对整个历史归一化": every valid position of every
// block shares one denominator, the unfilled tail of the last block is
// excluded, and the reduction is done in a numerically stable way (online
// max / sum, rescaling by exp(m_old - m_new)).  Positions are found through
// the block table: logical block u / BS, offset u % BS (gitcode.csdn.net
// "vLLM 推理引擎：PagedAttention 与 KVCache 管理", section 3).
//
// decode_valu_kernel -- the MHA path (one q head per kv head read).  Work item
// = (partition of P tokens, q head, sequence), one 256-thread workgroup.  Each
// of the 4 wavefronts streams a contiguous run of 16-token steps:
//   K  step = 16 token rows; lane (t = lane/4, c = lane%4) loads D/4 elements
//      of row t (64 B for fp16 D=128), dot2 with q, quad-reduce via DPP.
//   V  step = one 16-token slab [D][16] (two 8-token slabs when BS = 8);
//      lane owns D/64 full slab rows, so its accumulators are complete sums
//      and need no cross-lane reduction; the 16 weights are broadcast with
//      readlane into scalar registers.
// Loads for step i+1 are issued before step i is computed.  The four waves
// merge (m, l, acc) through LDS; a sequence longer than P writes fp32
// partials that decode_reduce.hip merges.
//
// decode_generic_kernel -- any head_dim <= 256 / block_size / dtype, one
// wavefront per (q head, sequence), one token at a time.  Used for shapes the
// fast kernels do not cover (e.g. head_dim 16, block_size 4).
#include <math.h>

#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStep = 16;  // tokens per wave step

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float bcast_lane(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}
__device__ __forceinline__ float xor_max(float x, int m) { return fmaxf(x, __shfl_xor(x, m)); }
__device__ __forceinline__ float wave_sum(float x) {
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
  return x;
}
__device__ __forceinline__ uint4 ld16(const char* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Storage-type helpers over the uint4 words a lane holds.
template <typename TT>
struct Words;
template <>
struct Words<F32> {
  static constexpr int per16 = 4;  // elements per 16 bytes
};
template <>
struct Words<F16> {
  static constexpr int per16 = 8;
};
template <>
struct Words<BF16> {
  static constexpr int per16 = 8;
};

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// dot of the lane's q slice with its K slice (NK uint4 words each)
template <int NK>
__device__ __forceinline__ float lane_dot(F32, const uint4 (&q)[NK], const uint4 (&k)[NK]) {
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    s0 = fmaf(__uint_as_float(q[i].x), __uint_as_float(k[i].x), s0);
    s1 = fmaf(__uint_as_float(q[i].y), __uint_as_float(k[i].y), s1);
    s0 = fmaf(__uint_as_float(q[i].z), __uint_as_float(k[i].z), s0);
    s1 = fmaf(__uint_as_float(q[i].w), __uint_as_float(k[i].w), s1);
  }
  return s0 + s1;
}
template <typename TT, int NK>
__device__ __forceinline__ float lane_dot(TT t, const uint4 (&q)[NK], const uint4 (&k)[NK]) {
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    s0 = dot2(t, q[i].x, k[i].x, s0);
    s1 = dot2(t, q[i].y, k[i].y, s1);
    s0 = dot2(t, q[i].z, k[i].z, s0);
    s1 = dot2(t, q[i].w, k[i].w, s1);
  }
  return s0 + s1;
}

// acc[r] += sum_tau p[tau] * v[r][tau] over the lane's V elements.
// Element e of the lane's data: piece j = e / (R*VS), row r = (e % (R*VS)) / VS,
// token tau = j*VS + e % VS.
template <typename TT, int R, int VS, int NK>
__device__ __forceinline__ void lane_pv(float (&acc)[R], const float (&p)[kStep],
                                        const uint4 (&v)[NK]) {
#pragma unroll
  for (int i = 0; i < NK; ++i)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x = word(v[i], w);
      if constexpr (TT::bytes == 4) {
        const int e = i * 4 + w;
        const int j = e / (R * VS), r = (e % (R * VS)) / VS, tau = j * VS + e % VS;
        acc[r] = fmaf(p[tau], __uint_as_float(x), acc[r]);
      } else {
        const int e = i * 8 + w * 2;
        const int j = e / (R * VS), r = (e % (R * VS)) / VS, tau = j * VS + e % VS;
        acc[r] = fmaf(p[tau], lo_to_float(TT{}, x), acc[r]);
        acc[r] = fmaf(p[tau + 1], hi_to_float(TT{}, x), acc[r]);
      }
    }
}

// Zero V elements of tokens >= nvalid (their bits may be NaN; 0 * NaN = NaN).
template <typename TT, int R, int VS, int NK>
__device__ __forceinline__ void mask_v(uint4 (&v)[NK], int nvalid) {
  constexpr int per16 = Words<TT>::per16;
  constexpr int eb = 16 / per16 * 8;  // bits per element
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    uint32_t w4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      constexpr int per_word = 32 / eb;
#pragma unroll
      for (int h = 0; h < per_word; ++h) {
        const int e = i * per16 + w * per_word + h;
        const int j = e / (R * VS), tau = j * VS + e % VS;
        if (tau >= nvalid) {
          const uint32_t m = eb == 32 ? 0xffffffffu : (0xffffu << (16 * h));
          w4[w] &= ~m;
        }
      }
    }
    v[i] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
  }
}

template <typename TT>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float x) {
  if constexpr (TT::bytes == 4)
    reinterpret_cast<float*>(out)[idx] = x;
  else
    reinterpret_cast<uint16_t*>(out)[idx] = to_bits(TT{}, x);
}

// Block-table window: lane i holds the physical id of logical block base + i
// (0 past the sequence's last block, and for ids outside the pool, so that a
// bad table never produces an out-of-range address).
struct TableWindow {
  int base;
  int entry;
  __device__ __forceinline__ void load(const int32_t* row, int nblk, int64_t num_blocks, int lb,
                                       int lane) {
    base = lb;
    const int idx = lb + lane;
    int e = idx < nblk ? row[idx] : 0;
    entry = (e < 0 || (int64_t)e >= num_blocks) ? 0 : e;
  }
  // physical id of logical blocks lb .. lb+n-1 must be in the window
  __device__ __forceinline__ void ensure(const int32_t* row, int nblk, int64_t num_blocks, int lb,
                                         int n, int lane) {
    if (lb < base || lb + n - base > 64) load(row, nblk, num_blocks, lb, lane);
  }
  __device__ __forceinline__ int get(int lb) const {
    return __builtin_amdgcn_readlane(entry, lb - base);
  }
};

template <typename TT, int D, int VS>
__global__ __launch_bounds__(kThreads) void decode_valu_kernel(DecodeArgs a) {
  constexpr int EB = TT::bytes;
  constexpr int LANE_BYTES = D * EB / 4;  // per lane per step, K and V alike
  constexpr int NK = LANE_BYTES / 16;
  constexpr int R = D / 64;  // slab rows owned by a lane
  constexpr int PIECES = kStep / VS;
  constexpr int PIECE_NK = NK / PIECES;
  static_assert(NK % PIECES == 0 && R >= 1, "unsupported shape");

  __shared__ float s_m[kWaves], s_l[kWaves];
  __shared__ float s_acc[kWaves][D];

  const int p = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int group = a.num_q_heads / a.num_kv_heads;
  const int g = h / group;
  const int bs = a.block_size;
  int L = a.context_lens[b];
  L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
  const int t0 = p * a.part;
  const int64_t orow = ((int64_t)b * a.num_q_heads + h) * D;
  if (t0 >= L) {
    if (p == 0)  // empty sequence: zero row
      for (int d = threadIdx.x; d < D; d += kThreads) store_out<TT>(a.out, orow + d, 0.f);
    return;
  }
  const int t1 = min(t0 + a.part, L);
  const int nblk = (L + bs - 1) / bs;
  const int32_t* trow = a.block_tables + (int64_t)b * a.max_blocks_per_seq;

  // this wave's steps
  const int nsteps = (t1 - t0 + kStep - 1) / kStep;
  const int s_begin = nsteps * w / kWaves, s_end = nsteps * (w + 1) / kWaves;

  const int tq = lane >> 2, c = lane & 3;
  const char* kbase = reinterpret_cast<const char*>(a.k_cache);
  const char* vbase = reinterpret_cast<const char*>(a.v_cache);

  // q slice of this lane: elements c*D/4 .. (c+1)*D/4
  uint4 qv[NK];
  {
    const char* qp = reinterpret_cast<const char*>(a.q) + (orow + c * (D / 4)) * EB;
#pragma unroll
    for (int i = 0; i < NK; ++i) qv[i] = ld16(qp + 16 * i);
  }

  TableWindow tw;
  tw.base = 0x7fffffff;
  tw.entry = 0;

  auto issue = [&](int s, uint4 (&kr)[NK], uint4 (&vr)[NK]) {
    const int tok = t0 + s * kStep;
    const int lb = tok / bs;
    if constexpr (VS == 16) {
      tw.ensure(trow, nblk, a.num_blocks, lb, 1, lane);
      const int64_t phys = tw.get(lb);
      const int off = tok - lb * bs;  // multiple of 16
      const char* kp =
          kbase + (((phys * a.num_kv_heads + g) * bs + off + tq) * D + c * (D / 4)) * EB;
#pragma unroll
      for (int i = 0; i < NK; ++i) kr[i] = ld16(kp + 16 * i);
      const char* vp =
          vbase +
          ((((phys * a.num_kv_heads + g) * (bs / 16) + off / 16) * D + lane * R) * 16) * EB;
#pragma unroll
      for (int i = 0; i < NK; ++i) vr[i] = ld16(vp + 16 * i);
    } else {  // BS == VS < 16: the step spans PIECES blocks
      tw.ensure(trow, nblk, a.num_blocks, lb, PIECES, lane);
      int64_t ph[PIECES];
#pragma unroll
      for (int j = 0; j < PIECES; ++j) ph[j] = tw.get(lb + j);
      int64_t mine = ph[0];
#pragma unroll
      for (int j = 1; j < PIECES; ++j)
        if (tq / VS == j) mine = ph[j];
      const char* kp =
          kbase + (((mine * a.num_kv_heads + g) * VS + tq % VS) * D + c * (D / 4)) * EB;
#pragma unroll
      for (int i = 0; i < NK; ++i) kr[i] = ld16(kp + 16 * i);
#pragma unroll
      for (int j = 0; j < PIECES; ++j) {
        const char* vp = vbase + (((ph[j] * a.num_kv_heads + g) * D + lane * R) * VS) * EB;
#pragma unroll
        for (int i = 0; i < PIECE_NK; ++i) vr[j * PIECE_NK + i] = ld16(vp + 16 * i);
      }
    }
  };

  float m_run = -INFINITY, l_lane = 0.f;
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;

  auto compute = [&](int s, const uint4 (&kr)[NK], uint4 (&vr)[NK]) {
    const int tok = t0 + s * kStep;
    const int nvalid = min(kStep, t1 - tok);
    float d = lane_dot(TT{}, qv, kr);
    d += dpp<0xB1>(d);  // quad_perm [1,0,3,2]
    d += dpp<0x4E>(d);  // quad_perm [2,3,0,1]
    float sc = d * a.scale_log2e;
    if (tq >= nvalid) sc = -INFINITY;  // select, never multiply: masked K may be NaN
    float mx = fmaxf(sc, dpp<0x124>(sc));  // row_ror:4
    mx = fmaxf(mx, dpp<0x128>(mx));        // row_ror:8
    mx = xor_max(mx, 16);
    mx = xor_max(mx, 32);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    const float pv = __builtin_amdgcn_exp2f(sc - m_new);
    l_lane = l_lane * alpha + (c == 0 ? pv : 0.f);
    m_run = m_new;
    float pt[kStep];
#pragma unroll
    for (int t = 0; t < kStep; ++t) pt[t] = bcast_lane(pv, 4 * t);
    if (nvalid < kStep) mask_v<TT, R, VS, NK>(vr, nvalid);
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] *= alpha;
    lane_pv<TT, R, VS, NK>(acc, pt, vr);
  };

  {
    uint4 ka[NK], va[NK], kb2[NK], vb2[NK];
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

  // merge the four waves
  const float l_w = wave_sum(l_lane);
  if (lane == 0) {
    s_m[w] = m_run;
    s_l[w] = l_w;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) s_acc[w][lane * R + r] = acc[r];
  __syncthreads();

  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) M = fmaxf(M, s_m[i]);
  float f[kWaves], Lt = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    f[i] = s_m[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s_m[i] - M);
    Lt += f[i] * s_l[i];
  }
  const bool split = (L + a.part - 1) / a.part > 1;
  for (int d = threadIdx.x; d < D; d += kThreads) {
    float o = 0.f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) o += f[i] * s_acc[i][d];
    if (!split) {
      store_out<TT>(a.out, orow + d, o / Lt);
    } else {
      const int64_t pi = ((int64_t)b * a.num_q_heads + h) * a.max_parts + p;
      a.ws_o[pi * D + d] = o;
      if (d == 0) {
        a.ws_m[pi] = M;
        a.ws_l[pi] = Lt;
      }
    }
  }
}

// ------------------------------------------------------------- generic --
template <typename TT>
__device__ __forceinline__ float load_elem(const void* base, int64_t i) {
  if constexpr (TT::bytes == 4) {
    return reinterpret_cast<const float*>(base)[i];
  } else {
    const uint32_t bits = reinterpret_cast<const uint16_t*>(base)[i];
    return lo_to_float(TT{}, bits);
  }
}

template <typename TT>
__global__ __launch_bounds__(64) void decode_generic_kernel(DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x;
  const int D = a.head_dim, bs = a.block_size, hkv = a.num_kv_heads;
  const int vs = v_slab(bs);
  const int g = h / (a.num_q_heads / hkv);
  int L = a.context_lens[b];
  L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
  const int64_t orow = ((int64_t)b * a.num_q_heads + h) * D;
  constexpr int MAXR = 4;  // head_dim <= 256
  float qd[MAXR], acc[MAXR];
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    const int d = lane + 64 * r;
    qd[r] = d < D ? load_elem<TT>(a.q, orow + d) : 0.f;
    acc[r] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int32_t* trow = a.block_tables + (int64_t)b * a.max_blocks_per_seq;
  for (int u = 0; u < L; ++u) {
    int blk = trow[u / bs];
    if (blk < 0 || (int64_t)blk >= a.num_blocks) blk = 0;
    const int off = u % bs;
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      const int d = lane + 64 * r;
      if (d < D)
        part += qd[r] * load_elem<TT>(a.k_cache, (((int64_t)blk * hkv + g) * bs + off) * D + d);
    }
    const float sc = wave_sum(part) * a.scale_log2e;
    const float m_new = fmaxf(m, sc);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    const float pw = __builtin_amdgcn_exp2f(sc - m_new);
    l = l * alpha + pw;
    m = m_new;
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      const int d = lane + 64 * r;
      if (d < D) {
        const int64_t vi =
            ((((int64_t)blk * hkv + g) * (bs / vs) + off / vs) * D + d) * vs + off % vs;
        acc[r] = acc[r] * alpha + pw * load_elem<TT>(a.v_cache, vi);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    const int d = lane + 64 * r;
    if (d < D) store_out<TT>(a.out, orow + d, L > 0 ? acc[r] / l : 0.f);
  }
}

template <typename TT, int D>
hipError_t launch_valu_d(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.max_parts, a.num_q_heads, a.num_seqs);
  if (a.block_size >= 16)
    hipLaunchKernelGGL((decode_valu_kernel<TT, D, 16>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((decode_valu_kernel<TT, D, 8>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <typename TT>
hipError_t launch_valu_t(const DecodeArgs& a, hipStream_t s) {
  switch (a.head_dim) {
    case 64: return launch_valu_d<TT, 64>(a, s);
    case 128: return launch_valu_d<TT, 128>(a, s);
    case 256: return launch_valu_d<TT, 256>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool decode_valu_supported(pa_dtype dt, int head_dim, int block_size) {
  (void)dt;
  const bool d_ok = head_dim == 64 || head_dim == 128 || head_dim == 256;
  const bool bs_ok = block_size == 8 || (block_size >= 16 && block_size % 16 == 0);
  return d_ok && bs_ok;
}

hipError_t launch_decode_valu(const DecodeArgs& a, pa_dtype dt, hipStream_t s) {
  if (a.num_seqs == 0) return hipSuccess;
  switch (dt) {
    case PA_F32: return launch_valu_t<F32>(a, s);
    case PA_F16: return launch_valu_t<F16>(a, s);
    case PA_BF16: return launch_valu_t<BF16>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_generic(const DecodeArgs& a, pa_dtype dt, hipStream_t s) {
  if (a.num_seqs == 0) return hipSuccess;
  dim3 grid(a.num_q_heads, a.num_seqs);
  switch (dt) {
    case PA_F32:
      hipLaunchKernelGGL(decode_generic_kernel<F32>, grid, dim3(64), 0, s, a);
      break;
    case PA_F16:
      hipLaunchKernelGGL(decode_generic_kernel<F16>, grid, dim3(64), 0, s, a);
      break;
    case PA_BF16:
      hipLaunchKernelGGL(decode_generic_kernel<BF16>, grid, dim3(64), 0, s, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace pa
