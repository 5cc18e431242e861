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
// decode_valu_kernel -- the MHA path (one q head per kv head read).  Work
// items are (sequence, q head); each wavefront is an independent worker that
// streams a contiguous, equal share of all items' 16-token steps
// (decode_split.h), writing finished rows or fp32 partials:
//   K  step = 16 token rows; lane (t = lane/4, c = lane%4) loads the 16-byte
//      chunks c, c+4, c+8, ... of row t (D/4 elements), so the four lanes of a
//      quad read 64 contiguous bytes per instruction; dot2 with the matching q
//      chunks, quad-reduce via DPP.
//   V  step = two 8-token slabs [D][8]; lane owns slab rows lane + 64*r, so
//      one load instruction covers 1 KiB of a slab contiguously and all lanes
//      hold the same 8 tokens -- the 16 weights are broadcast with readlane
//      into scalar registers, and each lane's accumulators are complete sums
//      needing no cross-lane reduction.
// The loads of a batch of steps are issued together, also across item
// boundaries.  Items split between workers are merged by decode_merge.hip.
//
// decode_generic_kernel -- any head_dim <= 256 / block_size / dtype, one
// wavefront per (q head, sequence), one token at a time.  Used for shapes the
// fast kernels do not cover (e.g. head_dim 16, block_size 4).
#include <math.h>

#include "decode_split.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStep = 16;  // tokens per wave step
// s_waitcnt operand: vmcnt 0, expcnt and lgkmcnt left at their maxima (gfx9 encoding)
constexpr int kVmcntZero = 0x0F70;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float bcast_lane(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}
__device__ __forceinline__ float wave_sum(float x) {
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
  return x;
}
__device__ __forceinline__ uint4 ld16(const char* p) {
  return *reinterpret_cast<const uint4*>(p);
}
// Streaming (non-temporal) 16-byte load for K/V data that is read exactly
// once per whole cache line: measured faster than a plain load on gfx950.
__device__ __forceinline__ uint4 ld16nt(const char* p) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

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

// V register j*R*NVR + r*NVR + u (piece j = tokens 8j .. 8j+7 of the step,
// slab row lane + 64*r, NVR uint4 per 8-token row piece) holds the tokens
// 8*j + u*EPV + e, EPV = elements per uint4.
template <typename TT, int R>
struct VMap {
  static constexpr int EPV = 16 / TT::bytes;
  static constexpr int NVR = 8 / EPV;
  static constexpr int token(int idx, int e) {
    return (idx / (R * NVR)) * 8 + (idx % NVR) * EPV + e;
  }
  static constexpr int row(int idx) { return (idx / NVR) % R; }
};

// acc[r] += sum_tau p[tau] * v[r][tau] over the lane's V elements.
template <typename TT, int R, int NK>
__device__ __forceinline__ void lane_pv(float (&acc)[R], const float (&p)[kStep],
                                        const uint4 (&v)[NK]) {
  using M = VMap<TT, R>;
#pragma unroll
  for (int i = 0; i < NK; ++i)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x = word(v[i], w);
      const int r = M::row(i);
      if constexpr (TT::bytes == 4) {
        acc[r] = fmaf(p[M::token(i, w)], __uint_as_float(x), acc[r]);
      } else {
        acc[r] = fmaf(p[M::token(i, 2 * w)], lo_to_float(TT{}, x), acc[r]);
        acc[r] = fmaf(p[M::token(i, 2 * w + 1)], hi_to_float(TT{}, x), acc[r]);
      }
    }
}

// Zero V elements of tokens >= nvalid (their bits may be NaN; 0 * NaN = NaN).
template <typename TT, int R, int NK>
__device__ __forceinline__ void mask_v(uint4 (&v)[NK], int nvalid) {
  using M = VMap<TT, R>;
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    uint32_t w4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if constexpr (TT::bytes == 4) {
        if (M::token(i, w) >= nvalid) w4[w] = 0u;
      } else {
        if (M::token(i, 2 * w) >= nvalid) w4[w] &= 0xffff0000u;
        if (M::token(i, 2 * w + 1) >= nvalid) w4[w] &= 0x0000ffffu;
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

// One element of a token row, widened.
template <typename TT>
__device__ __forceinline__ float new_elem(const char* p) {
  if constexpr (TT::bytes == 4)
    return *reinterpret_cast<const float*>(p);
  else
    return lo_to_float(TT{}, *reinterpret_cast<const uint16_t*>(p));
}

// Block-table window: lane i holds the physical id of logical block base + i
// (0 past the table row, and for ids outside the pool -- padding included --
// so that no entry ever produces an out-of-range address; such blocks only
// ever feed masked positions).
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

// FOLD (pa_decode_write): each sequence's last position, the new token, is
// left out of the stream -- it covers positions 0 .. L-2 -- and the worker
// that finishes an item adds the token's term from its K / V rows at that
// segment's end (one more online-softmax step of a single key), so a whole
// item still ends as its final row and a split one as partials that already
// hold the token.  The merge kernel stores the token into its slot.
//
// CASC (pa_decode_shared, tail pass): each sequence's steps start after its
// group's shared prefix (the prefix pass covers that), and a segment of such
// a sequence is always written as a partial, which the merge joins with the
// prefix pass's partial of the same row.
template <typename TT, int D, int NB, bool FOLD, bool CASC>
__global__ __launch_bounds__(kThreads) void decode_valu_kernel(DecodeArgs a) {
  constexpr int EB = TT::bytes;
  constexpr int NK = D * EB / 64;  // uint4 per lane per step, K and V alike
  constexpr int R = D / 64;        // slab rows owned by a lane
  constexpr int NVR = VMap<TT, R>::NVR;
  static_assert(R >= 1 && 2 * R * NVR == NK, "unsupported shape");
  extern __shared__ int smem[];  // split 1: s_pre[B+1], s_len[B], s_ppre[B+1]

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int worker = blockIdx.x * kWaves + wv;
  const int H = a.num_q_heads, B = a.num_seqs;
  const int group = H / a.num_kv_heads;
  const int bs = a.block_size;
  const int64_t hkv = a.num_kv_heads;
  const int tq = lane >> 2, c = lane & 3;
  const int C = a.part_steps;
  int* s_pre = smem;
  int* s_len = smem + B + 1;
  int* s_ppre = smem + 2 * B + 1;
  // CASC: first position and group of each sequence, group starts and prefixes
  int* s_st = smem + 3 * B + 2;
  int* s_grp = s_st + B;
  int* s_gs = s_grp + B;
  int* s_gp = s_gs + a.num_groups + 1;

  Cursor c0;
  int count;
  Split sp{};
  int64_t x0 = 0;  // split 1: first stream step of this worker
  if (a.split) {
    if constexpr (CASC) {
      if (wv == 0) load_groups(a, s_gs, s_gp);
      __syncthreads();
      if (wv == 0) wave_scan_tail(a, s_gs, s_gp, H, kStep, s_pre, s_len, s_st, s_grp);
    } else if (wv == 0) {
      wave_scan_steps(a.context_lens, B, H, a.len_cap, FOLD ? 1 : 0, kStep, C, s_pre, s_len,
                      s_ppre);
    }
    __syncthreads();
    if (blockIdx.x == 0 && wv == 0) {
      export_prefixes(s_pre, s_ppre, B, C, a.ws_pre, a.ws_ppre);
      if constexpr (CASC)
        export_groups(a, s_grp, s_gs, B);
    }
    const int N = s_pre[B];  // empty sequences get their zero rows from the merge
    if (N == 0) return;
    sp = make_split(a.num_workers, N, C, H, B, s_pre, s_ppre);
    if (worker >= sp.W) return;
    x0 = sp.start(worker);
    count = (int)(sp.start(worker + 1) - x0);
    c0 = locate(s_pre, s_len, CASC ? s_st : nullptr, B, H, kStep, (int)x0);
  } else {
    if (worker >= B * H) return;
    c0.b = worker / H;
    c0.h = worker % H;
    c0.k = 0;
    c0.s = 0;
    c0.L = clamp_len(a.context_lens[c0.b], a.len_cap);
    c0.n = (c0.L + kStep - 1) / kStep;
    count = c0.n;
    if (count == 0) {  // empty sequence: zero row
      const int64_t orow = ((int64_t)c0.b * H + c0.h) * D;
#pragma unroll
      for (int r = 0; r < R; ++r) store_out<TT>(a.out, orow + lane + 64 * r, 0.f);
      return;
    }
  }
  auto uniform = [](Cursor& x) {
    x.b = __builtin_amdgcn_readfirstlane(x.b);
    x.h = __builtin_amdgcn_readfirstlane(x.h);
    x.k = __builtin_amdgcn_readfirstlane(x.k);
    x.n = __builtin_amdgcn_readfirstlane(x.n);
    x.L = __builtin_amdgcn_readfirstlane(x.L);
    x.s = __builtin_amdgcn_readfirstlane(x.s);
  };
  uniform(c0);

  const char* kbase = reinterpret_cast<const char*>(a.k_cache);
  const char* vbase = reinterpret_cast<const char*>(a.v_cache);
  const char* qbase = reinterpret_cast<const char*>(a.q);

  // Block-table window of the sequence being issued (reloaded when the
  // sequence changes or the window runs out).
  TableWindow tw;
  int tw_b = -1;
  tw.base = 0;
  tw.entry = 0;

  // The step's tokens tok .. tok+15 form two 8-token slabs; slab j lies in
  // block (tok + 8j) / BS (BS is 8 or a multiple of 16).  The q slice of the
  // step's item travels with the step's K/V registers (reloaded only when the
  // buffer's item changes).
  // Loads that carry no data -- K rows of masked tokens, a masked second V
  // slab, and the whole issue when `live` is false (the pipeline's issue past
  // a worker's last step) -- are pointed at bytes this wavefront already has
  // in cache (token 0 of the same instruction, or the item's q row), so they
  // cost no HBM traffic while the number of loads, and so every wait count,
  // stays fixed.
  // FOLD: an item's last step also prefetches the new token's K pieces
  // c + 4i (kn) and V elements of rows lane + 64 r (vn), for the fold at the
  // end of that step; other steps load the same count from the item's q row
  // (in cache), so that the wait counts stay static.
  auto issue = [&](const Cursor& cu, uint4 (&kr)[NK], uint4 (&vr)[NK], uint4 (&qr)[NK],
                   int& qitem, bool live, uint4 (&kn)[NK], float (&vn)[R]) {
    const int item = cu.item(H);
    if constexpr (FOLD) {
      const bool want = live && cu.k == cu.n - 1;
      const int64_t row = (int64_t)cu.b * a.new_stride + (int64_t)(cu.h / group) * D;
      const char* kp = want ? reinterpret_cast<const char*>(a.k_new) + row * EB + c * 16
                            : qbase + (int64_t)item * D * EB + c * 16;
      const char* vp = want ? reinterpret_cast<const char*>(a.v_new) + row * EB
                            : qbase + (int64_t)item * D * EB;
#pragma unroll
      for (int i = 0; i < NK; ++i) kn[i] = ld16(kp + 64 * i);
#pragma unroll
      for (int r = 0; r < R; ++r) vn[r] = new_elem<TT>(vp + (lane + 64 * r) * EB);
    }
    if (qitem != item) {
      qitem = item;
      const char* qp = qbase + (int64_t)item * D * EB + c * 16;
#pragma unroll
      for (int i = 0; i < NK; ++i) qr[i] = ld16(qp + 64 * i);  // chunks c + 4i
    }
    const int32_t* trow = a.block_tables + (int64_t)cu.b * a.max_blocks_per_seq;
    const int tok = cu.tok(kStep);
    const int lb0 = tok / bs, lb1 = (tok + 8) / bs;
    if (tw_b != cu.b) {
      tw_b = cu.b;
      tw.load(trow, a.max_blocks_per_seq, a.num_blocks, lb0, lane);
    } else {
      tw.ensure(trow, a.max_blocks_per_seq, a.num_blocks, lb0, lb1 - lb0 + 1, lane);
    }
    const int64_t ph0 = tw.get(lb0), ph1 = tw.get(lb1);
    const int off0 = tok - lb0 * bs, off1 = tok + 8 - lb1 * bs;  // multiples of 8
    const int64_t g = cu.h / group;
    const int nv = cu.L - tok;  // valid tokens from tok on (>= 1)
    const char* cached = qbase + (int64_t)item * D * EB + ((lane * 16) & (D * EB - 1));
    {
      // 16-byte K piece c + 4i of token tq: for each i the wavefront reads
      // pieces 4i .. 4i+3 of 16 consecutive offsets, whole 128-byte lines.
      const bool kt = tq < nv;
      const bool hi = kt && tq >= 8;
      const int64_t phys = hi ? ph1 : ph0;
      const int off = (hi ? off1 : off0) + (kt ? (tq & 7) : 0);
      const char* kp = kbase + (((phys * hkv + g) * (4 * NK) + c) * bs + off) * 16;  // 4*NK pieces per row
      const int64_t pstride = (int64_t)4 * bs * 16;  // 4 pieces further
#pragma unroll
      for (int i = 0; i < NK; ++i) kr[i] = ld16nt(live ? kp + i * pstride : cached);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bool vlive = live && (j == 0 || nv > 8);
      const int64_t phys = j ? ph1 : ph0;
      const int off = j ? off1 : off0;
      const char* vp = vbase + (((phys * hkv + g) * (bs / 8) + off / 8) * D + lane) * (8 * EB);
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int u = 0; u < NVR; ++u)
          vr[(j * R + r) * NVR + u] =
              ld16nt(vlive ? vp + (int64_t)r * 64 * 8 * EB + 16 * u : cached);
    }
  };

  float m_run = -INFINITY, l_lane = 0.f;
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  int seg_k0 = c0.k;  // first step of the current segment within its item

  // A segment's result -- the item's final row, or its partial record --
  // waits in the registers of the step that ended it and is stored after the
  // next batch's loads are issued (flush): on this GPU a wavefront's stores
  // and loads share one wait counter, and a store issued before a load has to
  // complete before that load can be waited on (measured: the stores cost
  // the OPT-13B-shaped decode about 3.7 us when issued at the segment end).
  struct Pending {
    float v[R];     // output row values (final) or the partial's o
    float m, l;     // the partial's m and l
    int64_t dst;    // final row: element index of the row; partial: -(slot + 1)
    bool on;
  };
  auto store_result = [&](const Pending& p) {
    if (p.dst >= 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) store_out<TT>(a.out, p.dst + lane + 64 * r, p.v[r]);
    } else {
      // partial record (pa_internal.h): o, then the 128-byte m / l line
      float* rec = a.ws_part + (-p.dst - 1) * part_record(1, D);
#pragma unroll
      for (int r = 0; r < R; ++r) rec[lane + 64 * r] = p.v[r];
      if (lane < 32) rec[D + lane] = lane == 0 ? p.m : (lane == 16 ? p.l : 0.f);
    }
  };
  auto compute = [&](const Cursor& cu, const uint4 (&kr)[NK], uint4 (&vr)[NK],
                     const uint4 (&qr)[NK], int j, const uint4 (&kn)[NK], const float (&vn)[R],
                     Pending& pend) {
    if (segment_starts(cu, j)) {
      m_run = -INFINITY;
      l_lane = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = 0.f;
      seg_k0 = cu.k;
    }
    const int nvalid = min(kStep, cu.L - cu.tok(kStep));
    float d = lane_dot(TT{}, qr, kr);
    d += dpp<0xB1>(d);  // quad_perm [1,0,3,2]
    d += dpp<0x4E>(d);  // quad_perm [2,3,0,1]
    float sc = d * a.scale_log2e;
    if (tq >= nvalid) sc = -INFINITY;  // select, never multiply: masked K may be NaN
    float mx = fmaxf(sc, dpp<0x124>(sc));  // row_ror:4
    mx = fmaxf(mx, dpp<0x128>(mx));        // row_ror:8
    mx = xor16_max(mx);
    mx = xor32_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    const float pv = __builtin_amdgcn_exp2f(sc - m_new);
    l_lane = l_lane * alpha + (c == 0 ? pv : 0.f);
    m_run = m_new;
    float pt[kStep];
#pragma unroll
    for (int t = 0; t < kStep; ++t) pt[t] = bcast_lane(pv, 4 * t);
    if (nvalid < kStep) mask_v<TT, R, NK>(vr, nvalid);
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] *= alpha;
    lane_pv<TT, R, NK>(acc, pt, vr);

    if (segment_ends(cu, j, count - 1)) {
      if (FOLD && cu.k == cu.n - 1) {
        // the new token: score q . k_new (the quad's lanes hold q's pieces
        // c + 4i; so do their loads of k_new), weight, V row elements
        float sn = lane_dot(TT{}, qr, kn);
        sn += dpp<0xB1>(sn);
        sn += dpp<0x4E>(sn);
        sn *= a.scale_log2e;
        const float mn = fmaxf(m_run, sn);
        const float al = __builtin_amdgcn_exp2f(m_run - mn);
        const float pn = __builtin_amdgcn_exp2f(sn - mn);
        l_lane = l_lane * al + (lane == 0 ? pn : 0.f);
        m_run = mn;
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = fmaf(pn, vn[r], acc[r] * al);
      }
      const float l_tot = wave_sum(l_lane);
      const int item = cu.item(H);
      pend.on = true;
      if (seg_k0 == 0 && cu.k == cu.n - 1 && (!CASC || cu.s == 0)) {  // whole item: final row
        pend.dst = (int64_t)item * D;
#pragma unroll
        for (int r = 0; r < R; ++r) pend.v[r] = acc[r] / l_tot;
      } else {
        pend.dst = -((int64_t)item + worker) - 1;
        pend.m = m_run;
        pend.l = l_tot;
#pragma unroll
        for (int r = 0; r < R; ++r) pend.v[r] = acc[r];
      }
    }
  };

  // Steps are processed in batches of NB: the loads of all NB steps are
  // issued back to back, then the NB steps are computed in order.  A batch's
  // loads are in flight together while the other wavefronts of the CU
  // compute, and every load is consumed within the batch that issued it, so
  // the compiler's wait counts never hold a load of the next batch.  Issues
  // past the worker's last step read cached bytes (see `issue`).
  uint4 kr[NB][NK], vr[NB][NK], qr[NB][NK];
  uint4 kn[NB][NK];  // FOLD: the new token's rows, prefetched with its item's last step
  float vn[NB][R];
  int qi[NB];
  Pending pend[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    qi[u] = -1;
    pend[u].on = false;
  }
  auto flush = [&]() {
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (pend[u].on) {
        store_result(pend[u]);
        pend[u].on = false;
      }
  };
  Cursor cur = c0;
  for (int j = 0; j < count; j += NB) {
    Cursor cs[NB];
    cs[0] = cur;
#pragma unroll
    for (int u = 1; u < NB; ++u) {
      cs[u] = cs[u - 1];
      if (j + u < count) {
        advance(cs[u], s_pre, s_len, CASC ? s_st : nullptr, H, kStep);
        uniform(cs[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < NB; ++u)
      issue(cs[u], kr[u], vr[u], qr[u], qi[u], j + u < count, kn[u], vn[u]);
    flush();  // the previous batch's results, behind this batch's loads
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (j + u < count) compute(cs[u], kr[u], vr[u], qr[u], j + u, kn[u], vn[u], pend[u]);
    // All of the batch's loads have landed here on every path (the ones past
    // the last step are never consumed); saying so keeps the compiler from
    // waiting on them inside the next batch's issue.
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
    cur = cs[NB - 1];
    if (j + NB < count) {
      advance(cur, s_pre, s_len, CASC ? s_st : nullptr, H, kStep);
      uniform(cur);
    }
  }
  flush();
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
  // fused write (pa_decode_write): position L - 1 comes from the new rows
  const bool wr = a.k_new != nullptr && L > 0;
  const int64_t nrow = (int64_t)b * a.new_stride + (int64_t)g * D;
  for (int u = 0; u < L; ++u) {
    int blk = trow[u / bs];
    if (blk < 0 || (int64_t)blk >= a.num_blocks) blk = 0;
    const int off = u % bs;
    const bool nu = wr && u == L - 1;
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      const int d = lane + 64 * r;
      if (d < D)
        part += qd[r] * (nu ? load_elem<TT>(a.k_new, nrow + d)
                            : load_elem<TT>(a.k_cache,
                                            k_elem_index(blk, g, off, d, hkv, bs, D, TT::bytes)));
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
        acc[r] = acc[r] * alpha +
                 pw * (nu ? load_elem<TT>(a.v_new, nrow + d) : load_elem<TT>(a.v_cache, vi));
      }
    }
  }
  if (wr && h % (a.num_q_heads / hkv) == 0) {  // one q head per kv head stores the token
    const int pos = L - 1;
    const int blk = trow[pos / bs];
    const int off = pos % bs;
    if (blk >= 0 && (int64_t)blk < a.num_blocks) {
      using E = typename TT::raw;
      const E* kn = reinterpret_cast<const E*>(a.k_new);
      const E* vn = reinterpret_cast<const E*>(a.v_new);
      E* kc = reinterpret_cast<E*>(const_cast<void*>(a.k_cache));
      E* vc = reinterpret_cast<E*>(const_cast<void*>(a.v_cache));
#pragma unroll
      for (int r = 0; r < MAXR; ++r) {
        const int d = lane + 64 * r;
        if (d < D) {
          kc[k_elem_index(blk, g, off, d, hkv, bs, D, TT::bytes)] = kn[nrow + d];
          vc[((((int64_t)blk * hkv + g) * (bs / vs) + off / vs) * D + d) * vs + off % vs] =
              vn[nrow + d];
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    const int d = lane + 64 * r;
    if (d < D) store_out<TT>(a.out, orow + d, L > 0 ? acc[r] / l : 0.f);
  }
}

// Steps per batch: two while a lane's K / V / q registers of a step fit in
// 48 VGPRs (16-bit data up to D = 128, fp32 up to D = 64), else one, so
// that the kernel keeps at least two wavefronts per SIMD.  The plain
// decode of 16-bit data up to D = 128 takes three (186 VGPRs, still two
// wavefronts per SIMD): 107.0-107.3 against 108.0 us per OPT-13B-shaped
// call and 2636 against 2655 us on the OPT-66B-shaped batch; with the fused
// write (242 VGPRs) and in the shared decode's tail pass three were no
// faster.
template <typename TT, int D, bool FOLD, bool CASC>
constexpr int valu_batch() {
  return D * TT::bytes > 256 ? 1 : (TT::bytes == 2 && !FOLD && !CASC) ? 3 : 2;
}

template <typename TT, int D>
const void* valu_fn() {
  return reinterpret_cast<const void*>(
      &decode_valu_kernel<TT, D, valu_batch<TT, D, false, false>(), false, false>);
}

template <typename TT, int D>
hipError_t launch_valu_d(const DecodeArgs& a, hipStream_t s) {
  dim3 grid((a.num_workers + kWaves - 1) / kWaves);
  if (a.num_groups > 0)
    hipLaunchKernelGGL((decode_valu_kernel<TT, D, valu_batch<TT, D, false, true>(), false, true>),
                       grid, dim3(kThreads), decode_split_lds(a), s, a);
  else if (a.k_new)
    hipLaunchKernelGGL((decode_valu_kernel<TT, D, valu_batch<TT, D, true, false>(), true, false>),
                       grid, dim3(kThreads), decode_split_lds(a), s, a);
  else
    hipLaunchKernelGGL(
        (decode_valu_kernel<TT, D, valu_batch<TT, D, false, false>(), false, false>), grid,
        dim3(kThreads), decode_split_lds(a), s, a);
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

int decode_valu_waves_per_cu(pa_dtype dt, int head_dim) {
  const void* f = nullptr;
  switch (dt) {
    case PA_F32: f = head_dim == 64 ? valu_fn<F32, 64>() : head_dim == 128 ? valu_fn<F32, 128>()
                                                                            : valu_fn<F32, 256>();
      break;
    case PA_F16: f = head_dim == 64 ? valu_fn<F16, 64>() : head_dim == 128 ? valu_fn<F16, 128>()
                                                                            : valu_fn<F16, 256>();
      break;
    case PA_BF16: f = head_dim == 64 ? valu_fn<BF16, 64>() : head_dim == 128 ? valu_fn<BF16, 128>()
                                                                              : valu_fn<BF16, 256>();
      break;
  }
  int blocks = 0;
  if (!f || hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, f, kThreads, 0) != hipSuccess ||
      blocks <= 0)
    return kWaves;
  return blocks * kWaves;
}

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
