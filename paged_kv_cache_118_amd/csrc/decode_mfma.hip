// Paged decode attention for grouped-query heads on the gfx950 matrix cores.
//
// Same definition as decode_valu.hip (global softmax over all blocks, tail
// masked, stable online reduction: wq-win.github.io "079 | vLLM 与
// PagedAttention", section 二, the Z / o equations), for G = Hq / Hkv q heads
// sharing one kv head (the GQA storage the same page's section 二 mentions).
// The G q rows of one kv head form a real, if small, dense contraction, so
// each K and V element is read from HBM once per kv head and used G times.
//
// Work items are (sequence, kv head); every wavefront is an independent
// worker streaming an equal share of all items' 32-token groups
// (decode_split.h).  With lane = 16*kb + n (n = lane % 16,
// kb = lane / 16) and v_mfma_f32_16x16x32 (A: row n, k-slots of group kb;
// B: column n, same k-slots; C: column n, rows 4*kb .. 4*kb+3):
//   S^T = K Q^T  : A = K rows (tokens), B = Q^T (heads, zero past G), two
//                  16-token tiles x D/32 k-steps.  Tile j's row r is token
//                  16*j + r; k-step s of group kb is d = 32*s + 8*kb .. +7,
//                  i.e. 16-byte K piece 4*s + kb, so each load instruction
//                  reads pieces 4s .. 4s+3 of 16 consecutive offsets: whole
//                  128-byte lines of the piece-major K pool.  Lane (n, kb)
//                  gets the scores of head n for tokens 4*kb .. 4*kb+3 and
//                  16+4*kb .. 16+4*kb+3.
//   O^T += V^T P^T : A = V^T (16 d rows, 8 tokens per k-group, read as one
//                  16-byte row of an 8-token [D][8] V slab), B = P^T: lane
//                  (n, kb) needs the weights of tokens 8*kb .. 8*kb+7, which
//                  four lane permutes gather from the QK layout.  C = O^T
//                  keeps head n in lane n for every d tile, so the online-
//                  softmax rescale of the accumulators is lane-local.
// The max / sum over the 4 k-groups of a head cross lanes (xor 16, 32).
#include <math.h>

#include "decode_split.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kGroup = 32;  // tokens per wave step

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

// FOLD (pa_decode_write): each sequence's last position, the new token, is
// left out here -- the stream covers positions 0 .. L-2 -- and every segment
// is written as a partial, which the merge kernel combines with the new
// token's own term (fold_in_merge).
//
// CASC (pa_decode_shared): 1 = tail pass, as in decode_valu.hip (each
// sequence's steps start after its group's shared prefix; such sequences end
// in partials); 2 = prefix pass: items are (group, kv head), the group's
// shared prefix is the context, and the item's rows are the members' q heads
// of that kv head -- member m, q head h*G + i is row m*G + i (at most 16
// rows) -- so each shared block is read once for all of them; every segment
// ends in a 16-row partial for the merge.
template <typename TT, int D, bool FOLD, int CASC>
__global__ __launch_bounds__(kThreads, 2) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int VS = 8;       // V slab width (tokens)
  constexpr int EB = 2;
  constexpr int KN = D / 32;  // uint4 per lane per K tile (= QK k-steps)
  constexpr int MT = D / 16;  // d tiles of O^T
  extern __shared__ int smem[];  // split 1: s_pre[B+1], s_len[B], s_ppre[B+1]

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int worker = blockIdx.x * kWaves + wv;
  const int n = lane & 15, kb = lane >> 4;
  // the items' first index runs over sequences, or over groups (prefix pass)
  const int H = a.num_kv_heads, B = CASC == 2 ? a.num_groups : a.num_seqs;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int bs = a.block_size;
  const int64_t hkv = a.num_kv_heads;
  const int C = a.part_steps;
  int* s_pre = smem;
  int* s_len = smem + B + 1;
  int* s_ppre = smem + 2 * B + 1;
  // CASC 1: first position and group of each sequence; both passes: group
  // starts and prefix lengths
  int* s_st = smem + 3 * B + 2;
  int* s_grp = s_st + B;
  int* s_gs = CASC == 2 ? smem + 3 * B + 2 : s_grp + B;
  int* s_gp = s_gs + a.num_groups + 1;
  constexpr int RR = CASC == 2 ? kPrefixRows : 0;  // record rows (0: the group G)

  Cursor c0;
  int count;
  Split sp{};
  int64_t x0 = 0;  // split 1: first stream step of this worker
  if (a.split) {
    if constexpr (CASC != 0) {
      if (wv == 0) load_groups(a, s_gs, s_gp);
      __syncthreads();
    }
    if (wv == 0) {
      if constexpr (CASC == 1)
        wave_scan_tail(a, s_gs, s_gp, H, kGroup, s_pre, s_len, s_st, s_grp);
      else if constexpr (CASC == 2)  // the groups' prefixes are the contexts
        wave_scan_steps(s_gp, B, H, a.len_cap, 0, kGroup, 0, s_pre, s_len, s_ppre);
      else
        wave_scan_steps(a.context_lens, B, H, a.len_cap, FOLD ? 1 : 0, kGroup, C, s_pre, s_len,
                        s_ppre);
    }
    __syncthreads();
    if (blockIdx.x == 0 && wv == 0) {
      export_prefixes(s_pre, s_ppre, B, C, a.ws_pre, a.ws_ppre);
      if constexpr (CASC == 1)
        export_groups(a, s_grp, s_gs, B);
    }
    const int N = s_pre[B];  // empty sequences get their zero rows from the merge
    if (N == 0) return;
    sp = make_split(a.num_workers, N, C, H, B, s_pre, s_ppre);
    if (worker >= sp.W) return;
    x0 = sp.start(worker);
    count = (int)(sp.start(worker + 1) - x0);
    c0 = locate(s_pre, s_len, CASC == 1 ? s_st : nullptr, B, H, kGroup, (int)x0);
  } else {
    if (worker >= B * H) return;
    c0.b = worker / H;
    c0.h = worker % H;
    c0.k = 0;
    c0.s = 0;
    c0.L = clamp_len(a.context_lens[c0.b], a.len_cap);
    c0.n = (c0.L + kGroup - 1) / kGroup;
    count = c0.n;
    if (count == 0) {  // empty sequence: zero rows for the group's q heads
      const int64_t head0 = (int64_t)c0.b * a.num_q_heads + (int64_t)c0.h * G;
      for (int i = lane; i < G * D; i += 64) store_out<TT>(a.out, head0 * D + i, 0.f);
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
  // The sequence whose table and q rows an item uses (the group's first
  // member in the prefix pass), the q head of its row r, and its rows.
  // (Group starts are clamped to [0, num_seqs]; the first member to a real
  // sequence, so that malformed groups still read inside q and the tables.)
  auto seq_of = [&](const Cursor& cu) -> int {
    if constexpr (CASC == 2)
      return min(s_gs[cu.b], a.num_seqs - 1);
    else
      return cu.b;
  };
  auto row_head = [&](const Cursor& cu, int r) -> int64_t {
    if constexpr (CASC == 2)
      return (int64_t)min(seq_of(cu) + r / G, a.num_seqs - 1) * a.num_q_heads +
             (int64_t)cu.h * G + r % G;
    else
      return (int64_t)cu.b * a.num_q_heads + (int64_t)cu.h * G + r;
  };
  auto rows_of = [&](const Cursor& cu) -> int {
    if constexpr (CASC == 2)
      return min(kPrefixRows, max(s_gs[cu.b + 1] - s_gs[cu.b], 0) * G);
    else
      return G;
  };
  uniform(c0);

  const char* kbase = reinterpret_cast<const char*>(a.k_cache);
  const char* vbase = reinterpret_cast<const char*>(a.v_cache);
  const char* qbase = reinterpret_cast<const char*>(a.q);
  const int nb_grp = bs >= kGroup ? 1 : kGroup / bs;  // blocks touched by one group

  TableWindow tw;
  int tw_b = -1;
  tw.base = 0;
  tw.entry = 0;

  // K row of tile j for this lane plus (when the item changes) the Q^T
  // operand of the item: head n.  K-step s, element e of k-group kb carries
  // d = 32*s + 8*kb + e in both operands.
  constexpr int NC = D / 8;                     // 16-byte K pieces per token
  const int64_t pstride = (int64_t)4 * bs * 16;  // bytes from piece p to p + 4
  // Loads that carry no data -- K rows of masked tokens, V runs of masked
  // k-groups, and whole issues past the worker's last group (`live` false)
  // -- are pointed at bytes already in cache (the first row of the same
  // tile, or the item's first q row), so they cost no HBM traffic while the
  // number of loads, and so every wait count, stays fixed.
  auto cached_addr = [&](const Cursor& cu) {
    return qbase + row_head(cu, 0) * D * EB + ((lane * 16) & (D * EB - 1));
  };
  auto issue_k = [&](const Cursor& cu, uint4 (&kr)[2][KN], uint4 (&qr)[KN], int& qitem,
                     bool live) {
    const int item = cu.item(H);
    if (qitem != item) {
      qitem = item;
      const bool row = n < rows_of(cu);
      const char* qp = qbase + (row_head(cu, row ? n : 0) * D + kb * 8) * EB;
#pragma unroll
      for (int s = 0; s < KN; ++s) qr[s] = row ? ld16(qp + 64 * s) : make_uint4(0, 0, 0, 0);
    }
    const int32_t* trow = a.block_tables + (int64_t)seq_of(cu) * a.max_blocks_per_seq;
    const int tok = cu.tok(kGroup);
    const int lb0 = tok / bs;
    if (tw_b != cu.b) {
      tw_b = cu.b;
      tw.base = 0x7fffffff;
    }
    tw.ensure(trow, a.max_blocks_per_seq, a.num_blocks, lb0, nb_grp, lane);
    const int64_t g = cu.h;
    const int nv = cu.L - tok;  // valid tokens of the group (>= 1)
    const char* cached = cached_addr(cu);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bool tile = live && 16 * j < nv;  // the tile holds a valid token
      const int t = tok + 16 * j + (16 * j + n < nv ? n : 0);
      const int lb = t / bs;
      int64_t phys = tw.get(lb0);
      for (int q = 1; q < nb_grp; ++q)
        if (lb == lb0 + q) phys = tw.get(lb0 + q);
      const char* kp = kbase + (((phys * hkv + g) * NC + kb) * bs + (t - lb * bs)) * 16;
#pragma unroll
      for (int i = 0; i < KN; ++i) kr[j][i] = ld16nt(tile ? kp + i * pstride : cached);
    }
  };
  // The V token run of k-group kb (8 tokens of one slab row per d tile).  Its
  // group's K was issued earlier, so the table window already covers it.
  auto issue_v = [&](const Cursor& cu, uint4 (&vr)[MT], bool live) {
    const int tok = cu.tok(kGroup);
    const int lb0 = tok / bs;
    const bool run = live && kb * 8 < cu.L - tok;  // this k-group's 8 tokens hold data
    const int t = tok + kb * 8;
    const int lb = t / bs;
    int64_t phys = tw.get(lb0);
    for (int q = 1; q < nb_grp; ++q)
      if (lb == lb0 + q) phys = tw.get(lb0 + q);
    const int off = t - lb * bs;
    const char* vp =
        vbase + ((((phys * hkv + cu.h) * (bs / VS) + off / VS) * D + n) * VS) * EB;
    const char* cached = cached_addr(cu);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      vr[mt] = ld16nt(run ? vp + (int64_t)mt * 16 * VS * EB : cached);
  };

  float m_run = -INFINITY, l_lane = 0.f;
  float4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = float4_t{0.f, 0.f, 0.f, 0.f};
  int seg_k0 = c0.k;

  // Phase 1 of a group: S^T = K Q^T, online-softmax update, P^T operand.
  auto qk = [&](const Cursor& cu, const uint4 (&kr)[2][KN], const uint4 (&qr)[KN], int j,
                uint4& pb, int& nvalid) {
    if (segment_starts(cu, j)) {
      m_run = -INFINITY;
      l_lane = 0.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = float4_t{0.f, 0.f, 0.f, 0.f};
      seg_k0 = cu.k;
    }
    nvalid = min(kGroup, cu.L - cu.tok(kGroup));
    float4_t st[2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      st[jj] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < KN; ++i) st[jj] = mfma(TT{}, kr[jj][i], qr[i], st[jj]);
    }
    float sc[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sc[e] = st[0][e] * a.scale_log2e;
      sc[4 + e] = st[1][e] * a.scale_log2e;
    }
    if (nvalid < kGroup) {
#pragma unroll
      for (int e = 0; e < 8; ++e)  // token of sc[e]: 4*kb + e, then 16 + 4*kb + e-4
        if ((e < 4 ? 4 * kb + e : 12 + 4 * kb + e) >= nvalid)
          sc[e] = -INFINITY;  // select: masked K may be NaN
    }
    float mx = sc[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sc[e]);
    mx = xor16_max(mx);
    mx = xor32_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float pw[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pw[e] = __builtin_amdgcn_exp2f(sc[e] - m_new);
    m_run = m_new;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] *= alpha;
    // P^T operand: lane kb needs tokens 8*kb .. 8*kb+7, the 4-token runs of
    // tile kb/2 held by k-groups 2*(kb%2) and 2*(kb%2)+1.  Two permutes fetch
    // them.  In each, a source lane offers tile 0 or tile 1 by its own parity,
    // and the reader-to-source maps {0,2,1,3} and {1,3,0,2} send every reader
    // to a source offering the tile it needs.
    const uint32_t t0a = pack2(TT{}, pw[0], pw[1]), t0b = pack2(TT{}, pw[2], pw[3]);
    const uint32_t t1a = pack2(TT{}, pw[4], pw[5]), t1b = pack2(TT{}, pw[6], pw[7]);
    // the row sum takes the same rounded weights the P^T operand carries
    // (every token's pair sits in exactly one lane before the permutes)
    l_lane = psum2(TT{}, t1b, psum2(TT{}, t1a, psum2(TT{}, t0b, psum2(TT{}, t0a, l_lane * alpha))));
    const bool ev = (kb & 1) == 0;
    const int p1 = ((kb & 1) << 1) | (kb >> 1);
    const int src1 = (n + 16 * p1) * 4, src2 = (n + 16 * (p1 ^ 1)) * 4;
    const uint32_t a0 = __builtin_amdgcn_ds_bpermute(src1, ev ? t0a : t1a);
    const uint32_t a1 = __builtin_amdgcn_ds_bpermute(src1, ev ? t0b : t1b);
    const uint32_t b0 = __builtin_amdgcn_ds_bpermute(src2, ev ? t1a : t0a);
    const uint32_t b1 = __builtin_amdgcn_ds_bpermute(src2, ev ? t1b : t0b);
    pb = kb < 2 ? make_uint4(a0, a1, b0, b1) : make_uint4(b0, b1, a0, a1);
  };

  // Phase 2: O^T += V^T P^T, and the segment's output at its end.
  bool seg_end = false;  // pv ended a segment; finish stores its result
  auto pv = [&](const Cursor& cu, uint4 (&vr)[MT], const uint4& pb, int nvalid, int j) {
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
    for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma(TT{}, vr[mt], pb, acc[mt]);
    seg_end = segment_ends(cu, j, count - 1);
  };
  // The result of a segment that pv ended -- the item's final rows or its
  // partial record -- stored once the next group's K loads are issued: on
  // this GPU a wavefront's stores and loads share one wait counter, and a
  // store issued before a load has to complete before that load can be
  // waited on.  acc and the softmax state hold until the next step begins.
  auto finish = [&](const Cursor& cu) {
    {
      float l_tot = l_lane + __shfl_xor(l_lane, 16);
      l_tot += __shfl_xor(l_tot, 32);
      const int64_t orow0 = (int64_t)cu.b * a.num_q_heads + (int64_t)cu.h * G;
      if (!FOLD && CASC != 2 && (CASC == 0 || cu.s == 0) && seg_k0 == 0 &&
          cu.k == cu.n - 1) {  // the whole item: final rows
        if (n < G) {
          const int64_t orow = (orow0 + n) * D;
          const float inv = 1.f / l_tot;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              store_out<TT>(a.out, orow + mt * 16 + 4 * kb + e, acc[mt][e] * inv);
        }
      } else {
        // Partial record (pa_internal.h): for each d tile the group's lanes
        // write one contiguous run of 64 G bytes; then the 128-byte m / l
        // line, written whole (lanes kb = 2, 3 write its zero half).
        const int64_t slot = (int64_t)cu.item(H) + worker;
        const int rr = RR ? RR : G, nr = rows_of(cu);
        float* rec = a.ws_part + slot * part_record(rr, D);
        if (n < nr) {
          float* o = rec + (kb * rr + n) * 4;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) *reinterpret_cast<float4_t*>(o + mt * 16 * rr) = acc[mt];
        }
        if (lane < 32) rec[rr * D + lane] = (lane & 15) < nr ? (lane < 16 ? m_run : l_tot) : 0.f;
      }
    }
  };

  auto next = [&](Cursor& c, int idx) {  // cursor of group idx, given idx-1's
    if (idx < count) {
      advance(c, s_pre, s_len, CASC == 1 ? s_st : nullptr, H, kGroup);
      uniform(c);
    }
  };
  // Pipeline, per group j: qk(j) | issue V(j+1) | pv(j) | issue K(j+2).
  // Each load is issued a full group ahead of its use, yet only three of
  // the four K/V register sets are live at any time.  Issues past the
  // worker's last group read cached bytes instead, keeping the waits static.
  uint4 kA[2][KN], kB[2][KN], vA[MT], vB[MT], qA[KN], qB[KN];
  int qia = -1, qib = -1;
  Cursor c1 = c0;
  next(c1, 1);
  issue_k(c0, kA, qA, qia, true);
  issue_v(c0, vA, true);
  issue_k(c1, kB, qB, qib, 1 < count);
  int j = 0;
  for (;;) {
    Cursor c2 = c1;
    next(c2, j + 2);
    {
      uint4 pb;
      int nv;
      qk(c0, kA, qA, j, pb, nv);
      issue_v(c1, vB, j + 1 < count);
      pv(c0, vA, pb, nv, j);
      issue_k(c2, kA, qA, qia, j + 2 < count);
      if (seg_end) finish(c0);
    }
    if (++j >= count) break;
    c0 = c1;
    c1 = c2;
    c2 = c1;
    next(c2, j + 2);
    {
      uint4 pb;
      int nv;
      qk(c0, kB, qB, j, pb, nv);
      issue_v(c1, vA, j + 1 < count);
      pv(c0, vB, pb, nv, j);
      issue_k(c2, kB, qB, qib, j + 2 < count);
      if (seg_end) finish(c0);
    }
    if (++j >= count) break;
    c0 = c1;
    c1 = c2;
  }
}

template <typename TT, int D>
const void* mfma_fn() {
  return reinterpret_cast<const void*>(&decode_mfma_kernel<TT, D, false, 0>);
}

template <typename TT, int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
  dim3 grid((a.num_workers + kWaves - 1) / kWaves);
  if (a.num_groups > 0)
    hipLaunchKernelGGL((decode_mfma_kernel<TT, D, false, 1>), grid, dim3(kThreads),
                       decode_split_lds(a), s, a);
  else if (a.k_new)
    hipLaunchKernelGGL((decode_mfma_kernel<TT, D, true, 0>), grid, dim3(kThreads),
                       decode_split_lds(a), s, a);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<TT, D, false, 0>), grid, dim3(kThreads),
                       decode_split_lds(a), s, a);
  return hipGetLastError();
}

// The prefix pass of a shared-prefix decode: a.num_workers, a.ws_part and
// a.ws_pre are the pass's own (the caller swaps them in).
template <typename TT, int D>
hipError_t launch_prefix_d(const DecodeArgs& a, hipStream_t s) {
  dim3 grid((a.num_workers + kWaves - 1) / kWaves);
  const size_t lds = split_lds_bytes(a.num_groups) + sizeof(int) * (2 * (size_t)a.num_groups + 1);
  hipLaunchKernelGGL((decode_mfma_kernel<TT, D, false, 2>), grid, dim3(kThreads), lds, s, a);
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

int decode_mfma_waves_per_cu(pa_dtype dt, int head_dim) {
  const void* f = dt == PA_F16 ? (head_dim == 64 ? mfma_fn<F16, 64>() : mfma_fn<F16, 128>())
                               : (head_dim == 64 ? mfma_fn<BF16, 64>() : mfma_fn<BF16, 128>());
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, f, kThreads, 0) != hipSuccess ||
      blocks <= 0)
    return kWaves;
  return blocks * kWaves;
}

hipError_t launch_decode_prefix(const DecodeArgs& a, pa_dtype dt, hipStream_t s) {
  if (a.num_groups == 0) return hipSuccess;
  if (dt == PA_F16) return a.head_dim == 64 ? launch_prefix_d<F16, 64>(a, s)
                                            : launch_prefix_d<F16, 128>(a, s);
  if (dt == PA_BF16) return a.head_dim == 64 ? launch_prefix_d<BF16, 64>(a, s)
                                             : launch_prefix_d<BF16, 128>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, pa_dtype dt, hipStream_t s) {
  if (a.num_seqs == 0) return hipSuccess;
  if (dt == PA_F16) return launch_t<F16>(a, s);
  if (dt == PA_BF16) return launch_t<BF16>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace pa
