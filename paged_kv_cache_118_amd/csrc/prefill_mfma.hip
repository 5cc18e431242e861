// Paged chunked-prefill attention on the gfx950 matrix cores.
//
// A prompt processed in chunks (zhy-blog.vercel.app vLLM post, section 4.2
// "Chunked Prefill的解决方案"): the chunk's query tokens are the last ql tokens
// of their sequence's context (their K/V already written to the pool), and
// each attends to the cache through the block table with a mask set by its
// position in the whole prompt: token at position p sees positions 0 .. p.
// One softmax over all of them (the Z / o equations of wq-win.github.io "079 |
// vLLM 与 PagedAttention", section 二), evaluated online in the base-2 domain.
// Query rows are packed [num_tokens][num_q_heads][head_dim] as in the forward
// of gitcode.csdn.net "vLLM 推理引擎：PagedAttention 与 KVCache 管理", section 3.
//
// Unlike decode, each K/V element now meets many queries, so the work is a
// real dense contraction.  A wavefront owns 16 or 32 query rows of one q
// head; a workgroup holds 2 or 4 consecutive row tiles of the same head and
// stages each key group's K/V once in LDS for all of them; all workgroups
// reading one kv head's K/V run on one XCD at about the same time, so the
// cache lines of a key group come from HBM about once and are served to the
// others from L2 (plain, temporal loads).  16-row tiles, with lane =
// 16*kb + n and v_mfma_f32_16x16x32 (32-row tiles: see compute32):
//   S^T = K Q^T  : A = 16 keys x 32 dims (16-byte K pieces), B = Q^T (query
//                  row n), two 16-key tiles per 32-key group whose rows are
//                  ordered so that lane (n, kb) gets query n's scores of keys
//                  8kb .. 8kb+7;
//   O^T += V^T P^T : A = 16 dims x 32 keys (one 16-byte row of an 8-token V
//                  slab per k-group), B = P^T, those eight scores packed.
// The mask compares each key's position with the lane's query position, so
// only the groups that reach past the tile's first row pay for it.
#include <math.h>
#include <stdlib.h>

#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kKeys = 32;  // keys per step

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;
// s_waitcnt operand: vmcnt 0, expcnt and lgkmcnt at their maxima (gfx9).
constexpr int kVmcntZero = 0x0F70;

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
// v_mfma_f32_32x32x16: lane l holds A[row l % 32][k 8 (l / 32) .. +7],
// B[k 8 (l / 32) .. +7][column l % 32], and C register r is
// C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
typedef float float16_t __attribute__((ext_vector_type(16)));
__device__ __forceinline__ float16_t mfma32(F16, const uint4& a, const uint4& b, float16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a),
                                                __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ float16_t mfma32(BF16, const uint4& a, const uint4& b, float16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf168_t, a),
                                                 __builtin_bit_cast(bf168_t, b), c, 0, 0, 0);
}
// Two fp32 values to one packed pair, round to nearest even (one
// v_cvt_pk_{f16,bf16}_f32).
__device__ __forceinline__ uint32_t pack2(F16, float lo, float hi) {
  const half2_t h = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ uint32_t pack2(BF16, float lo, float hi) {
  const bf162_t h = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, h);
}

// Lane i holds the physical id of logical block base + i (0 for entries past
// the row or outside the pool: such blocks only feed masked keys).
struct TableWindow {
  int base = 0x7fffffff;
  int entry = 0;
  __device__ __forceinline__ void load(const int32_t* row, int nblk, int64_t num_blocks, int lb,
                                       int lane) {
    base = lb;
    const int idx = lb + lane;
    const int e = idx < nblk ? row[idx] : 0;
    entry = (e < 0 || (int64_t)e >= num_blocks) ? 0 : e;
  }
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

// Slack of the running maximum (base-2 exponent): the output accumulators are
// rescaled only when a row's maximum grows by more than this, so the weights
// exp2(s - m) stay below 2^kSlack -- harmless in fp32 sums and 16-bit P
// (relative precision does not depend on magnitude) -- and most key groups
// skip the rescale altogether.
constexpr float kSlack = 8.f;

// Sequences up to which the workgroups take them longest context first.
constexpr int kOrderSeqs = 64;
// Block ids of rows up to this many blocks are staged in LDS for the direct
// loads (4 KiB per workgroup); longer rows read them through a table window.
constexpr int kTabBlocks = 1024;

// Longest query chunk from which the 32-rows-per-wavefront kernel is used.
constexpr int kPrefill32MinRows = 64;


// NBG = physical blocks one 32-key group spans: 4 (block size 8), 2 (16),
// 1 (a multiple of 32).
//
// The WV wavefronts of a workgroup hold WV * WR consecutive query rows of one
// q head and need the same keys, so each 32-key group's K and V are loaded
// from the pool once per workgroup, by all its threads, into LDS, and every
// wavefront reads its MFMA operands from there; two LDS buffers alternate,
// one barrier per group.  The loads take one of two routes:
//  - DMA (32-row wavefronts): global_load_lds straight into LDS, one group
//    ahead (layout at the kernel's LDS declarations);
//  - registers (16-row wavefronts, or PA_PREFILL_DMA=0): 16-byte loads two
//    groups ahead into registers, written to LDS at the top of the group's
//    step.  K in LDS: 32 rows [key][D], pitch D*2 + 16 bytes (the 16 keys
//    one operand read touches fall in distinct banks); V: 4 slabs of 8 keys,
//    [slab][D][8], as in the pool, pitch D*16 + 16.
// WR = query rows per wavefront: 16 (16x16x32 MFMAs) or 32 (32x32x16 MFMAs,
// each K/V operand read from LDS then serves twice as many rows); WV =
// wavefronts per workgroup; DMA = the load route.
template <typename TT, int D, int NBG, int WR, int WV, bool DMA>
__global__ __launch_bounds__(64 * WV) void prefill_mfma_kernel(PrefillArgs a) {
  constexpr int kWaves = WV;
  constexpr int kThreads = 64 * WV;
  constexpr int VS = 8;       // V slab width (tokens)
  constexpr int EB = 2;
  constexpr int KN = D / 32;  // k-steps of S^T
  constexpr int MT = D / 16;  // d tiles of O^T
  constexpr int NC = D / 8;   // 16-byte K pieces per token
  constexpr int KP = D * EB + 16;          // LDS pitch of a K row
  constexpr int VSP = D * VS * EB + 16;    // LDS pitch of a V slab
  constexpr int KBUF = kKeys * KP;
  constexpr int BUF = KBUF + (kKeys / VS) * VSP;
  constexpr int NCK = kKeys * NC / kThreads;       // K chunks per thread and group
  constexpr int NCV = (kKeys / VS) * D / kThreads;  // V chunks per thread and group
  static_assert(NCK >= 1 && NCV >= 1, "head_dim too small for the cooperative load");
  // Direct global -> LDS loads (32-row wavefronts): each 16-byte load of a
  // wavefront lands at LDS base + 16 * lane, so a load instruction fills 1
  // KiB contiguously and the layout is chosen by what each lane fetches:
  //   K: [piece][32 keys][16 B], key slot s of a piece row holding key
  //      krow(s) -- the key the S^T operand's lane s reads -- so a half
  //      wavefront's operand read is one contiguous 512-byte run;
  //   V: [slab][D][16 B], as in the pool, unpadded.
  // No staging registers: the loads of group g + 1 fly while group g is
  // computed and the wavefront waits for them before the next barrier.
  static_assert(!DMA || WR == 32, "direct LDS loads only with 32-row wavefronts");
  constexpr int KBUFD = NC * kKeys * 16;
  constexpr int BUFD = KBUFD + (kKeys / VS) * D * 16;
  constexpr int NID = 2 * D / 16;  // 1-KiB load instructions per group (K, then V)
  static_assert(!DMA || NID % (2 * WV) == 0, "direct loads must split evenly over the wavefronts");
  __shared__ __align__(16) char lds[DMA ? BUFD : 2 * BUF];
  // second buffer of the direct-load path, a separate object: with both
  // buffers in one array the compiler could not tell the operand reads of
  // one from the loads in flight into the other, and waited for the loads
  __shared__ __align__(16) char lds_b[DMA ? BUFD : 16];
  __shared__ int s_tab[DMA && NBG <= 2 ? kTabBlocks : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, kb = lane >> 4;  // 16-row lane roles
  const int c32 = lane & 31, hh = lane >> 5;  // 32-row lane roles
  const int qrow = WR == 16 ? n : c32;        // the lane's query row in the tile
  const int G = a.num_q_heads / a.num_kv_heads;
  // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin by id, so
  // every workgroup of one (sequence, kv head) unit -- its q heads and query
  // tiles, which read the same K/V -- gets ids of one residue mod 8 (the same
  // XCD and L2) and consecutive in time.
  const int tpg = (a.max_query_len + kWaves * WR - 1) / (kWaves * WR);
  const int sub_n = G * tpg;  // workgroups per unit
  const int id = blockIdx.x;
  const int unit = (id / 8 / sub_n) * 8 + id % 8;  // rank of the unit in dispatch order
  const int sub = (id / 8) % sub_n;
  if (unit >= a.num_seqs * a.num_kv_heads) return;
  int seq = unit / a.num_kv_heads;
  // Longest contexts first (up to kOrderSeqs sequences): the workgroups are
  // dispatched in id order as slots free up, so starting the long units
  // first keeps one of them from setting the end of the kernel.  The rank of
  // a sequence counts the longer ones (ties by index); every workgroup
  // ranks the clamped lengths itself.
  if (a.num_seqs <= kOrderSeqs) {
    __shared__ int s_clen[kOrderSeqs];
    __shared__ int s_order[kOrderSeqs];
    const int B = a.num_seqs;
    if (tid < B) {
      const int Lt = a.context_lens[tid];
      s_clen[tid] = Lt < 0 ? 0 : (Lt > a.len_cap ? a.len_cap : Lt);
    }
    __syncthreads();
    if (tid < B) {
      const int mine = s_clen[tid];
      int rank = 0;
      for (int j = 0; j < B; ++j) {
        const int o = s_clen[j];
        rank += o > mine || (o == mine && j < tid);
      }
      s_order[rank] = tid;
    }
    __syncthreads();
    seq = s_order[seq];
  }
  const int h = (unit % a.num_kv_heads) * G + sub / tpg;
  const int qs = a.query_start[seq];
  const int ql = a.query_start[seq + 1] - qs;
  int L = a.context_lens[seq];
  L = L < 0 ? 0 : (L > a.len_cap ? a.len_cap : L);
  const int rwg = (sub % tpg) * kWaves * WR;  // the workgroup's first row
  if (ql <= 0 || ql > L || rwg >= ql) return;   // (ql > L is a caller error: rows left alone)
  const int last_wg = L - ql + min(ql, rwg + kWaves * WR) - 1;  // last position any row needs
  const int r0 = rwg + wv * WR;                    // this wavefront's first row
  const int nrows = max(0, min(ql - r0, WR));      // 0: the wavefront only helps to load
  const int pos0 = L - ql + r0;                    // position of the tile's first row
  const int last = pos0 + max(nrows, 1) - 1;       // position of its last valid row
  const int mypos = pos0 + (qrow < nrows ? qrow : max(nrows, 1) - 1);  // the lane's query position
  const int64_t g = h / G;
  const int64_t hkv = a.num_kv_heads;
  // block size: a compile-time constant for groups spanning 2 or 4 blocks
  constexpr int BSC = NBG == 4 ? 8 : NBG == 2 ? 16 : 0;
  const int bs = BSC ? BSC : a.block_size;
  const int64_t kblock = (int64_t)hkv * NC * bs * 16;  // bytes of one block of the K pool
  const int64_t vblock = (int64_t)hkv * D * bs * EB;   // ... and of the V pool
  const int64_t khead = g * NC * bs * 16, vhead = g * D * bs * EB;

  const char* kbase = reinterpret_cast<const char*>(a.k_cache);
  const char* vbase = reinterpret_cast<const char*>(a.v_cache);
  const char* qbase = reinterpret_cast<const char*>(a.q);
  const int32_t* trow = a.block_tables + (int64_t)seq * a.max_blocks_per_seq;

  // Q^T operand: query row qrow of the tile, the lane's k-slices -- dims
  // 32 s + 8 kb .. +7 (16 rows) or 16 s + 8 hh .. +7 (32 rows) -- zero for
  // rows past the chunk.
  constexpr int QN = WR == 16 ? D / 32 : D / 16;
  uint4 qr[QN];
  {
    const int64_t row = (int64_t)qs + (qrow < nrows ? r0 + qrow : 0);
    const char* qp = qbase + ((row * a.num_q_heads + h) * D + (WR == 16 ? kb : hh) * 8) * EB;
#pragma unroll
    for (int s = 0; s < QN; ++s)
      qr[s] = qrow < nrows ? ld16(qp + (WR == 16 ? 64 : 32) * s) : make_uint4(0, 0, 0, 0);
  }
  // Scores are used as s * scl with scl = |scale * log2 e| >= 0 (so the
  // maximum of the raw dot products gives the maximum score, and the scale
  // folds into the exponent's fma); a negative scale flips q's sign bits
  // instead, which is exact.
  const float scl = fabsf(a.scale_log2e);
  if (a.scale_log2e < 0.f) {
#pragma unroll
    for (int s = 0; s < QN; ++s) {
      qr[s].x ^= 0x80008000u;
      qr[s].y ^= 0x80008000u;
      qr[s].z ^= 0x80008000u;
      qr[s].w ^= 0x80008000u;
    }
  }

  float m_run = -INFINITY, l_lane = 0.f;
  float4_t acc[MT];        // 16 rows: O^T tile mt (dims 16 mt ..)
  float16_t acc32[D / 32];  // 32 rows: O^T tile mt (dims 32 mt ..)
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc32[mt][r] = 0.f;

  TableWindow tw;
  const int ngroups = last_wg / kKeys + 1;
  // Keys past the workgroup's last position are loaded from that position
  // instead (valid, finite data; their scores are masked).  Only a V slab
  // that reaches past the context can hold bytes that were never written
  // (NaN in tests): those elements are zeroed after the operand read.
  const bool vtail = (last_wg | (VS - 1)) >= L;

  // Cooperative loads of group grp into registers: K chunk c = tid + 256 r
  // is piece c / 32 of key c % 32; V chunk c is row c % D of slab c / D.
  auto load = [&](int grp, uint4 (&pk)[NCK], uint4 (&pv)[NCV]) {
    const int tok = grp * kKeys;
    const int lb0 = BSC ? tok / BSC : tok / bs;
    if (lb0 < tw.base || lb0 + NBG > tw.base + 64)
      tw.load(trow, a.max_blocks_per_seq, a.num_blocks, lb0, lane);
    const uint32_t o0 = (uint32_t)(tok - lb0 * bs);  // 0 unless NBG == 1
    const uint32_t lim = (uint32_t)(last_wg - tok);
    const char* kblk[NBG];
    const char* vblk[NBG];
#pragma unroll
    for (int q = 0; q < NBG; ++q) {
      const int64_t ph = tw.get(lb0 + q);
      kblk[q] = kbase + ph * kblock + khead;
      vblk[q] = vbase + ph * vblock + vhead;
    }
    // base of the block holding key tok + rel
    auto pick = [&](const char* const (&b)[NBG], uint32_t rel) {
      if constexpr (NBG == 4) {
        // bit tests on copies of the four bases: with a chain of compares
        // the compiler formed an indexed load from the array, which put the
        // array in scratch memory
        const char* b0 = b[0];
        const char* b1 = b[1];
        const char* b2 = b[2];
        const char* b3 = b[3];
        const uint32_t q = rel / (uint32_t)(BSC > 0 ? BSC : 1);  // 0 .. 3
        const char* lo = (q & 1) ? b1 : b0;
        const char* hi = (q & 1) ? b3 : b2;
        return (q & 2) ? hi : lo;
      } else {
        const char* p = b[0];
        if constexpr (NBG > 1) p = rel >= (uint32_t)BSC ? b[1] : p;
        return p;
      }
    };
#pragma unroll
    for (int r = 0; r < NCK; ++r) {
      const int c = tid + kThreads * r;
      const uint32_t rel = min((uint32_t)(c % kKeys), lim);
      const uint32_t off = NBG == 1 ? o0 + rel : rel & (uint32_t)(BSC - 1);
      pk[r] = ld16(pick(kblk, rel) + ((uint32_t)(c / kKeys) * bs + off) * 16);
    }
#pragma unroll
    for (int r = 0; r < NCV; ++r) {
      const int c = tid + kThreads * r;
      const uint32_t relv = min((uint32_t)(c / D) * VS, lim & ~(uint32_t)(VS - 1));
      const uint32_t offv = NBG == 1 ? o0 + relv : relv & (uint32_t)(BSC - 1);
      pv[r] = ld16(pick(vblk, relv) + ((offv / VS) * D + (uint32_t)(c % D)) * (VS * EB));
    }
  };
  // Direct loads of group grp into LDS buffer buf: a K load instruction i
  // (i < D / 16) fills pieces 2 i and 2 i + 1 (lane: piece 2 i + lane / 32,
  // key krow(lane % 32)), a V load instruction iv 64 rows of slab
  // iv / (D / 64).
  // TAB: the block ids come from the row staged in s_tab (no window check in
  // the loop: 2% fewer cycles on the 66B chunk writers), else from the window
  auto dma = [&](int grp, char* buf, auto tab) {
    constexpr bool TAB = decltype(tab)::value;
    const int tok = grp * kKeys;
    const int lb0 = tok / (BSC ? BSC : bs);
    if (!TAB && (lb0 < tw.base || lb0 + NBG > tw.base + 64))
      tw.load(trow, a.max_blocks_per_seq, a.num_blocks, lb0, lane);
    const uint32_t o0 = (uint32_t)(tok - lb0 * bs);
    const uint32_t lim = (uint32_t)(last_wg - tok);
    const char* kblk[NBG];
    const char* vblk[NBG];
#pragma unroll
    for (int q = 0; q < NBG; ++q) {
      const int64_t ph = TAB ? __builtin_amdgcn_readfirstlane(s_tab[lb0 + q]) : tw.get(lb0 + q);
      kblk[q] = kbase + ph * kblock + khead;
      vblk[q] = vbase + ph * vblock + vhead;
    }
    auto pick = [&](const char* const (&b)[NBG], uint32_t rel) {
      if constexpr (NBG == 4) {
        const char* b0 = b[0];
        const char* b1 = b[1];
        const char* b2 = b[2];
        const char* b3 = b[3];
        const uint32_t q = rel / (uint32_t)(BSC > 0 ? BSC : 1);
        const char* lo = (q & 1) ? b1 : b0;
        const char* hi = (q & 1) ? b3 : b2;
        return (q & 2) ? hi : lo;
      } else {
        const char* p = b[0];
        if constexpr (NBG > 1) p = rel >= (uint32_t)BSC ? b[1] : p;
        return p;
      }
    };
    const int key = 16 * (c32 >> 4) + 8 * ((c32 >> 2) & 1) + 4 * ((c32 >> 3) & 1) + (c32 & 3);
    const uint32_t rel = min((uint32_t)key, lim);
    const uint32_t off = NBG == 1 ? o0 + rel : rel & (uint32_t)(BSC - 1);
    const char* kp = pick(kblk, rel) + ((uint32_t)hh * bs + off) * 16;  // piece hh of the key
    // every wavefront issues NID / (2 WV) K loads, then as many V loads
    constexpr int NIH = NID / 2 / WV;
#pragma unroll
    for (int t = 0; t < NIH; ++t) {
      const int i = wv * NIH + t;  // K pieces 2 i, 2 i + 1
      __builtin_amdgcn_global_load_lds((glb_void*)(kp + (int64_t)2 * i * bs * 16),
                                       (lds_void*)(buf + i * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < NIH; ++t) {
      const int iv = wv * NIH + t, slab = iv / (D / 64);  // rows (iv % (D / 64)) * 64 + lane
      const uint32_t relv = min((uint32_t)slab * VS, lim & ~(uint32_t)(VS - 1));
      const uint32_t offv = NBG == 1 ? o0 + relv : relv & (uint32_t)(BSC - 1);
      const char* vp = pick(vblk, relv) +
                       ((offv / VS) * D + (uint32_t)((iv % (D / 64)) * 64 + lane)) * (VS * EB);
      __builtin_amdgcn_global_load_lds((glb_void*)vp, (lds_void*)(buf + KBUFD + iv * 1024), 16, 0,
                                       0);
    }
  };
  auto store = [&](char* buf, const uint4 (&pk)[NCK], const uint4 (&pv)[NCV]) {
#pragma unroll
    for (int r = 0; r < NCK; ++r) {
      const int c = tid + kThreads * r;
      *reinterpret_cast<uint4*>(buf + (c % kKeys) * KP + (c / kKeys) * 16) = pk[r];
    }
#pragma unroll
    for (int r = 0; r < NCV; ++r) {
      const int c = tid + kThreads * r;
      *reinterpret_cast<uint4*>(buf + KBUF + (c / D) * VSP + (c % D) * 16) = pv[r];
    }
  };

  auto compute = [&](int grp, const char* buf) {
    const int tok = grp * kKeys;
    // Operands are read from LDS next to the matrix op that takes them (fewer
    // registers, four wavefronts per SIMD to cover the reads).
    // Row r of tile j's A operand is key 8 (r / 4) + 4 j + r % 4, so the
    // output lane (n, kb) holds query n's scores of keys 8 kb .. 8 kb + 3
    // (tile 0) and 8 kb + 4 .. 8 kb + 7 (tile 1): exactly the eight keys its
    // slice of the P^T operand needs, with no lane exchange.
    float4_t st[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      st[j] = float4_t{0.f, 0.f, 0.f, 0.f};
      const char* kr = buf + (8 * (n >> 2) + 4 * j + (n & 3)) * KP + kb * 16;
#pragma unroll
      for (int i = 0; i < KN; ++i)
        st[j] = mfma(TT{}, *reinterpret_cast<const uint4*>(kr + 64 * i), qr[i], st[j]);
    }
    const char* vr = buf + KBUF + kb * VSP + n * 16;  // V^T operand: slab kb, row d = n + 16 mt
    float sc[8];  // raw dot products; the score is sc * scl
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sc[e] = st[0][e];
      sc[4 + e] = st[1][e];
    }
    if (tok + kKeys - 1 > pos0) {  // the group reaches past the tile's first row
#pragma unroll
      for (int e = 0; e < 8; ++e)  // key of sc[e]: 8 kb + e
        if (tok + 8 * kb + e > mypos) sc[e] = -INFINITY;  // select: masked scores may be NaN
    }
    float mx = sc[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sc[e]);
    mx = xor16_max(mx);
    mx = xor32_max(mx) * scl;
    // mx is finite: key 0 is in every row's range, and the first group of
    // every row reaches here with m_run = -inf
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kSlack) != 0) {
      const float m_new = mx > m_run + kSlack ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_lane *= alpha;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] *= alpha;
      m_run = m_new;
    }
    float pw[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pw[e] = __builtin_amdgcn_exp2f(fmaf(sc[e], scl, -m_run));
    if (tok + kKeys - 1 > pos0) {  // masked keys weigh 0 also at scale 0 (-inf * 0 is NaN)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (tok + 8 * kb + e > mypos) pw[e] = 0.f;
    }
    // P^T operand: keys 8 kb .. 8 kb + 7 of query n, all held by this lane;
    // the row sum takes the same rounded weights the matrix op does
    const uint4 pb = make_uint4(pack2(TT{}, pw[0], pw[1]), pack2(TT{}, pw[2], pw[3]),
                                pack2(TT{}, pw[4], pw[5]), pack2(TT{}, pw[6], pw[7]));
    l_lane = psum2(TT{}, pb.w, psum2(TT{}, pb.z, psum2(TT{}, pb.y, psum2(TT{}, pb.x, l_lane))));
    uint4 v[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) v[mt] = *reinterpret_cast<const uint4*>(vr + mt * 16 * 16);
    if (vtail && tok + kKeys > last) {  // zero V of positions past `last` in this group
      const int keep = min(max(last + 1 - tok - kb * VS, 0), VS);
      uint32_t m4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        m4[i] = ((2 * i < keep) ? 0xffffu : 0u) | ((2 * i + 1 < keep) ? 0xffff0000u : 0u);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        v[mt].x &= m4[0];
        v[mt].y &= m4[1];
        v[mt].z &= m4[2];
        v[mt].w &= m4[3];
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma(TT{}, v[mt], pb, acc[mt]);
  };

  // 32 rows per wavefront.  Row rho of the S^T A operand is key
  // 16 (rho / 16) + 8 ((rho / 4) % 2) + 4 ((rho / 8) % 2) + rho % 4, so C
  // register r of lane (c32, hh) holds query c32's score of key
  // 8 hh + r + 8 [r >= 8]: registers 0-7 are the P^T slice of keys 0-15,
  // 8-15 that of keys 16-31, with no lane exchange.
  auto compute32 = [&](int grp, const char* buf) {
    const int tok = grp * kKeys;
    const int krow = 16 * (c32 >> 4) + 8 * ((c32 >> 2) & 1) + 4 * ((c32 >> 3) & 1) + (c32 & 3);
    float16_t st;
#pragma unroll
    for (int r = 0; r < 16; ++r) st[r] = 0.f;
    // K operand of k-step s2: piece 2 s2 + hh of key krow
    const char* kr = DMA ? buf + (hh * kKeys + c32) * 16 : buf + krow * KP + hh * 16;
    constexpr int KSTEP = DMA ? 2 * kKeys * 16 : 32;
#pragma unroll
    for (int s2 = 0; s2 < D / 16; ++s2)
      st = mfma32(TT{}, *reinterpret_cast<const uint4*>(kr + KSTEP * s2), qr[s2], st);
    float sc[16];  // raw dot products; the score is sc * scl
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = st[r];
    if (tok + kKeys - 1 > pos0) {  // the group reaches past the tile's first row
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (tok + 8 * hh + r + (r >= 8 ? 8 : 0) > mypos) sc[r] = -INFINITY;
    }
    float mx = sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[r]);
    mx = xor32_max(mx) * scl;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kSlack) != 0) {
      const float m_new = mx > m_run + kSlack ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_lane *= alpha;
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) acc32[mt] *= alpha;
      m_run = m_new;
    }
    float pw[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) pw[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], scl, -m_run));
    if (tok + kKeys - 1 > pos0) {  // masked keys weigh 0 also at scale 0 (-inf * 0 is NaN)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (tok + 8 * hh + r + (r >= 8 ? 8 : 0) > mypos) pw[r] = 0.f;
    }
    uint4 pb[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
      pb[kh] = make_uint4(pack2(TT{}, pw[8 * kh], pw[8 * kh + 1]),
                          pack2(TT{}, pw[8 * kh + 2], pw[8 * kh + 3]),
                          pack2(TT{}, pw[8 * kh + 4], pw[8 * kh + 5]),
                          pack2(TT{}, pw[8 * kh + 6], pw[8 * kh + 7]));
    // the row sum takes the same rounded weights the matrix op does
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
      l_lane = psum2(TT{}, pb[kh].w,
                     psum2(TT{}, pb[kh].z, psum2(TT{}, pb[kh].y, psum2(TT{}, pb[kh].x, l_lane))));
    // V^T operand of key half kh: slab 2 kh + hh, row d = 32 mt + c32
    const bool vmask = vtail && tok + kKeys > last;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const char* vr = DMA ? buf + KBUFD + (2 * kh + hh) * (D * 16) + c32 * 16
                           : buf + KBUF + (2 * kh + hh) * VSP + c32 * 16;
      uint4 v[D / 32];
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) v[mt] = *reinterpret_cast<const uint4*>(vr + mt * 32 * 16);
      // Only the operands depend on the branch, so the accumulators stay in
      // place (MFMAs on both sides of a branch made the compiler copy all of
      // them at the join).
      if (vmask) {  // zero V of positions past `last` in this group
        const int keep = min(max(last + 1 - tok - VS * (2 * kh + hh), 0), VS);
        uint32_t m4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          m4[i] = ((2 * i < keep) ? 0xffffu : 0u) | ((2 * i + 1 < keep) ? 0xffff0000u : 0u);
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) {
          v[mt].x &= m4[0];
          v[mt].y &= m4[1];
          v[mt].z &= m4[2];
          v[mt].w &= m4[3];
        }
      }
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) acc32[mt] = mfma32(TT{}, v[mt], pb[kh], acc32[mt]);
    }
  };

  if constexpr (DMA) {
    // group g in LDS buffer g % 2: its loads were issued during group g - 1;
    // this wavefront waits for its own, the barrier for everyone's (and for
    // every wavefront to be done with group g - 1, whose buffer the loads of
    // group g + 1 then overwrite)
    auto run = [&](auto tab) {
      auto step = [&](int grp, char* cur, char* nxt) {
        __builtin_amdgcn_s_waitcnt(kVmcntZero);
        __syncthreads();
        if (grp + 1 < ngroups) dma(grp + 1, nxt, tab);
        if (nrows > 0 && grp * kKeys <= last) compute32(grp, cur);
      };
      dma(0, lds, tab);
      for (int grp = 0; grp < ngroups; grp += 2) {
        step(grp, lds, lds_b);
        if (grp + 1 >= ngroups) break;
        step(grp + 1, lds_b, lds);
      }
    };
    // every block id a group can touch -- up to last_wg / bs, and up to
    // NBG - 1 past it in the last group (block 0 there, as in the window)
    // (not with four blocks per key group: the second loop took the 32-row
    // kernel past three wavefronts' registers per SIMD)
    const int need = last_wg / bs + 1;
    if constexpr (NBG <= 2) {
      if (need + NBG <= kTabBlocks) {  // the same for the whole workgroup
        for (int j = tid; j < need + NBG; j += kThreads) {
          const int e = (j < need && j < a.max_blocks_per_seq) ? trow[j] : 0;
          s_tab[j] = (e < 0 || (int64_t)e >= a.num_blocks) ? 0 : e;
        }
        __syncthreads();
        run(std::true_type{});
      } else {
        run(std::false_type{});
      }
    } else {
      run(std::false_type{});
    }
  } else {
  // Group g's K/V travel HBM -> registers two groups ahead of their use
  // (register sets A and B alternate), then registers -> LDS buffer g % 2
  // just before the group's barrier.  Buffer g % 2 was last read by group
  // g - 2, which every wavefront finished before the barrier of group g - 1.
  auto step = [&](int grp, uint4 (&pk)[NCK], uint4 (&pv)[NCV]) {
    char* buf = lds + (grp & 1) * BUF;
    store(buf, pk, pv);
    if (grp + 2 < ngroups) load(grp + 2, pk, pv);
    __syncthreads();
    // wavefronts without rows, or whose rows all end before this group,
    // only help with the loads
    if (nrows > 0 && grp * kKeys <= last) {
      if constexpr (WR == 16) compute(grp, buf); else compute32(grp, buf);
    }
  };
  uint4 pkA[NCK], pvA[NCV], pkB[NCK], pvB[NCV];
  load(0, pkA, pvA);
  if (ngroups > 1) load(1, pkB, pvB);
  for (int grp = 0; grp < ngroups; grp += 2) {
    step(grp, pkA, pvA);
    if (grp + 1 >= ngroups) break;
    step(grp + 1, pkB, pvB);
  }
  }

  if constexpr (WR == 16) {
    float l_tot = l_lane + __shfl_xor(l_lane, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (n < nrows) {
      const float inv = 1.f / l_tot;
      uint16_t* out = reinterpret_cast<uint16_t*>(a.out) +
                      (((int64_t)qs + r0 + n) * a.num_q_heads + h) * D + 4 * kb;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) out[mt * 16 + e] = to_bits(TT{}, acc[mt][e] * inv);
    }
  } else {
    const float l_tot = xor32_add(l_lane);
    if (c32 < nrows) {
      const float inv = 1.f / l_tot;
      uint16_t* out = reinterpret_cast<uint16_t*>(a.out) +
                      (((int64_t)qs + r0 + c32) * a.num_q_heads + h) * D + 4 * hh;
      // register r holds dim 32 mt + 8 (r / 4) + 4 hh + r % 4
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint2 w;
          w.x = pack2(TT{}, acc32[mt][4 * q] * inv, acc32[mt][4 * q + 1] * inv);
          w.y = pack2(TT{}, acc32[mt][4 * q + 2] * inv, acc32[mt][4 * q + 3] * inv);
          *reinterpret_cast<uint2*>(out + 32 * mt + 8 * q) = w;
        }
    }
  }
}

template <typename TT, int D, int NBG, int WR, int WV, bool DMA = false>
hipError_t launch_w(const PrefillArgs& a, hipStream_t s) {
  const int64_t tpg = (a.max_query_len + WV * WR - 1) / (WV * WR);
  const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads;
  const int64_t wgs = (units + 7) / 8 * 8 * (a.num_q_heads / a.num_kv_heads) * tpg;
  if (wgs > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid((unsigned)wgs);
  hipLaunchKernelGGL((prefill_mfma_kernel<TT, D, NBG, WR, WV, DMA>), grid, dim3(64 * WV), 0, s, a);
  return hipGetLastError();
}

// Shape of the workgroup (launch_g): rows per wavefront, wavefronts per
// workgroup and how K/V reach LDS, from the longest chunk and the context
// bound; PA_PREFILL_ROWS / _WAVES / _DMA override them (tests, tuning).
template <typename TT, int D, int NBG>
hipError_t launch_g(const PrefillArgs& a, hipStream_t s) {
  // 32-row wavefronts from 64-row chunks on, four of them per workgroup
  // from 128 rows on: each key group's LDS fill then serves twice the rows
  // (with the direct loads this pays on long contexts, 256-row chunks of
  // 600-8000 tokens, and on the ragged 1-512-row chunks of 513-1024-token
  // prompts alike: 1.87 against 1.92 ms and 2.87 against 3.12 ms there).
  int wr = a.max_query_len >= kPrefill32MinRows ? 32 : 16;
  int wv = wr == 16 || a.max_query_len >= 4 * 32 ? 4 : 2;
  if (const char* e = std::getenv("PA_PREFILL_ROWS")) wr = atoi(e) == 32 ? 32 : atoi(e) == 16 ? 16 : wr;
  if (const char* e = std::getenv("PA_PREFILL_WAVES")) wv = atoi(e) == 2 ? 2 : 4;
  if (wr == 32) {
    // Direct global -> LDS loads (0.71-0.73 against 0.65-0.67 PFLOP/s on
    // the 66B chunk writers; 3-4% faster on the short contexts of the
    // prefix-sharing prompts, two wavefronts).  PA_PREFILL_DMA = 0 selects
    // the register-staged loads.
    bool dma = true;
    if (const char* e = std::getenv("PA_PREFILL_DMA")) dma = atoi(e) != 0;
    if (dma)
      return wv == 2 ? launch_w<TT, D, NBG, 32, 2, true>(a, s)
                     : launch_w<TT, D, NBG, 32, 4, true>(a, s);
    return wv == 2 ? launch_w<TT, D, NBG, 32, 2>(a, s) : launch_w<TT, D, NBG, 32, 4>(a, s);
  }
  return wv == 2 ? launch_w<TT, D, NBG, 16, 2>(a, s) : launch_w<TT, D, NBG, 16, 4>(a, s);
}

template <typename TT, int D>
hipError_t launch_d(const PrefillArgs& a, hipStream_t s) {
  if (a.block_size == 8) return launch_g<TT, D, 4>(a, s);
  if (a.block_size == 16) return launch_g<TT, D, 2>(a, s);
  return launch_g<TT, D, 1>(a, s);
}

}  // namespace

bool prefill_supported(pa_dtype dt, int head_dim, int block_size) {
  const bool dt_ok = dt == PA_F16 || dt == PA_BF16;
  const bool d_ok = head_dim == 64 || head_dim == 128;
  const bool bs_ok = block_size == 8 || block_size == 16 || (block_size % 32 == 0);
  return dt_ok && d_ok && bs_ok;
}

hipError_t launch_prefill(const PrefillArgs& a, pa_dtype dt, hipStream_t s) {
  if (a.num_seqs == 0 || a.max_query_len == 0) return hipSuccess;
  if (dt == PA_F16) return a.head_dim == 64 ? launch_d<F16, 64>(a, s) : launch_d<F16, 128>(a, s);
  if (dt == PA_BF16)
    return a.head_dim == 64 ? launch_d<BF16, 64>(a, s) : launch_d<BF16, 128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace pa
