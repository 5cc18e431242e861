// Token-balanced work split shared by the decode kernels and their merge.
//
// Work items are (sequence b, head h) pairs, h < H (q heads for the MHA
// kernel, kv heads for the GQA kernel), ordered b-major.  Item (b, h) has
// n_b = ceil(L_b / STEP) steps of STEP tokens.  Laid end to end the items form
// one stream of N = sum_b H * n_b steps; worker w (one wavefront) takes the
// steps [w*N/W, (w+1)*N/W), so shares differ by at most one step and every
// worker streams the same number of K/V bytes whatever the lengths.  A worker
// prefetches straight across item boundaries.
//
// Partitions.  When a partition size P = C * STEP is given, item steps
// [p*C, (p+1)*C) form partition p of the item, and the shares are made of
// whole partitions: worker w takes partitions [w*Pn/W, (w+1)*Pn/W) of the Pn
// partitions laid end to end, so no partition is divided between wavefronts.
// Shares then differ by at most one partition.
//
// Segments.  A worker's steps of one item form a segment.  A segment that is
// a whole item is written as the final output row.  Otherwise it becomes an
// fp32 partial (m, l, o) of the item: running max in the base-2 domain, sum
// of 2^(s - m), unnormalised output; the merge kernel (decode_merge.hip)
// combines an item's partials.  A worker owning several consecutive
// partitions of an item folds them into one partial in registers (the online
// softmax is exact over any number of keys).
//
// Slots.  The partial of the segment of item i by worker w goes to slot i + w.
// Along the stream every new segment increases the item, the worker or both,
// so slots are unique; the merge recomputes from the same arithmetic which
// workers an item has.
#pragma once

#include "pa_internal.h"

namespace pa {

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

// s_waitcnt operand: vmcnt 0, expcnt and lgkmcnt left at their maxima (gfx9
// encoding).
constexpr int kVmcntZero = 0x0F70;

// Dynamic LDS a decode launch with these arguments needs (the prefix pass of
// a shared-prefix decode sizes its own: its sequences are the groups).
inline size_t decode_split_lds(const DecodeArgs& a) {
  if (!a.split) return 0;
  return a.num_groups > 0 ? cascade_lds_bytes(a.num_seqs, a.num_groups)
                          : split_lds_bytes(a.num_seqs);
}

// Exclusive prefixes over sequences of H * n_b (LDS s_pre[0..B]) and, when
// C > 0, of H * ceil(n_b / C) (s_ppre[0..B]), plus the clamped lengths less
// `drop` trailing positions (s_len[0..B-1]; drop = 1 leaves out the new token
// that the merge folds in), computed by ONE wavefront: lane i handles a
// contiguous run of sequences, then a shuffle scan across lanes.  The caller
// publishes the arrays to the other wavefronts with a barrier.  Returns
// N = s_pre[B] (in every lane).
__device__ inline int wave_scan_steps(const int32_t* lens, int B, int H, int cap, int drop,
                                      int step, int C, int* s_pre, int* s_len, int* s_ppre) {
  const int lane = threadIdx.x & 63;
  const int per = (B + 63) / 64;
  const int j0 = min(lane * per, B), j1 = min(j0 + per, B);
  int local = 0, plocal = 0;
  for (int j = j0; j < j1; ++j) {
    const int L = max(clamp_len(lens[j], cap) - drop, 0);
    s_len[j] = L;
    const int n = (L + step - 1) / step;
    local += H * n;
    if (C > 0) plocal += H * ((n + C - 1) / C);
  }
  int incl = local, pincl = plocal;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    const int py = __shfl_up(pincl, off);
    if (lane >= off) {
      incl += y;
      pincl += py;
    }
  }
  int run = incl - local, prun = pincl - plocal;
  for (int j = j0; j < j1; ++j) {
    const int n = (s_len[j] + step - 1) / step;
    s_pre[j] = run;
    run += H * n;
    if (C > 0) {
      s_ppre[j] = prun;
      prun += H * ((n + C - 1) / C);
    }
  }
  if (lane == 63) {
    s_pre[B] = incl;
    if (C > 0) s_ppre[B] = pincl;
  }
  return __shfl(incl, 63);
}

// Balanced shares are at least kMinChunk steps, so that a worker's start-up
// is amortised.
constexpr int kMinChunk = 8;

// Largest b in [0, B-1] with a[b] <= v, for non-decreasing a[0..B].
__device__ __forceinline__ int last_le(const int* a, int B, int64_t v) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a[mid] <= v) lo = mid; else hi = mid - 1;
  }
  return lo;
}

struct Split {
  int64_t N;  // steps in the stream (> 0)
  int W;      // workers that take steps
  // partition-granular shares (C > 0): Pn partitions; pre / ppre are the step
  // and partition prefixes per sequence, B sequences, H items per sequence
  int C, Pn, H, B;
  const int* pre;
  const int* ppre;

  // first stream step of partition g (g < Pn)
  __device__ __forceinline__ int64_t partition_start(int64_t g) const {
    const int b = last_le(ppre, B, g);
    const int n = (pre[b + 1] - pre[b]) / H, np = (n + C - 1) / C;
    const int r = (int)(g - ppre[b]);
    return pre[b] + (int64_t)(r / np) * n + (int64_t)(r % np) * C;
  }
  // partition holding stream step x
  __device__ __forceinline__ int64_t partition_of(int64_t x) const {
    const int b = last_le(pre, B, x);
    const int n = (pre[b + 1] - pre[b]) / H, np = (n + C - 1) / C;
    const int r = (int)(x - pre[b]);
    return ppre[b] + (int64_t)(r / n) * np + (r % n) / C;
  }
  // First step of worker w's share (start(W) == N).
  __device__ __forceinline__ int64_t start(int w) const {
    if (C == 0) return (int64_t)w * N / W;
    const int64_t g = (int64_t)w * Pn / W;
    return g >= Pn ? N : partition_start(g);
  }
  // The worker whose share holds stream step x: the largest w with start(w) <= x.
  __device__ __forceinline__ int worker_of(int64_t x) const {
    if (C == 0) return (int)(((x + 1) * W - 1) / N);
    return (int)(((partition_of(x) + 1) * W - 1) / Pn);
  }
};

// The split of N stream steps over at most num_workers workers; with C > 0,
// in whole partitions (pre / ppre as exported by the decode kernels).
__device__ __forceinline__ Split make_split(int num_workers, int N, int C = 0, int H = 1,
                                            int B = 0, const int* pre = nullptr,
                                            const int* ppre = nullptr) {
  Split s;
  s.N = N;
  s.C = C;
  s.H = H;
  s.B = B;
  s.pre = pre;
  s.ppre = ppre;
  s.Pn = C > 0 ? ppre[B] : 0;
  int cap = N / kMinChunk;
  if (C > 0 && s.Pn < cap) cap = s.Pn;  // every worker gets at least one partition
  s.W = num_workers < cap ? num_workers : (cap > 0 ? cap : 1);
  return s;
}

// Position in the step stream: sequence b, head h, step k of n, length L;
// the item's steps cover positions s .. L-1 (s > 0 only for the tail pass of
// a shared-prefix decode, where positions below s are the group's prefix),
// step k starting at position s + k * STEP.
struct Cursor {
  int b, h, k, n, L, s;
  __device__ __forceinline__ int item(int H) const { return b * H + h; }
  __device__ __forceinline__ int tok(int step) const { return s + k * step; }
};

// Cursor of stream step x: the sequence with s_pre[b] <= x < s_pre[b+1].
// s_st: the first position of each sequence's steps (null: 0).
__device__ __forceinline__ Cursor locate(const int* s_pre, const int* s_len, const int* s_st,
                                         int B, int H, int step, int x) {
  int lo = 0, hi = B;  // first index with s_pre[idx] > x, searched in [0, B]
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (s_pre[mid] > x) hi = mid; else lo = mid + 1;
  }
  Cursor c;
  c.b = lo - 1;
  c.L = s_len[c.b];
  c.s = s_st ? s_st[c.b] : 0;
  c.n = (c.L - c.s + step - 1) / step;
  const int r = x - s_pre[c.b];
  c.h = r / c.n;
  c.k = r - c.h * c.n;
  return c;
}

// Next step of the stream (skips empty sequences).
__device__ __forceinline__ void advance(Cursor& c, const int* s_pre, const int* s_len,
                                        const int* s_st, int H, int step) {
  if (++c.k < c.n) return;
  c.k = 0;
  if (++c.h < H) return;
  c.h = 0;
  do {
    ++c.b;
  } while (s_pre[c.b + 1] == s_pre[c.b]);
  c.L = s_len[c.b];
  c.s = s_st ? s_st[c.b] : 0;
  c.n = (c.L - c.s + step - 1) / step;
}

// ----------------------------------------------------------- shared prefix --
// pa_decode_shared: groups of consecutive sequences, group g = sequences
// gs[g] .. gs[g+1]-1, whose first gp[g] positions (whole blocks) are the same
// physical blocks in every member's table.  The prefix pass reads those
// blocks once per (group, kv head) for all the members' q rows; the tail pass
// streams each sequence from its group's prefix length on; the merge joins
// the two partials of every row.

// The prefix length a group's passes use: a whole number of blocks, no more
// than its first member's length (the caller guarantees every member's; the
// kernels only keep every access inside the tables).
__device__ __forceinline__ int group_prefix(const DecodeArgs& a, int g, int L_first) {
  const int P = clamp_len(a.group_prefix[g], L_first);
  return P - P % a.block_size;
}

// Group starts s_gs[0..G] (clamped to [0, B]) and prefix lengths s_gp[0..G-1]
// into LDS, by one wavefront (the caller publishes them with a barrier).
__device__ inline void load_groups(const DecodeArgs& a, int* s_gs, int* s_gp) {
  const int G = a.num_groups, B = a.num_seqs;
  for (int i = threadIdx.x & 63; i <= G; i += 64) {
    const int s0 = min(max(a.group_start[i], 0), B);
    s_gs[i] = s0;
    if (i < G) s_gp[i] = group_prefix(a, i, clamp_len(a.context_lens[min(s0, B - 1)], a.len_cap));
  }
}

// Tail pass scan: as wave_scan_steps (no partitions, no dropped position),
// with each sequence's first position s_st[b] = its group's prefix length
// and its group s_grp[b].  s_gs / s_gp as load_groups left them.
__device__ inline int wave_scan_tail(const DecodeArgs& a, const int* s_gs, const int* s_gp, int H,
                                     int step, int* s_pre, int* s_len, int* s_st, int* s_grp) {
  const int B = a.num_seqs, G = a.num_groups;
  const int lane = threadIdx.x & 63;
  const int per = (B + 63) / 64;
  const int j0 = min(lane * per, B), j1 = min(j0 + per, B);
  int g = 0, hi = G;  // last group with s_gs[g] <= j0
  while (g < hi) {
    const int mid = (g + hi + 1) >> 1;
    if (mid < G && s_gs[mid] <= j0) g = mid; else hi = mid - 1;
  }
  int local = 0;
  for (int j = j0; j < j1; ++j) {
    while (g + 1 < G && s_gs[g + 1] <= j) ++g;
    const int L = clamp_len(a.context_lens[j], a.len_cap);
    const int st = min(s_gp[g], L);
    s_len[j] = L;
    s_st[j] = st;
    s_grp[j] = g;
    local += H * ((L - st + step - 1) / step);
  }
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  int run = incl - local;
  for (int j = j0; j < j1; ++j) {
    s_pre[j] = run;
    run += H * ((s_len[j] - s_st[j] + step - 1) / step);
  }
  if (lane == 63) s_pre[B] = incl;
  return __shfl(incl, 63);
}

// The step ends a segment of a worker whose last stream step has index
// `last_j` within its share (j = index of this step within the share).
__device__ __forceinline__ bool segment_ends(const Cursor& c, int j, int last_j) {
  return j == last_j || c.k == c.n - 1;
}
__device__ __forceinline__ bool segment_starts(const Cursor& c, int j) {
  return j == 0 || c.k == 0;
}

// For the cascade merge, per sequence j four ints at ws_grp + 4 j: its group
// g, the group's first member, and the group's range [pws_pre[g],
// pws_pre[g + 1]) of prefix-pass steps (exported by the prefix pass, which
// runs before the tail pass).  One wavefront; s_grp / s_gs as the tail scan
// and load_groups left them.
__device__ inline void export_groups(const DecodeArgs& a, const int* s_grp, const int* s_gs,
                                     int B) {
  for (int j = threadIdx.x & 63; j < B; j += 64) {
    const int g = s_grp[j];
    *reinterpret_cast<int4*>(a.ws_grp + 4 * j) =
        make_int4(g, min(s_gs[g], B - 1), a.pws_pre[g], a.pws_pre[g + 1]);
  }
}

// Copies the scan's prefixes to global memory for the merge kernel:
// pre[0..B] = s_pre, ppre[0..B] = s_ppre (C > 0).  Called by one wavefront
// after the barrier that published them.
__device__ inline void export_prefixes(const int* s_pre, const int* s_ppre, int B, int C,
                                       int* pre, int* ppre) {
  for (int j = threadIdx.x & 63; j <= B; j += 64) {
    pre[j] = s_pre[j];
    if (C > 0) ppre[j] = s_ppre[j];
  }
}

}  // namespace pa
