// Token-balanced work split shared by the decode kernels and their merge.
//
// Work items are (sequence b, head h) pairs, h < H (q heads for the MHA
// kernel, kv heads for the GQA kernel), ordered b-major.  Item (b, h) has
// n_b = ceil(L_b / STEP) steps of STEP tokens.  Laid end to end the items form
// one stream of N = sum_b H * n_b steps; worker w (one wavefront) takes steps
// [start(w), start(w+1)): either W equal shares (start(w) = w*N/W, so shares
// differ by at most one step) or fixed chunks of C steps.  Every worker
// therefore streams the same number of K/V bytes regardless of how lengths
// are distributed, and it prefetches straight across item boundaries.
//
// A worker that sees all of an item's steps writes the final output row;
// otherwise it writes its partial (m, l, o) to slot item + w.  That slot is
// unique: along the stream every new (item, worker) segment increases the
// item index, the worker index or both.  Item i starting at stream step S_i
// is shared by the workers F = worker_of(S_i) .. Lw = worker_of(S_i + n - 1);
// worker F records (F, Lw - F + 1) for the merge kernel, which combines the
// slots.
#pragma once

#include "pa_internal.h"

namespace pa {

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

// Exclusive prefix over sequences of H * n_b (LDS s_pre[0..B]) and the
// clamped lengths (LDS s_len[0..B-1]), computed by ONE wavefront: lane i
// handles a contiguous run of sequences, then a shuffle scan across lanes.
// The caller publishes the arrays to the other wavefronts with a barrier.
// Returns N = s_pre[B] (in every lane).
__device__ inline int wave_scan_steps(const int32_t* lens, int B, int H, int cap, int step,
                                      int* s_pre, int* s_len) {
  const int lane = threadIdx.x & 63;
  const int per = (B + 63) / 64;
  const int j0 = min(lane * per, B), j1 = min(j0 + per, B);
  int local = 0;
  for (int j = j0; j < j1; ++j) {
    const int L = clamp_len(lens[j], cap);
    s_len[j] = L;
    local += H * ((L + step - 1) / step);
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
    run += H * ((s_len[j] + step - 1) / step);
  }
  if (lane == 63) s_pre[B] = incl;
  return __shfl(incl, 63);
}

// Balanced shares are at least kMinChunk steps, so that a worker's start-up
// is amortised and an item never has more than n / kMinChunk + 2 partials.
constexpr int kMinChunk = 8;

struct Split {
  int64_t N;  // steps in the stream (> 0)
  int W;      // workers that take steps
  int C;      // fixed steps per worker, 0 = W equal shares
  // First step of worker w's share (for w == W: N with equal shares, possibly
  // past N with fixed chunks -- callers clamp).
  __device__ __forceinline__ int64_t start(int w) const {
    return C ? (int64_t)w * C : (int64_t)w * N / W;
  }
  // The worker whose share holds stream step x: the largest w with start(w) <= x.
  __device__ __forceinline__ int worker_of(int64_t x) const {
    return C ? (int)(x / C) : (int)(((x + 1) * W - 1) / N);
  }
};

__device__ __forceinline__ Split make_split(const DecodeArgs& a, int N) {
  Split s;
  s.N = N;
  if (a.chunk_steps > 0) {
    s.C = a.chunk_steps;
    s.W = (N + s.C - 1) / s.C;
  } else {
    s.C = 0;
    const int cap = N / kMinChunk;
    s.W = a.num_workers < cap ? a.num_workers : (cap > 0 ? cap : 1);
  }
  return s;
}

// Position in the step stream: sequence b, head h, step k of n, length L.
struct Cursor {
  int b, h, k, n, L;
  __device__ __forceinline__ int item(int H) const { return b * H + h; }
};

// Cursor of stream step x (flat mode): the sequence with s_pre[b] <= x < s_pre[b+1].
__device__ __forceinline__ Cursor locate(const int* s_pre, const int* s_len, int B, int H,
                                         int step, int x) {
  int lo = 0, hi = B;  // first index with s_pre[idx] > x, searched in [0, B]
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (s_pre[mid] > x) hi = mid; else lo = mid + 1;
  }
  Cursor c;
  c.b = lo - 1;
  c.L = s_len[c.b];
  c.n = (c.L + step - 1) / step;
  const int r = x - s_pre[c.b];
  c.h = r / c.n;
  c.k = r - c.h * c.n;
  return c;
}

// Next step of the stream (flat mode: skips empty sequences).
__device__ __forceinline__ void advance(Cursor& c, const int* s_pre, const int* s_len, int H,
                                        int step) {
  if (++c.k < c.n) return;
  c.k = 0;
  if (++c.h < H) return;
  c.h = 0;
  do {
    ++c.b;
  } while (s_pre[c.b + 1] == s_pre[c.b]);
  c.L = s_len[c.b];
  c.n = (c.L + step - 1) / step;
}

}  // namespace pa
