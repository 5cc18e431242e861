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
//
// For pa_decode_write it is also where the step's new token enters: the
// decode kernel leaves the token out and writes partials only, and the merge
// adds the token's own term and stores the token into its slot (the write
// that precedes attention in wq-win.github.io "079 | vLLM 与 PagedAttention",
// section 三; no kernel reads that slot before the merge runs).
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

// Four consecutive outputs from index idx (a multiple of 4) in one store.
template <typename TT>
__device__ __forceinline__ void store_out4(void* out, int64_t idx, float4 x) {
  if constexpr (TT::bytes == 4) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + idx) = x;
  } else {
    const uint2 w = make_uint2(to_bits(TT{}, x.x) | ((uint32_t)to_bits(TT{}, x.y) << 16),
                               to_bits(TT{}, x.z) | ((uint32_t)to_bits(TT{}, x.w) << 16));
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + idx) = w;
  }
}

// Partials folded per memory round trip: each thread loads (m, l, o) of up to
// NB pieces back to back, then folds them in with one rescale.  Items of a
// few pieces (the common case: an item split once or twice) take the short
// batch, so no thread issues loads for pieces that do not exist.
// The long batch holds 8 pieces: with four outputs a thread, 16 pieces'
// 16-byte o loads took 128 VGPRs and spilled.
constexpr int kBatchShort = 4;
constexpr int kBatch = 8;

template <typename TT>
__device__ __forceinline__ float elem(const void* base, int64_t i) {
  if constexpr (TT::bytes == 4)
    return reinterpret_cast<const float*>(base)[i];
  else
    return lo_to_float(TT{}, reinterpret_cast<const uint16_t*>(base)[i]);
}

// pa_decode_write: where sequence b's new token goes -- element d of kv head
// g at position L - 1 -- as element indices into the K and V pools; -1 when
// the table entry is not a block of the pool (nothing is stored then).
struct NewSlot {
  int64_t k, v;
};
__device__ __forceinline__ NewSlot new_slot(const DecodeArgs& a, int32_t blk, int g, int L,
                                            int d, int elem_bytes) {
  const int D = a.head_dim, bs = a.block_size, pos = L - 1;
  if (blk < 0 || (int64_t)blk >= a.num_blocks) return {-1, -1};
  const int off = pos % bs, vs = v_slab(bs);
  const int64_t hkv = a.num_kv_heads;
  return {k_elem_index(blk, g, off, d, hkv, bs, D, elem_bytes),
          ((((int64_t)blk * hkv + g) * (bs / vs) + off / vs) * D + d) * vs + off % vs};
}

// Running (max, sum, outputs) of four consecutive output elements of one
// row while pieces are folded in.
struct MergeState4 {
  float M, Lt;
  float4 acc;
};
// Folds pieces into st in batches of NB, each batch's m, l and o loaded in
// one memory round trip: pieces k < K from records of RR rows at sa(k) of
// pa (row r), then K <= k < K + Kp from the prefix pass's records of
// kPrefixRows rows at sb(k - K) of pb (row rp); the thread's elements are
// dims d0 .. d0 + 3 (one 16-byte load of o per piece).
template <int NB, typename SlotA, typename SlotB>
__device__ __forceinline__ void fold_two(MergeState4& st, const float* pa, SlotA sa, int K, int RR,
                                         int r, const float* pb, SlotB sb, int Kp, int rp, int d0,
                                         int D) {
  // o of (row, d) sits at q4 * rows + 4 row + d % 4 in a record of `rows` rows
  const int q4 = ((d0 >> 4) * 4 + ((d0 & 15) >> 2)) * 4;
  const int RSa = part_record(RR, D), RSb = part_record(kPrefixRows, D);
  const int T = K + Kp;
  for (int k0 = 0; k0 < T; k0 += NB) {
    float m[NB], l[NB];
    float4 o[NB];
#pragma unroll
    for (int w = 0; w < NB; ++w) {
      const bool ok = k0 + w < T;
      const int k = ok ? k0 + w : T - 1;
      const bool ta = k < K;
      const float* rec = ta ? pa + (int64_t)sa(k) * RSa : pb + (int64_t)sb(k - K) * RSb;
      const int rows = ta ? RR : kPrefixRows, row = ta ? r : rp;
      m[w] = ok ? rec[rows * D + row] : -INFINITY;
      l[w] = ok ? rec[rows * D + 16 + row] : 0.f;
      o[w] = *reinterpret_cast<const float4*>(rec + q4 * rows + row * 4);
    }
    float Mn = st.M;
#pragma unroll
    for (int w = 0; w < NB; ++w) Mn = fmaxf(Mn, m[w]);
    const float sc = st.M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.M - Mn);
    st.Lt *= sc;
    st.acc.x *= sc;
    st.acc.y *= sc;
    st.acc.z *= sc;
    st.acc.w *= sc;
#pragma unroll
    for (int w = 0; w < NB; ++w) {
      // a piece past the end has m = -inf: weight 0, its (valid) o ignored
      const float f = m[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[w] - Mn);
      st.Lt += f * l[w];
      st.acc.x += f * o[w].x;
      st.acc.y += f * o[w].y;
      st.acc.z += f * o[w].z;
      st.acc.w += f * o[w].w;
    }
    st.M = Mn;
  }
}

// A group of threads per item (b, h), one thread per four consecutive
// outputs (q row r, dims d0 .. d0 + 3).
// FOLD (pa_decode_write): the decode kernel covered positions 0 .. L-2 and
// the new token at L - 1 enters here, one of two ways.  With a.fold_in_merge
// (the grouped-query kernel) every segment left a partial and the merge adds
// the token's own term -- score s = scale q . k_new, weight 2^(s - s) = 1,
// value v_new; otherwise the decode kernel already added it, and only
// sequences with no earlier position (L = 1: the row is v_new) need a row
// here.  In both, the item that owns the kv head's first q row stores the
// token into its slot.
// Several items share a workgroup (ipw of them, `per` threads each), except
// when the merge adds the new token's term (it synchronises the workgroup).
template <typename TT, bool FOLD>
__global__ __launch_bounds__(1024) void decode_merge_kernel(DecodeArgs a, int H, int R, int ipw) {
  using E = typename TT::raw;
  const int D = a.head_dim, B = a.num_seqs;
  const int per = blockDim.x / ipw;  // threads per item
  const int item = blockIdx.x * ipw + threadIdx.x / per;
  const int tid = threadIdx.x - (threadIdx.x / per) * per;
  if (item >= B * H) return;
  const int b = item / H, h = item - b * H;
  const int* pre = a.ws_pre;
  const int64_t orow0 = ((int64_t)b * a.num_q_heads + (int64_t)h * R) * D;
  const int total = R * D / 4;  // groups of four outputs
  // items are q heads (R = 1) or the G q heads of a kv head (R = G)
  const int G = a.num_q_heads / a.num_kv_heads;
  const int g = R == 1 ? h / G : h;
  const int64_t nrow = (int64_t)b * a.new_stride + (int64_t)g * D;
  // first round of loads, all independent: lengths and prefixes, and (FOLD)
  // the thread's element d = tid of the new token's rows (FOLD launches at
  // least D threads per item, so the token's loads and stores run along the
  // rows, one element a thread)
  const int n = (pre[b + 1] - pre[b]) / H;
  const int L = FOLD ? clamp_len(a.context_lens[b], a.len_cap) : 0;
  E kx = 0, vx = 0;
  const int td = tid < D ? tid : 0;
  if constexpr (FOLD) {
    kx = reinterpret_cast<const E*>(a.k_new)[nrow + td];
    vx = reinterpret_cast<const E*>(a.v_new)[nrow + td];
  }
  if (FOLD ? L == 0 : n == 0) {  // empty sequence: zero rows
    for (int t = tid; t < R * D; t += per) store_out<TT>(a.out, orow0 + t, 0.f);
    return;
  }
  // second round: the new token's block, and the partials (below)
  const bool stores = FOLD && (R > 1 || h % G == 0) && tid < D;
  const int32_t blk =
      stores ? a.block_tables[(int64_t)b * a.max_blocks_per_seq + (L - 1) / a.block_size] : -1;
  auto store_token = [&]() {
    if (!stores) return;
    // non-temporal: these scattered pieces of lines are not read again here
    // (measured: the step's token stores 6 us cheaper than plain stores)
    const NewSlot ns = new_slot(a, blk, g, L, tid, TT::bytes);
    if (ns.k < 0) return;
    __builtin_nontemporal_store(kx, reinterpret_cast<E*>(const_cast<void*>(a.k_cache)) + ns.k);
    __builtin_nontemporal_store(vx, reinterpret_cast<E*>(const_cast<void*>(a.v_cache)) + ns.v);
  };
  int F = 0, K = 0;  // the decode kernel's pieces: workers F .. F + K - 1
  if (n > 0) {
    const Split sp = make_split(a.num_workers, pre[B], a.part_steps, H, B, pre, a.ws_ppre);
    const int64_t S = pre[b] + (int64_t)h * n, E2 = S + n;
    F = sp.worker_of(S);
    const int Lw = sp.worker_of(E2 - 1);
    if ((!FOLD || !a.fold_in_merge) && F == Lw) {  // one piece: the decode kernel wrote the row
      store_token();
      return;
    }
    K = Lw - F + 1;
  }
  // one piece per worker F .. F + K - 1, in slots item + F ..
  const int base = item + F;
  auto slot_of = [base](int k) { return base + k; };
  auto none = [](int) { return 0; };
  // the row's four outputs from the pieces and a term (m0, l0, o0) in hand
  auto merged = [&](int t, float m0, float l0, float4 o0) {
    const int r = (4 * t) / D, d0 = 4 * t - r * D;
    MergeState4 st{m0, l0, o0};
    if (K <= kBatchShort)
      fold_two<kBatchShort>(st, a.ws_part, slot_of, K, R, r, a.ws_part, none, 0, 0, d0, D);
    else
      fold_two<kBatch>(st, a.ws_part, slot_of, K, R, r, a.ws_part, none, 0, 0, d0, D);
    const float inv = 1.f / st.Lt;
    store_out4<TT>(a.out, orow0 + 4 * t,
                   make_float4(st.acc.x * inv, st.acc.y * inv, st.acc.z * inv, st.acc.w * inv));
  };
  auto v_new4 = [&](int t) {
    const int d0 = (4 * t) % D;
    return make_float4(elem<TT>(a.v_new, nrow + d0), elem<TT>(a.v_new, nrow + d0 + 1),
                       elem<TT>(a.v_new, nrow + d0 + 2), elem<TT>(a.v_new, nrow + d0 + 3));
  };
  if (!FOLD || !a.fold_in_merge) {
    // the pieces hold every position; a sequence of one (FOLD, n = 0) is
    // its new token alone: weight 1, row v_new
    const bool only_new = FOLD && n == 0;
    for (int t = tid; t < total; t += per)
      merged(t, only_new ? 0.f : -INFINITY, only_new ? 1.f : 0.f,
             only_new ? v_new4(t) : make_float4(0.f, 0.f, 0.f, 0.f));
  } else {
    __shared__ float s_new[16];  // the new token's score per q row (base-2 domain)
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
    for (int r = wv; r < R; r += nw) {
      float p = 0.f;
      for (int d = lane; d < D; d += 64)
        p = fmaf(elem<TT>(a.q, orow0 + (int64_t)r * D + d), elem<TT>(a.k_new, nrow + d), p);
      for (int m = 1; m < 64; m <<= 1) p += __shfl_xor(p, m);
      if (lane == 0) s_new[r] = p * a.scale_log2e;
    }
    __syncthreads();
    for (int t = threadIdx.x; t < total; t += blockDim.x)
      merged(t, s_new[(4 * t) / D], 1.f, v_new4(t));
  }
  store_token();
}

// pa_decode_shared: a group of threads per item (sequence b, head h), one
// thread per four consecutive outputs of a q row.  Joins the tail pass's
// partials of the item (its workers F .. F+K-1) with, when the sequence's
// group has a shared prefix, the prefix pass's partials of item (group, kv
// head) at row (b - first member) * G + q head % G of their 16-row records;
// all share one denominator after rescaling to the common maximum (the Z / o
// equations of wq-win.github.io "079 | vLLM 与 PagedAttention", section 二).
// The sequence's group facts come from one record the tail pass exported,
// so that every index load but the partials' is issued at once.
template <typename TT>
__global__ __launch_bounds__(1024) void cascade_merge_kernel(DecodeArgs a, int H, int R,
                                                             int ipw) {
  const int D = a.head_dim, B = a.num_seqs, NG = a.num_groups;
  const int per = blockDim.x / ipw;  // threads per item
  const int item = blockIdx.x * ipw + threadIdx.x / per;
  const int tid = threadIdx.x - (threadIdx.x / per) * per;
  if (item >= B * H) return;
  // items head-major: a workgroup holds consecutive sequences of one head,
  // so the members of a group read the rows of their shared prefix records
  // from one CU instead of one XCD each
  const int h = item / B, b = item - h * B;
  const int it = b * H + h;  // the item's index in the tail pass
  const int Gq = a.num_q_heads / a.num_kv_heads;
  const int kvh = R == 1 ? h / Gq : h;
  const int* pre = a.ws_pre;
  const int4 gr = *reinterpret_cast<const int4*>(a.ws_grp + 4 * b);
  const int n = (pre[b + 1] - pre[b]) / H;  // tail steps of the item
  const int p_total = a.pws_pre[NG];
  const int g = min(max(gr.x, 0), NG - 1);
  const int first = min(max(gr.y, 0), B - 1);
  const int np = (gr.w - gr.z) / a.num_kv_heads;  // prefix steps per kv head
  const int64_t orow0 = ((int64_t)b * a.num_q_heads + (int64_t)h * R) * D;
  const int total = R * D / 4;  // groups of four outputs
  if (n == 0 && np == 0) {  // empty sequence: zero rows
    for (int t = tid; t < R * D; t += per) store_out<TT>(a.out, orow0 + t, 0.f);
    return;
  }
  int F = 0, K = 0;
  if (n > 0) {
    const Split sp = make_split(a.num_workers, pre[B]);
    const int64_t S = pre[b] + (int64_t)h * n, E = S + n;
    F = sp.worker_of(S);
    const int Lw = sp.worker_of(E - 1);
    if (np == 0 && F == Lw) return;  // no prefix, one piece: the tail pass wrote the row
    K = Lw - F + 1;
  }
  int Fp = 0, Kp = 0;
  if (np > 0) {
    const Split pp = make_split(a.p_num_workers, p_total);
    const int64_t S = gr.z + (int64_t)kvh * np, E = S + np;
    Fp = pp.worker_of(S);
    Kp = pp.worker_of(E - 1) - Fp + 1;
  }
  const int base = it + F, pbase = g * a.num_kv_heads + kvh + Fp;
  auto sa = [base](int k) { return base + k; };
  auto sb = [pbase](int k) { return pbase + k; };
  for (int t = tid; t < total; t += per) {
    const int r = (4 * t) / D, d0 = 4 * t - r * D;
    MergeState4 st{-INFINITY, 0.f, make_float4(0.f, 0.f, 0.f, 0.f)};
    const int rp = (b - first) * Gq + (R == 1 ? h % Gq : r);  // row in the prefix records
    const int kp = rp >= 0 && rp < kPrefixRows ? Kp : 0;
    if (K + kp <= kBatchShort)
      fold_two<kBatchShort>(st, a.ws_part, sa, K, R, r, a.pws_part, sb, kp, rp, d0, D);
    else
      fold_two<kBatch>(st, a.ws_part, sa, K, R, r, a.pws_part, sb, kp, rp, d0, D);
    const float inv = 1.f / st.Lt;
    store_out4<TT>(a.out, orow0 + 4 * t,
                   make_float4(st.acc.x * inv, st.acc.y * inv, st.acc.z * inv, st.acc.w * inv));
  }
}

// The store alone, for a pa_decode_write whose decode runs unsplit (the
// plain kernel then reads the token from the pool): one workgroup per
// (sequence, kv head), one thread per element.
template <typename TT>
__global__ __launch_bounds__(256) void store_new_tokens_kernel(DecodeArgs a) {
  using E = typename TT::raw;
  const int b = blockIdx.y, g = blockIdx.x;
  const int L = clamp_len(a.context_lens[b], a.len_cap);
  if (L == 0) return;
  const int32_t blk = a.block_tables[(int64_t)b * a.max_blocks_per_seq + (L - 1) / a.block_size];
  const int64_t nrow = (int64_t)b * a.new_stride + (int64_t)g * a.head_dim;
  for (int d = threadIdx.x; d < a.head_dim; d += blockDim.x) {
    const NewSlot ns = new_slot(a, blk, g, L, d, TT::bytes);
    if (ns.k < 0) return;
    __builtin_nontemporal_store(reinterpret_cast<const E*>(a.k_new)[nrow + d],
                                reinterpret_cast<E*>(const_cast<void*>(a.k_cache)) + ns.k);
    __builtin_nontemporal_store(reinterpret_cast<const E*>(a.v_new)[nrow + d],
                                reinterpret_cast<E*>(const_cast<void*>(a.v_cache)) + ns.v);
  }
}


}  // namespace

namespace {
// Threads per item (at most 1024; a multiple of 64 where the workgroup
// syncs, else of 32: such items may share a wavefront) and items per
// workgroup: one where it syncs; 512 threads' worth where the merge stores
// the step's tokens (every item has work: fewer, larger workgroups measured
// faster); else as many as leave about four workgroups per CU (at most 512
// threads: most items of a batch of short contexts are unsplit and exit).
void merge_shape(int outputs, bool single, bool stores, int items, int* per, int* ipw) {
  const int q = single ? 64 : 32;
  *per = outputs >= 1024 ? 1024 : (outputs + q - 1) / q * q;
  *ipw = single ? 1
         : stores ? std::max(1, 512 / *per)
                  : std::max(1, std::min(items / (4 * device_cus()), 512 / *per));
}
}  // namespace

hipError_t launch_decode_merge(const DecodeArgs& a, pa_dtype dt, int items_per_seq,
                               hipStream_t s) {
  if (a.num_seqs == 0 || !a.split) return hipSuccess;
  const int R = a.num_q_heads / items_per_seq;
  const bool fold = a.k_new != nullptr;
  int per, ipw;
  const int items = a.num_seqs * items_per_seq;
  // a thread per four outputs; when the merge stores the new tokens, at
  // least a thread per dim (their stores run along the rows, one element a
  // thread: the OPT-13B step's merge took 12.2 us with four a thread, 10.4
  // with one)
  merge_shape(std::max(R * a.head_dim / 4, fold ? a.head_dim : 0), fold && a.fold_in_merge, fold,
              items, &per, &ipw);
  dim3 grid((items + ipw - 1) / ipw), block(per * ipw);
  switch (dt) {
    case PA_F32:
      if (fold)
        hipLaunchKernelGGL((decode_merge_kernel<F32, true>), grid, block, 0, s, a, items_per_seq,
                           R, ipw);
      else
        hipLaunchKernelGGL((decode_merge_kernel<F32, false>), grid, block, 0, s, a, items_per_seq,
                           R, ipw);
      break;
    case PA_F16:
      if (fold)
        hipLaunchKernelGGL((decode_merge_kernel<F16, true>), grid, block, 0, s, a, items_per_seq,
                           R, ipw);
      else
        hipLaunchKernelGGL((decode_merge_kernel<F16, false>), grid, block, 0, s, a, items_per_seq,
                           R, ipw);
      break;
    case PA_BF16:
      if (fold)
        hipLaunchKernelGGL((decode_merge_kernel<BF16, true>), grid, block, 0, s, a,
                           items_per_seq, R, ipw);
      else
        hipLaunchKernelGGL((decode_merge_kernel<BF16, false>), grid, block, 0, s, a,
                           items_per_seq, R, ipw);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_cascade_merge(const DecodeArgs& a, pa_dtype dt, int items_per_seq,
                                hipStream_t s) {
  if (a.num_seqs == 0) return hipSuccess;
  const int R = a.num_q_heads / items_per_seq;
  // a thread per four outputs (items share wavefronts: no barrier inside),
  // up to a group of 8 members per workgroup
  const int per = std::min(1024, (R * a.head_dim / 4 + 31) / 32 * 32);
  const int ipw = std::max(1, std::min(8, 1024 / per));
  const int items = a.num_seqs * items_per_seq;
  dim3 grid((items + ipw - 1) / ipw), block(per * ipw);
  switch (dt) {
    case PA_F32:
      hipLaunchKernelGGL(cascade_merge_kernel<F32>, grid, block, 0, s, a, items_per_seq, R, ipw);
      break;
    case PA_F16:
      hipLaunchKernelGGL(cascade_merge_kernel<F16>, grid, block, 0, s, a, items_per_seq, R, ipw);
      break;
    case PA_BF16:
      hipLaunchKernelGGL(cascade_merge_kernel<BF16>, grid, block, 0, s, a, items_per_seq, R, ipw);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_store_new_tokens(const DecodeArgs& a, pa_dtype dt, hipStream_t s) {
  if (a.num_seqs == 0 || !a.k_new) return hipSuccess;
  dim3 grid(a.num_kv_heads, a.num_seqs);
  switch (dt) {
    case PA_F32:
      hipLaunchKernelGGL(store_new_tokens_kernel<F32>, grid, dim3(128), 0, s, a);
      break;
    case PA_F16:
      hipLaunchKernelGGL(store_new_tokens_kernel<F16>, grid, dim3(128), 0, s, a);
      break;
    case PA_BF16:
      hipLaunchKernelGGL(store_new_tokens_kernel<BF16>, grid, dim3(128), 0, s, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace pa
