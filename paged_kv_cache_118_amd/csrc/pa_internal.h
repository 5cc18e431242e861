// Internal declarations shared by libpa's HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// ---------------------------------------------------------------- storage --
// Tag types for the three storage dtypes.  Raw elements are moved as bits;
// arithmetic is always fp32.
struct F32 {
  using raw = float;
  static constexpr int bytes = 4;
};
struct F16 {
  using raw = uint16_t;
  static constexpr int bytes = 2;
};
struct BF16 {
  using raw = uint16_t;
  static constexpr int bytes = 2;
};

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf168_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float lo_to_float(F16, uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float hi_to_float(F16, uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
__device__ __forceinline__ float lo_to_float(BF16, uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_to_float(BF16, uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}

// fp32 -> storage bits, round to nearest even.
__device__ __forceinline__ uint16_t to_bits(F16, float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ uint16_t to_bits(BF16, float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ float to_bits(F32, float f) { return f; }

// Dot product of two packed pairs accumulated in fp32.
__device__ __forceinline__ float dot2(F16, uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                false);
}
__device__ __forceinline__ float dot2(BF16, uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a),
                                         __builtin_bit_cast(bf162_t, b), c, false);
}

// c + the two elements of a packed pair, in fp32 (a dot product with 1, 1):
// a row sum over exactly the rounded weights a matrix op consumes.
__device__ __forceinline__ float psum2(F16, uint32_t w, float c) {
  return dot2(F16{}, w, 0x3C003C00u, c);
}
__device__ __forceinline__ float psum2(BF16, uint32_t w, float c) {
  return dot2(BF16{}, w, 0x3F803F80u, c);
}

// ------------------------------------------------------- lane exchanges --
// max / sum of x and x in the lane 32 (16) apart, without LDS: one
// v_permlane32_swap (v_permlane16_swap) of x with a copy of itself leaves,
// in every lane, x and its partner's x in the two registers.
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_add(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// ------------------------------------------------------------ decode args --
struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float scale_log2e;   // scale * log2(e): scores live in the base-2 domain
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t head_dim;
  int32_t max_blocks_per_seq;
  int32_t len_cap;     // min(max_context_len, max_blocks_per_seq * block_size)
  int64_t num_blocks;
  // work split (decode_split.h)
  int32_t split;        // 0: one item per worker, 1: token-balanced stream split
  int32_t part_steps;   // split 1: steps per partition (partials cut there), 0 = none
  int32_t num_workers;  // wavefronts launched
  // split 1: partials (decode_split.h), one record of part_record(rows, D)
  // floats per slot; rows of an item are its q heads (1 for the MHA kernel,
  // the group for GQA).  Record layout: o of (row r, dim d) at
  // ((d/16)*4 + d%16/4)*rows*4 + r*4 + d%4 (for one row simply d), then a
  // 128-byte tail: m of row r at rows*D + r, l at rows*D + 16 + r, the rest
  // zero.  A record is written whole by one wavefront, in whole cache lines.
  float* ws_part;       // [slots][part_record(rows, D)]
  int32_t* ws_pre;      // [B+1] step prefix per sequence (for the merge)
  int32_t* ws_ppre;     // [B+1] partition prefix per sequence (part_steps > 0)
  // Fused cache write (pa_decode_write), or null: sequence b's new token
  // (position L_b - 1), K and V rows [Hkv][D] at element b * new_stride of
  // k_new / v_new.  The split decode kernels then cover positions 0 .. L_b-2;
  // the token's own term is added by the worker that finishes the item (MHA
  // kernel) or, with fold_in_merge, by the merge kernel (grouped-query
  // kernel, which then writes partials only); the merge kernel stores the
  // token into its slot (through k_cache / v_cache).  The generic kernel
  // does everything itself.
  const void* k_new;
  const void* v_new;
  int64_t new_stride;
  int32_t fold_in_merge;  // 1: the decode kernel leaves the token's term to the merge
  // Shared-prefix decode (pa_decode_shared), or num_groups = 0: groups of
  // consecutive sequences, gs[g] .. gs[g+1]-1, whose first group_prefix[g]
  // positions are the same physical blocks.  The tail pass streams every
  // sequence from its group's prefix on and exports each sequence's group
  // facts (ws_grp, four ints per sequence: export_groups); the prefix pass
  // (its own split: pws_part, pws_pre, p_num_workers; records of 16 rows)
  // reads each shared block once for the members' q rows; the merge joins
  // both passes' partials of every row.
  const int32_t* group_start;
  const int32_t* group_prefix;
  int32_t num_groups;
  int32_t* ws_grp;
  float* pws_part;
  int32_t* pws_pre;
  int32_t p_num_workers;
};

// Compute units of the current device (256 if the query fails).
int device_cus();

// Rows of a prefix-pass partial record (members x q heads per kv head).
constexpr int kPrefixRows = 16;

// ----------------------------------------------------------- prefill args --
struct PrefillArgs {
  void* out;                   // [num_tokens][num_q_heads][head_dim]
  const void* q;               // [num_tokens][num_q_heads][head_dim]
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;  // [num_seqs + 1]
  float scale_log2e;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t head_dim;
  int32_t max_blocks_per_seq;
  int32_t max_query_len;
  int32_t len_cap;             // min(max_context_len, max_blocks_per_seq * block_size)
  int64_t num_blocks;
};

// pa_decode / pa_decode_write behind argument checks (capi.cpp).
pa_status decode_impl(void* out, const void* q, const void* k_new, const void* v_new,
                      int64_t new_stride, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, float scale,
                      int32_t block_size, int32_t num_kv_heads, int32_t num_seqs,
                      int32_t num_q_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                      int32_t max_context_len, int64_t num_blocks, pa_dtype dtype,
                      int32_t partition_size, void* workspace, size_t workspace_bytes,
                      void* stream);

hipError_t launch_prefill(const PrefillArgs& a, pa_dtype dt, hipStream_t s);
bool prefill_supported(pa_dtype dt, int head_dim, int block_size);

// Launchers (return hipSuccess or the launch error).
hipError_t launch_decode_valu(const DecodeArgs& a, pa_dtype dt, hipStream_t s);
hipError_t launch_decode_mfma(const DecodeArgs& a, pa_dtype dt, hipStream_t s);
hipError_t launch_decode_generic(const DecodeArgs& a, pa_dtype dt, hipStream_t s);
// Merge of the split items' partials (decode_merge.hip); step = tokens per
// worker step of the decode kernel that ran.
hipError_t launch_decode_merge(const DecodeArgs& a, pa_dtype dt, int items_per_seq,
                               hipStream_t s);
// pa_decode_shared: the prefix pass (matrix cores; a.num_workers / ws_part /
// ws_pre must be the pass's own) and the merge of both passes' partials.
hipError_t launch_decode_prefix(const DecodeArgs& a, pa_dtype dt, hipStream_t s);
hipError_t launch_cascade_merge(const DecodeArgs& a, pa_dtype dt, int items_per_seq,
                                hipStream_t s);
// pa_decode_write with an unsplit decode: store the new tokens first (the
// decode then reads them from the pool).
hipError_t launch_store_new_tokens(const DecodeArgs& a, pa_dtype dt, hipStream_t s);
bool decode_valu_supported(pa_dtype dt, int head_dim, int block_size);
// Resident wavefronts per CU of the kernel a call with these arguments runs.
int decode_valu_waves_per_cu(pa_dtype dt, int head_dim);
int decode_mfma_waves_per_cu(pa_dtype dt, int head_dim);
bool decode_mfma_supported(pa_dtype dt, int head_dim, int block_size, int group);

hipError_t launch_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                                    const int64_t* slots, int32_t num_tokens, int64_t k_stride,
                                    int64_t v_stride, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int64_t num_blocks, int elem_bytes,
                                    hipStream_t s);
hipError_t launch_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                              const int64_t* pairs, int32_t num_pairs, int64_t block_bytes,
                              int64_t src_blocks, int64_t dst_blocks, hipStream_t s);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs,
                              int32_t num_pairs, int64_t block_bytes, int64_t num_blocks,
                              hipStream_t s);

// Dynamic LDS of a split decode launch (one workgroup): the per-sequence step
// and partition prefixes and the clamped lengths, 3 * num_seqs + 2 ints.
__host__ __device__ inline size_t split_lds_bytes(int num_seqs) {
  return sizeof(int) * (3 * (size_t)num_seqs + 2);
}
// ... and of a shared-prefix pass: the tail pass adds each sequence's first
// position and group, both passes the group starts and prefix lengths.
__host__ __device__ inline size_t cascade_lds_bytes(int num_seqs, int num_groups) {
  return split_lds_bytes(num_seqs) + sizeof(int) * (2 * (size_t)num_seqs + 2 * (size_t)num_groups + 1);
}

// Floats per partial record (see DecodeArgs::ws_part); rows <= 16.
__host__ __device__ inline int part_record(int rows, int head_dim) { return rows * head_dim + 32; }

// Tokens per V slab: V is stored as [block][head][BS/VS][D][VS].
__host__ __device__ inline int v_slab(int block_size) { return block_size < 8 ? block_size : 8; }

// K is stored as 16-byte pieces, [block][head][D/X][BS][X] with X = 16 / element
// size: piece p of every offset of a block's head is adjacent, so 16
// consecutive tokens' piece p form one 256-byte run.  Element index of
// (block, head, offset, d):
__host__ __device__ inline int64_t k_elem_index(int64_t blk, int64_t h, int off, int d,
                                                int64_t hkv, int bs, int D, int elem_bytes) {
  const int x = 16 / elem_bytes;
  return (((blk * hkv + h) * (D / x) + d / x) * bs + off) * x + d % x;
}

}  // namespace pa
