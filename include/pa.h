/*
 * pa.h -- C ABI of libpa: paged decode attention, KV-cache write, block copy
 * and a host block allocator, for AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages on PagedAttention):
 *  [P5] wq-win.github.io, "079 | vLLM 与 PagedAttention" (digest of Kwon et al.,
 *       SOSP 2023): section 二 (the Z / o equations, copy-on-write, tail
 *       waste), section 三 (per-iteration block management).
 *  [P1] gitcode.csdn.net, "vLLM 推理引擎：PagedAttention 与 KVCache 管理":
 *       section 1 (block data structures), section 3 (the forward signature
 *       query / key_cache / value_cache / block_tables / context_lens).
 *  [P3] deepinsea.top, "PagedAttention 内存管理深度解析", section
 *       "分页机制设计" (free list, all-or-nothing allocation).
 *  [P4] vkads.cloudxian.cn, "vLLM PagedAttention源码：KV Cache", kernel
 *       pseudocode (flat slot numbering of a block).
 *
 * Conventions for every call
 *  - Device pointers are caller-owned (e.g. torch tensors); libpa never
 *    allocates or frees device memory.  The decode split path uses the
 *    caller's workspace.
 *  - Calls return a pa_status and never abort or throw.  GPU calls are
 *    asynchronous on `stream` (a hipStream_t; NULL = the null stream) and run
 *    in issue order; a launch failure is PA_EHIP.
 *  - Host-visible arguments are checked (null pointers, sizes, alignment,
 *    supported dtype / head_dim / block_size, workspace size).  Device data
 *    (block ids, slots, lengths) is not checked on the hot path; kernels
 *    clamp or skip out-of-range ids so that a bad id never faults, but the
 *    result for that sequence / token is then undefined.  With the
 *    environment variable PA_VALIDATE=1, the GPU calls first copy the index
 *    arrays to the host, synchronise `stream`, and return PA_EVALIDATE on an
 *    out-of-range id, a duplicate slot or an overlapping copy pair.
 *
 * KV pool layout (one layer).  BS = block_size, D = head_dim, Hkv = kv heads,
 * X = 16 / element size (4 for fp32, 8 for fp16 / bf16), VS = min(BS, 8).
 * Element (physical block b, kv head h, offset o, dim d):
 *   K:  k_cache[(((b*Hkv + h)*(D/X) + d/X)*BS + o)*X + d%X]
 *   V:  v_cache[(((b*Hkv + h)*(BS/VS) + o/VS)*D + d)*VS + o%VS]
 *  K stores 16-byte pieces of X dims; piece p of all BS offsets of a block's
 *  head is one run, so the pieces p .. p+3 of 16 consecutive tokens form one
 *  contiguous kilobyte: exactly what a wavefront loads for one step of the
 *  dot products q . K[u] (four lanes per token on the VALU path, one MFMA
 *  operand of 16 tokens for grouped heads), in whole cache lines.  V stores
 *  slabs of VS tokens, each slab [D][VS] (token index fastest): one 16-byte
 *  load is 8 tokens of one V row, which is what the weighted sum over tokens
 *  consumes, and a wavefront reads each slab with contiguous 16-byte loads.
 *  A token's slot is b*BS + o ([P4]).  BS must be 1, 2, 4, 8 or a multiple
 *  of 16; D must be a multiple of X.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_EINVAL = -1,    /* bad argument (null pointer, size, alignment) */
  PA_ENOTSUP = -2,   /* valid but unsupported dtype / head_dim / block_size */
  PA_ENOMEM = -3,    /* allocator: not enough free blocks (nothing changed) */
  PA_EHIP = -4,      /* a HIP runtime call or kernel launch failed */
  PA_EVALIDATE = -5, /* PA_VALIDATE=1 found a bad index in device data */
  PA_ENOENT = -6,    /* allocator: unknown sequence id, or id already used */
  PA_ESCRATCH = -7   /* pa_decode_noalloc: the call needs more than its static scratch */
} pa_status;

typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 } pa_dtype;

/* Message for a status code (static storage). */
const char* pa_strerror(pa_status s);

/* ------------------------------------------------------------------------
 * pa_decode -- single-query paged attention for every (sequence, q head).
 *
 * Computes, for sequence b with L = context_lens[b] valid positions and q
 * head h reading kv head g = h / (num_q_heads / num_kv_heads):
 *   s_u = scale * q[b,h,:] . K[u],  o = sum_u exp(s_u) V[u] / sum_u exp(s_u)
 * over u = 0 .. L-1, with one denominator shared by all blocks and the
 * unfilled tail of the last block excluded ([P5] section 二, the Z / o
 * equations).  Position u lives in physical block block_tables[b][u / BS] at
 * offset u % BS ([P1] section 3).  L = 0 gives a zero row.  fp32 accumulation;
 * the output is rounded to nearest-even in `dtype`.
 *
 *  out          [num_seqs][num_q_heads][head_dim] of dtype (device, written)
 *  q            [num_seqs][num_q_heads][head_dim] of dtype (device)
 *  k_cache      K pool, layout above, num_blocks blocks (device)
 *  v_cache      V pool, layout above (device)
 *  block_tables [num_seqs][max_blocks_per_seq] int32 (device); entries past
 *               ceil(L / BS) are never used (the kernels may load them, within
 *               the row's max_blocks_per_seq entries, as part of a 64-entry
 *               window; padding is conventionally -1)
 *  context_lens [num_seqs] int32 (device).  Must satisfy
 *               L <= max_context_len and L <= max_blocks_per_seq * BS;
 *               positions beyond either bound are ignored.
 *  scale        score scale (1/sqrt(head_dim) for standard attention)
 *  partition_size  how the context is split:
 *               0  = token-balanced: all (sequence, head) items are laid end
 *                    to end and each of a fixed number of wavefronts per CU
 *                    (all resident at once) takes an equal share of the
 *                    tokens, whatever the lengths; an
 *                    item shared by several wavefronts yields one fp32
 *                    (max, sum, unnormalised output) partial per wavefront;
 *               >0 = split-context partitions: each sequence's context is
 *                    cut into partitions of this many tokens (a multiple of
 *                    256) from its start, and the wavefronts take balanced
 *                    shares of whole partitions (no partition is divided
 *                    between two); a wavefront folds the consecutive
 *                    partitions it holds of an item into one fp32 partial,
 *                    so an item spread over several wavefronts yields one
 *                    partial per wavefront, as above;
 *               -1 = one wavefront per (sequence, head) item, nothing split.
 *               The partials of an item are reduced by a second kernel
 *               (rescaled to their common maximum: one denominator, as in the
 *               Z / o equations); results agree across modes within rounding.
 *  workspace    device scratch of at least pa_decode_workspace_bytes(...)
 *               bytes (may be NULL when that size is 0); contents need no
 *               initialisation and are clobbered.  Calls that run
 *               concurrently must not share a workspace.
 * Requirements: num_q_heads % num_kv_heads == 0; head_dim in {16, 32, 64,
 * 128, 256}; q, out and the pools 16-byte aligned.
 * ---------------------------------------------------------------------- */
pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens, float scale,
                    int32_t block_size, int32_t num_kv_heads, int32_t num_seqs,
                    int32_t num_q_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                    int32_t max_context_len, int64_t num_blocks, pa_dtype dtype,
                    int32_t partition_size, void* workspace, size_t workspace_bytes,
                    void* stream);

/* ------------------------------------------------------------------------
 * pa_decode_write -- one decode iteration's cache write and attention in a
 * single launch: the write of each sequence's new token followed by
 * attention over the context that includes it ([P5] section 三: the new
 * token's K/V is stored into its slot before the iteration attends).
 *
 * For every sequence b with L = context_lens[b] >= 1, the token at position
 * L - 1 has K row k_new[b*new_token_stride ...] and V row v_new[...] (each
 * [num_kv_heads][head_dim] contiguous, dtype).  The call stores both rows
 * into that position's slot, block_tables[b][(L-1)/BS] * BS + (L-1) % BS
 * (bit for bit, as pa_reshape_and_cache with that slot would), and computes
 * `out` exactly as pa_decode would over the pools after that store; the
 * kernels read position L - 1 from the new rows themselves.  Sequences with
 * L = 0 write nothing.  A table entry outside the pool skips the store (the
 * row's result is then undefined, as for pa_decode).
 *  k_new, v_new      device rows, 16-byte aligned; new_token_stride in
 *                    elements, >= num_kv_heads * head_dim, a multiple of 16
 *                    bytes.  Host pointers are PA_EINVAL before any launch.
 *  other arguments   as pa_decode (same workspace size).
 * Every new token's slot must belong to its sequence alone in this call: no
 * two sequences write one slot, and no sequence reads another's new slot as
 * one of its positions (a block about to be written is private, which the
 * allocator's copy-on-write pairs, copied first, ensure).  PA_VALIDATE=1
 * checks this too.
 * ---------------------------------------------------------------------- */
pa_status pa_decode_write(void* out, const void* q, const void* k_new, const void* v_new,
                          int64_t new_token_stride, void* k_cache, void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens, float scale,
                          int32_t block_size, int32_t num_kv_heads, int32_t num_seqs,
                          int32_t num_q_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                          int32_t max_context_len, int64_t num_blocks, pa_dtype dtype,
                          int32_t partition_size, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ------------------------------------------------------------------------
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory: code under graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, result and checks as pa_decode, minus
 * the workspace: the split's scratch is a static array inside libpa, one per
 * device, of pa_decode_noalloc_scratch_bytes() bytes (32 MiB), held by every
 * device the library runs on until the process ends.  A call whose
 * pa_decode_workspace_bytes(...) exceeds it returns PA_ESCRATCH before any
 * launch.  Nothing is allocated on any call.  Every call on a device shares
 * that device's array, so calls that overlap on one device (e.g. on two
 * streams) race and must not be issued; nothing in the array needs clearing
 * between calls.
 * ---------------------------------------------------------------------- */
pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            float scale, int32_t block_size, int32_t num_kv_heads,
                            int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                            int32_t max_blocks_per_seq, int32_t max_context_len,
                            int64_t num_blocks, pa_dtype dtype, int32_t partition_size,
                            void* stream);
/* Bytes of pa_decode_noalloc's static scratch (the largest workspace it serves). */
size_t pa_decode_noalloc_scratch_bytes(void);

/* ------------------------------------------------------------------------
 * pa_decode_shared -- pa_decode for a batch in which groups of sequences
 * share their leading blocks (a beam or parallel-sampling family, prompts
 * with a common prefix: [P5] section 二 "共享与写时复制" -- the shared blocks
 * are held once, by reference count).  Same result as pa_decode (one softmax
 * over all of each sequence's positions, [P5] section 二, the Z / o
 * equations), but each shared block is read from memory once per group
 * instead of once per member.
 *
 * Groups are runs of consecutive sequences: group g is sequences
 * group_start[g] .. group_start[g+1]-1, and its first group_prefix_len[g]
 * positions (a multiple of BS, at most every member's length) lie in the
 * same physical blocks in every member's table.  group_start[0] = 0,
 * group_start[num_groups] = num_seqs, every group has at least one member
 * and members * (num_q_heads / num_kv_heads) <= 16; a prefix of 0 is allowed
 * (a group that shares nothing).  pa_alloc_share_groups produces such groups
 * from an allocator's tables.
 *
 * How: a prefix pass on the matrix cores reads each group's shared blocks
 * once per kv head and scores them against the q rows of all its members (a
 * small dense contraction: members x q heads per kv head), a tail pass
 * streams each sequence from its group's prefix on, and a merge combines
 * the two fp32 partial softmax states of every row.
 *  group_start       [num_groups + 1] int32 (device)
 *  group_prefix_len  [num_groups] int32 (device), tokens
 *  workspace         at least pa_decode_shared_workspace_bytes(...) bytes
 *  other arguments   as pa_decode (the split is the token-balanced one)
 * The prefix pass needs f16 / bf16, head_dim 64 or 128 and block_size 8, 16
 * or a multiple of 32; otherwise, and for num_groups = 0, the call is a plain
 * pa_decode with partition_size 0 (the same result).  Group data is not
 * checked on the hot path (PA_VALIDATE=1 checks all of the above, table
 * entries included); groups that break the rules give undefined rows, never
 * an access outside the tables, pools or workspace.
 * ---------------------------------------------------------------------- */
pa_status pa_decode_shared(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens, float scale,
                           int32_t block_size, int32_t num_kv_heads, int32_t num_seqs,
                           int32_t num_q_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                           int32_t max_context_len, int64_t num_blocks, pa_dtype dtype,
                           const int32_t* group_start, const int32_t* group_prefix_len,
                           int32_t num_groups, void* workspace, size_t workspace_bytes,
                           void* stream);
size_t pa_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_groups,
                                        int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size,
                                        int32_t max_context_len, pa_dtype dtype);

/* Workspace bytes pa_decode needs for these sizes (0 when nothing splits).
 * Pass the same arguments as to pa_decode, on the device it will run on (the
 * balanced split sizes itself by the device's CU count). */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                 int32_t partition_size, pa_dtype dtype);

/* The split pa_decode uses for these arguments: -1 = one wavefront per
 * item, 0 = token-balanced, > 0 = balanced shares of whole partitions of that
 * many tokens. */
int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                 int32_t partition_size, pa_dtype dtype);

/* ------------------------------------------------------------------------
 * pa_prefill -- chunked-prefill attention over the paged cache.
 *
 * A prompt processed in chunks (zhy-blog.vercel.app, vLLM post, section 4.2
 * "Chunked Prefill的解决方案"): sequence b's query tokens query_start[b] ..
 * query_start[b+1]-1 are the last ql_b of its L_b = context_lens[b] positions,
 * already written to the pools (pa_reshape_and_cache), so the token at index
 * r of the chunk sits at position p = L_b - ql_b + r.  Token p, q head h
 * attends to positions 0 .. p only (the mask follows the token's place in the
 * whole prompt) through the block table, with one softmax over all of them
 * ([P5] section 二, restricted to u <= p); kv head h / (Hq / Hkv).  fp32
 * accumulation; output rounded to nearest-even in `dtype`.
 *
 *  out, q        [num_tokens][num_q_heads][head_dim] of dtype (device); rows
 *                packed as in [P1] section 3's forward
 *  query_start   [num_seqs + 1] int32 (device): query_start[0] = 0, non-
 *                decreasing; ql_b = query_start[b+1] - query_start[b] must not
 *                exceed max_query_len nor L_b (rows of a sequence with
 *                ql_b > L_b are left unwritten)
 *  block_tables, context_lens, pools, scale: as pa_decode
 * Supported: f16 / bf16, head_dim 64 or 128, block_size 8, 16 or a multiple
 * of 32 (PA_ENOTSUP otherwise).  No workspace.
 * ---------------------------------------------------------------------- */
pa_status pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, const int32_t* context_lens,
                     const int32_t* query_start, float scale, int32_t block_size,
                     int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads,
                     int32_t head_dim, int32_t max_blocks_per_seq, int32_t max_query_len,
                     int32_t max_context_len, int64_t num_blocks, pa_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * pa_reshape_and_cache -- write new tokens' K and V rows into their slots.
 *
 * Token t (row k[t*k_token_stride ...], [num_kv_heads][head_dim] contiguous,
 * same for v) goes to slot = slot_mapping[t] = block * BS + offset ([P4]
 * pseudocode), in both pools, bit for bit.  A negative slot is padding and is
 * skipped.  Slots must be distinct within one call (duplicates race).  This is
 * the write that precedes attention in each iteration ([P5] section 三).
 *  k, v          device token rows of dtype; strides in elements, >= Hkv*D
 *  slot_mapping  [num_tokens] int64 (device)
 * Requirements: head_dim * element size a multiple of 16 bytes; k, v and the
 * pools 16-byte aligned; strides a multiple of 16 bytes.  k and v must be
 * device memory (or pinned host memory mapped at the same address): any
 * other pointer, e.g. pageable host memory, is PA_EINVAL before any launch.
 * ---------------------------------------------------------------------- */
pa_status pa_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                               const int64_t* slot_mapping, int32_t num_tokens,
                               int64_t k_token_stride, int64_t v_token_stride,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int64_t num_blocks, pa_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * pa_swap_blocks -- move whole blocks between two pools of the same layout,
 * typically the device pool and a pinned host pool: the swap that preempts a
 * sequence group when device memory runs short and brings its cache back
 * later (deepinsea.top, "PagedAttention 内存管理深度解析", part "Swap 机制";
 * [P5] section 三, the swap-out / swap-in steps of each iteration).
 *
 * For each pair p, every byte of block src_dst_pairs[2p] of (src_k, src_v)
 * (all heads, all BS slots) is copied to block src_dst_pairs[2p+1] of
 * (dst_k, dst_v), on `stream`, by a kernel that reads and writes through the
 * pointers.  Every pointer must therefore be device memory or pinned host
 * memory mapped at the same address (e.g. hipHostMalloc, torch pin_memory);
 * anything else, such as pageable host memory, is PA_EINVAL and nothing runs.
 * Destinations must be distinct.  Pairs with an id outside its pool are
 * skipped (PA_VALIDATE=1: PA_EVALIDATE).
 *  src_dst_pairs  [num_pairs][2] int64, device or pinned host memory
 * ---------------------------------------------------------------------- */
pa_status pa_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                         const int64_t* src_dst_pairs, int32_t num_pairs, int64_t src_num_blocks,
                         int64_t dst_num_blocks, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, pa_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * pa_copy_blocks -- copy-on-write of whole blocks ([P5] section 二, part
 * "共享与写时复制"; [P1] / [P3] copy-on-write).
 *
 * For each pair p, every byte of block src_dst_pairs[2p] (all heads, all BS
 * slots, K and V) is copied to block src_dst_pairs[2p+1].  Destinations must
 * be distinct and no destination may be a source in the same call.
 *  src_dst_pairs  [num_pairs][2] int64 (device)
 * ---------------------------------------------------------------------- */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* src_dst_pairs,
                         int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int64_t num_blocks, pa_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * Host block allocator ([P1] section 1 PhysicalTokenBlock / BlockTable,
 * [P3] BlockManager, [P5] sections 二 and 三).  Host memory only; not thread
 * safe (one allocator per scheduler thread).
 *
 * Physical ids are shuffled once from shuffle_seed (splitmix64-driven
 * Fisher-Yates; seed 0 keeps ids in order) and then taken from the end of the
 * free list and returned to its end (LIFO).  A sequence holds ceil(L / BS)
 * blocks.  Every block has a reference count; a block returns to the free
 * list only when its count reaches 0.
 * ---------------------------------------------------------------------- */
typedef struct pa_alloc pa_alloc;

/* NULL on bad arguments or host OOM. */
pa_alloc* pa_alloc_create(int64_t num_blocks, int32_t block_size, uint64_t shuffle_seed);
void pa_alloc_destroy(pa_alloc* a);

/* New sequence holding num_tokens (>= 0) tokens: ceil(num_tokens / BS) fresh
 * blocks, all or nothing (PA_ENOMEM leaves the allocator unchanged). */
pa_status pa_alloc_add_seq(pa_alloc* a, int64_t seq_id, int32_t num_tokens);

/* child shares every block of parent (each count + 1) and its length. */
pa_status pa_alloc_fork(pa_alloc* a, int64_t parent_id, int64_t child_id);

/* Reserve slots for the next n_tokens tokens of seq_id.  If the first write
 * goes into a partially filled tail block whose count is > 1, the block is
 * copied first: a fresh block replaces it in this sequence only, the old
 * block loses one reference, and the pair (old, new) is written to
 * cow_pairs_out[0..1] with *n_cow_out = 1 (else 0); the caller must run
 * pa_copy_blocks with it before pa_reshape_and_cache.  A new block is taken
 * whenever a position crosses a block boundary ([P5] section 三).
 * slots_out receives n_tokens slots.  All or nothing on PA_ENOMEM. */
pa_status pa_alloc_append(pa_alloc* a, int64_t seq_id, int32_t n_tokens, int64_t* slots_out,
                          int64_t* cow_pairs_out, int32_t* n_cow_out);

/* One step for n sequences in a single call: pa_alloc_append(seq_ids[i],
 * n_tokens[i]) for i = 0 .. n-1 in that order.  slots_out receives the slots
 * of all sequences back to back (sum of n_tokens entries); cow_pairs_out
 * receives the copy-on-write pairs, [*n_cow_out][2] in sequence order, room
 * for n pairs (may be NULL only if no sequence writes into a shared tail
 * block, else PA_EINVAL for that sequence).  Stops at the first sequence
 * that fails and returns its status: the *n_done_out sequences before it were
 * appended (their slots and pairs are written), it and those after it are
 * untouched.  Host memory only. */
pa_status pa_alloc_append_batch(pa_alloc* a, const int64_t* seq_ids, const int32_t* n_tokens,
                                int32_t n, int64_t* slots_out, int64_t* cow_pairs_out,
                                int32_t* n_cow_out, int32_t* n_done_out);

/* Drop the sequence, from its last block to its first: each block loses one
 * reference; a block at 0 is reclaimed (a prefix-cache entry stays cached,
 * evictable, see below). */
pa_status pa_alloc_free_seq(pa_alloc* a, int64_t seq_id);

/* pa_alloc_free_seq for a sequence whose reserved slots were never written
 * (e.g. its iteration was abandoned): every block it entered into the prefix
 * table leaves the table first, so that no later request can reuse a block
 * without its K/V, and then its blocks are released as by pa_alloc_free_seq
 * (those entries' blocks go to the free list).  Entries the sequence reused
 * from others are untouched. */
pa_status pa_alloc_discard_seq(pa_alloc* a, int64_t seq_id);

/* Groups for pa_decode_shared from the tables of seq_ids[0..n-1], in that
 * order: sequence j joins the group of an earlier sequence i (the group's
 * first member) when their tables begin with the same physical blocks, full
 * in both, and -- for the third member on -- at least as many of them as the
 * first two share; the group's prefix is the number of such blocks the first
 * two share (times block_size; 0 for a group of one).  A group never has more
 * than max_members members (pass 16 / (num_q_heads / num_kv_heads)).
 * Writes group_start_out[0..G] and group_prefix_out[0..G-1], *num_groups_out
 * = G; both arrays need room for n + 1 and n entries.  Host memory only. */
pa_status pa_alloc_share_groups(const pa_alloc* a, const int64_t* seq_ids, int32_t n,
                                int32_t max_members, int32_t* group_start_out,
                                int32_t* group_prefix_out, int32_t* num_groups_out);

/* Host rows for pa_decode: tables_out [n][max_blocks] (padded with -1) and
 * lens_out [n].  PA_EINVAL if a sequence holds more than max_blocks blocks. */
pa_status pa_alloc_block_tables(const pa_alloc* a, const int64_t* seq_ids, int32_t n,
                                 int32_t max_blocks, int32_t* tables_out, int32_t* lens_out);

/* Blocks a request can take: free ones plus evictable cache entries. */
int64_t pa_alloc_num_free(const pa_alloc* a);
/* Reference count of a physical block (-1 for an out-of-range id). */
int32_t pa_alloc_refcount(const pa_alloc* a, int64_t block);
/* Length / number of blocks of a sequence (-1 if unknown). */
int32_t pa_alloc_seq_len(const pa_alloc* a, int64_t seq_id);
int32_t pa_alloc_seq_num_blocks(const pa_alloc* a, int64_t seq_id);

/* ------------------------------------------------------------------------
 * Automatic prefix caching (zhy-blog.vercel.app, vLLM post, section 2.2 (5)
 * "自动前缀缓存": every cached block sits in one table under a hash of its
 * own tokens and all tokens before it; a new request looks its blocks up
 * and reuses the ones found.  wq-win.github.io "079 | vLLM 与 PagedAttention",
 * self-test question 2: only the same prefix under the same conditions may
 * share K/V.)
 *
 * Rules (readings of the pages where they are silent):
 *  - Only full blocks are cached.  Block i of a sequence whose tokens are
 *    known is identified by d_i = pa_prefix_block_hash(d_{i-1}, salt, its BS
 *    tokens), d_{-1} = NULL: a chain over (salt, tokens 0 .. (i+1)*BS - 1).
 *    The salt stands for "the same conditions" (model, adapter, ...).
 *  - A block enters the table when it becomes full (at pa_alloc_add_seq_tokens
 *    for the prompt's full blocks, at pa_alloc_append_tokens for a block the
 *    new tokens fill), unless its prefix already has an entry.  The caller
 *    must write the K/V of every slot it reserved (pa_reshape_and_cache)
 *    before any other sequence can read it, i.e. within the same iteration.
 *  - A request reuses the longest run of its leading full blocks that have
 *    entries (one more reference each) and stops at the first that has none.
 *  - An entry whose count drops to 0 stays in the table, evictable.  Free
 *    blocks are taken first; when none is left, the evictable entry released
 *    longest ago is evicted (least recently used) and its block reused.
 * Sequences made by pa_alloc_add_seq, and any sequence after a plain
 * pa_alloc_append, have unknown tokens and add nothing to the table.  Table
 * memory (about 50 bytes per block) is allocated on the first call that
 * needs it.
 * ---------------------------------------------------------------------- */

/* New sequence whose prompt is tokens[0 .. num_tokens-1].  On success
 * *num_cached_out = the number of leading tokens whose K/V already sits in
 * reused blocks (a multiple of BS, possibly num_tokens): the caller computes
 * and writes only the positions from there on.  All or nothing on
 * PA_ENOMEM; PA_ENOENT if seq_id is taken. */
pa_status pa_alloc_add_seq_tokens(pa_alloc* a, int64_t seq_id, const int32_t* tokens,
                                  int32_t num_tokens, uint64_t salt, int32_t* num_cached_out);

/* pa_alloc_append for known tokens (same slots, copy-on-write pair and
 * errors); blocks the tokens fill enter the table. */
pa_status pa_alloc_append_tokens(pa_alloc* a, int64_t seq_id, const int32_t* tokens,
                                 int32_t n_tokens, int64_t* slots_out, int64_t* cow_pairs_out,
                                 int32_t* n_cow_out);

/* Entries in the table (in use or evictable), and evictable entries alone. */
int64_t pa_alloc_num_cached(const pa_alloc* a);
int64_t pa_alloc_num_evictable(const pa_alloc* a);

/* Forget every entry; evictable blocks return to the free list, oldest
 * release first (so the most recent is taken first). */
pa_status pa_alloc_reset_prefix_cache(pa_alloc* a);

/* The block identity: SHA-256 (FIPS 180-4) of parent (32 bytes; NULL = 32
 * zero bytes) | salt (8 bytes, little-endian) | each token (4 bytes, little-
 * endian), written to digest_out[0..31].  Exposed so that a caller can key
 * its own structures (e.g. route requests by prefix) the same way. */
pa_status pa_prefix_block_hash(const uint8_t* parent, uint64_t salt, const int32_t* tokens,
                               int32_t num_tokens, uint8_t* digest_out);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
