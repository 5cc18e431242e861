/*
 * Reference oracle for paged decode attention and the two KV-cache ops.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no source with the HIP path: the pool
 * layout below is re-derived here from its written definition.
 *
 * Arithmetic is IEEE fp64 on the exact input values (fp16 / bf16 / fp32 are
 * widened exactly).  Everything is a direct transcription of the definitions;
 * nothing is blocked, fused or reordered.
 *
 * Sources (web pages on PagedAttention):
 *  [P5]  wq-win.github.io, "079 | vLLM 与 PagedAttention" -- digest of Kwon et
 *        al., SOSP 2023.  Section 二, part "分块以后，注意力仍需对整个历史归一化":
 *        the Z / o equations (one softmax denominator shared by all blocks,
 *        unfilled positions of the last block excluded, numerically stable
 *        evaluation required).
 *  [P1]  gitcode.csdn.net, "vLLM 推理引擎：PagedAttention 与 KVCache 管理",
 *        section 3 "PagedAttention 核心算法": forward(query, key_cache,
 *        value_cache, block_tables, context_lens): gather a sequence's blocks
 *        through its block table, keep the first context_len positions, then
 *        softmax(q k^T / sqrt(d)) v.
 *  [P4]  vkads.cloudxian.cn, "vLLM PagedAttention源码：KV Cache", kernel
 *        pseudocode: physical block b holds the flat slots b*BLOCK_SIZE ...
 *        (b+1)*BLOCK_SIZE-1.
 *
 * Readings where the pages are silent (each is also listed in the design
 * notes):
 *  - q-head h reads kv-head h / (Hq / Hkv) (contiguous GQA groups).
 *  - scale is passed by the caller (the pages use 1/sqrt(d_h)).
 *  - context_len 0 gives a zero output row.
 *  - a negative slot in the cache-write is padding and is skipped.
 *
 * Pool layout (the product's documented layout, re-implemented here):
 *   K element (blk, h, off, d)  at  (((blk*Hkv + h)*(D/X) + d/X)*BS + off)*X + d%X
 *   V element (blk, h, off, d)  at  (((blk*Hkv + h)*(BS/VS) + off/VS)*D + d)*VS + off%VS
 *   with X = 16 / element size (K is stored as 16-byte pieces of X dims, the
 *   pieces of all BS offsets for the same dims adjacent) and VS = min(BS, 8)
 *   (V is stored as 8-token slabs, each slab [D][VS]).  D must be a multiple
 *   of X.
 *
 * Parity status of each function: see the module docstring of the Python
 * wrapper; every function here is pinned by CPU tests.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0 /* >0 only in mutation tests: plants one known mistake */
#endif

static size_t elem_bytes(int dtype) { return dtype == OR_F32 ? 4 : 2; }

/* IEEE binary16 -> double, exact (sign, 5-bit exponent, 10-bit fraction). */
static double half_bits_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(f | 0x400), e - 25); /* (1024+f) * 2^(e-15-10) */
  return sign ? -v : v;
}

/* bfloat16 is the top half of an IEEE binary32. */
static double bf16_bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static double load_elem(const void* base, int dtype, int64_t i) {
  if (dtype == OR_F32) return (double)((const float*)base)[i];
  uint16_t bits = ((const uint16_t*)base)[i];
  return dtype == OR_F16 ? half_bits_to_double(bits) : bf16_bits_to_double(bits);
}

static int v_slab(int bs) { return bs < 8 ? bs : 8; }

/* Dims per 16-byte K piece. */
static int k_piece(int dtype) { return (int)(16 / elem_bytes(dtype)); }

static int64_t k_index(int64_t blk, int h, int off, int d, int hkv, int bs, int D, int x) {
  return (((blk * hkv + h) * (D / x) + d / x) * (int64_t)bs + off) * x + d % x;
}

static int64_t v_index(int64_t blk, int h, int off, int d, int hkv, int bs, int D) {
  int vs = v_slab(bs);
#if ORACLE_MUTANT == 7 /* mutant: V read as plain token-major rows */
  (void)vs;
  return ((blk * hkv + h) * bs + off) * (int64_t)D + d;
#else
  return (((blk * hkv + h) * (bs / vs) + off / vs) * (int64_t)D + d) * vs + off % vs;
#endif
}

typedef struct {
  double* out;
  const void *q, *kc, *vc;
  const int32_t *tables, *lens;
  double scale;
  int bs, hkv, B, hq, D, maxb, dtype;
  int64_t nblocks;
  int64_t item_begin, item_end; /* items are (seq, q-head) pairs */
  int status;
} decode_job;

/* One (sequence, q-head) output row: the Z / o equations of [P5] section 二,
 * evaluated as max-subtracted two-pass softmax (the stable form the same
 * passage asks for).  Positions u < L are gathered through the block table
 * (logical block u / BS, offset u % BS, [P1] section 3 and [P4]). */
static int decode_one(const decode_job* j, int b, int h, double* scores) {
  const int D = j->D, bs = j->bs;
  double* out = j->out + ((int64_t)b * j->hq + h) * D;
  int L = j->lens[b];
  int group = j->hq / j->hkv;
#if ORACLE_MUTANT == 3 /* mutant: wrong q-head -> kv-head map */
  int g = h % j->hkv;
#else
  int g = h / group;
#endif
  (void)group;
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  if (L <= 0) return 0;
#if ORACLE_MUTANT == 2 /* mutant: no tail mask, whole last block is attended */
  L = ((L + bs - 1) / bs) * bs;
#endif
  if ((L + bs - 1) / bs > j->maxb) return -1;
  const int64_t qrow = ((int64_t)b * j->hq + h) * D;

  for (int u = 0; u < L; ++u) {
#if ORACLE_MUTANT == 6 /* mutant: off-by-one logical block */
    int lb = (u + 1) / bs < (L + bs - 1) / bs ? (u + 1) / bs : u / bs;
#else
    int lb = u / bs;
#endif
    int64_t blk = j->tables[(int64_t)b * j->maxb + lb];
    if (blk < 0 || blk >= j->nblocks) return -1;
    double dot = 0.0;
    for (int d = 0; d < D; ++d) {
#if ORACLE_MUTANT == 4 /* mutant: K and V swapped */
      double kv = load_elem(j->vc, j->dtype, v_index(blk, g, u % bs, d, j->hkv, bs, D));
#else
      double kv = load_elem(j->kc, j->dtype, k_index(blk, g, u % bs, d, j->hkv, bs, D, k_piece(j->dtype)));
#endif
      dot += load_elem(j->q, j->dtype, qrow + d) * kv;
    }
#if ORACLE_MUTANT == 5 /* mutant: scale dropped */
    scores[u] = dot;
#else
    scores[u] = j->scale * dot;
#endif
  }

#if ORACLE_MUTANT == 1
  /* mutant: each block normalised on its own and the results added (the
   * counter-example the [P5] self-test rejects) */
  for (int start = 0; start < L; start += bs) {
    int end = start + bs < L ? start + bs : L;
    double m = -INFINITY, z = 0.0;
    for (int u = start; u < end; ++u) m = scores[u] > m ? scores[u] : m;
    for (int u = start; u < end; ++u) z += exp(scores[u] - m);
    for (int u = start; u < end; ++u) {
      int64_t blk = j->tables[(int64_t)b * j->maxb + u / bs];
      double w = exp(scores[u] - m) / z;
      for (int d = 0; d < D; ++d)
        out[d] += w * load_elem(j->vc, j->dtype, v_index(blk, g, u % bs, d, j->hkv, bs, D));
    }
  }
  return 0;
#else
  double m = -INFINITY;
  for (int u = 0; u < L; ++u) m = scores[u] > m ? scores[u] : m;
  double z = 0.0;
  for (int u = 0; u < L; ++u) {
    scores[u] = exp(scores[u] - m); /* weights now */
    z += scores[u];
  }
  for (int u = 0; u < L; ++u) {
    int64_t blk = j->tables[(int64_t)b * j->maxb + u / bs];
    for (int d = 0; d < D; ++d) {
#if ORACLE_MUTANT == 4
      double vv = load_elem(j->kc, j->dtype, k_index(blk, g, u % bs, d, j->hkv, bs, D, k_piece(j->dtype)));
#else
      double vv = load_elem(j->vc, j->dtype, v_index(blk, g, u % bs, d, j->hkv, bs, D));
#endif
      out[d] += scores[u] * vv;
    }
  }
  for (int d = 0; d < D; ++d) out[d] /= z;
  return 0;
#endif
}

static void* decode_worker(void* arg) {
  decode_job* j = (decode_job*)arg;
  double* scores = (double*)malloc(sizeof(double) * ((size_t)j->maxb * j->bs + 1));
  if (!scores) {
    j->status = -2;
    return NULL;
  }
  for (int64_t it = j->item_begin; it < j->item_end && j->status == 0; ++it) {
    int b = (int)(it / j->hq), h = (int)(it % j->hq);
    if (decode_one(j, b, h, scores) != 0) j->status = -1;
  }
  free(scores);
  return NULL;
}

/* Decode oracle.  out: [num_seqs][num_q_heads][head_dim] doubles.
 * q: [num_seqs][num_q_heads][head_dim] of dtype; pools in the layout above;
 * block_tables: [num_seqs][max_blocks_per_seq] int32; context_lens: [num_seqs].
 * Returns 0, or -1 on a malformed table / size, -2 on allocation failure. */
int oracle_decode(double* out, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, const int32_t* context_lens, double scale,
                  int block_size, int num_kv_heads, int num_seqs, int num_q_heads, int head_dim,
                  int max_blocks_per_seq, int64_t num_blocks, int dtype, int nthreads) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_q_heads % num_kv_heads != 0 || (block_size > 16 && block_size % 16 != 0) ||
      head_dim % k_piece(dtype) != 0)
    return -1;
  if (nthreads < 1) nthreads = 1;
  int64_t items = (int64_t)num_seqs * num_q_heads;
  if (items == 0) return 0;
  if (nthreads > items) nthreads = (int)items;
  decode_job* jobs = (decode_job*)calloc((size_t)nthreads, sizeof(decode_job));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !th) {
    free(jobs);
    free(th);
    return -2;
  }
  for (int t = 0; t < nthreads; ++t) {
    decode_job* j = &jobs[t];
    j->out = out;
    j->q = q;
    j->kc = k_cache;
    j->vc = v_cache;
    j->tables = block_tables;
    j->lens = context_lens;
    j->scale = scale;
    j->bs = block_size;
    j->hkv = num_kv_heads;
    j->B = num_seqs;
    j->hq = num_q_heads;
    j->D = head_dim;
    j->maxb = max_blocks_per_seq;
    j->dtype = dtype;
    j->nblocks = num_blocks;
    j->item_begin = items * t / nthreads;
    j->item_end = items * (t + 1) / nthreads;
  }
  for (int t = 1; t < nthreads; ++t)
    if (pthread_create(&th[t], NULL, decode_worker, &jobs[t]) != 0) jobs[t].status = -3;
  decode_worker(&jobs[0]);
  int rc = 0;
  for (int t = 1; t < nthreads; ++t) {
    if (jobs[t].status == -3) {
      jobs[t].status = 0; /* thread could not start: run its items here */
      decode_worker(&jobs[t]);
    } else {
      pthread_join(th[t], NULL);
    }
  }
  for (int t = 0; t < nthreads; ++t)
    if (jobs[t].status != 0) rc = jobs[t].status == -2 ? -2 : -1;
  free(jobs);
  free(th);
  return rc;
}

/* Chunked-prefill oracle (zhy-blog.vercel.app vLLM post, section 4.2 "Chunked
 * Prefill的解决方案": a prompt is processed in chunks, each chunk attends to the
 * KV cache its predecessors wrote, and its attention mask follows the chunk's
 * position in the whole prompt; query rows as in the forward of [P1] section 3,
 * [num_tokens][num_heads][head_size]).
 *
 * Sequence i owns query tokens query_start[i] .. query_start[i+1]-1; they are
 * the last ql_i tokens of its context, so token t sits at position
 * p = L_i - ql_i + (t - query_start[i]) with L_i = context_lens[i] (their K/V
 * are already in the pools).  Token t, q-head h attends causally to positions
 * 0 .. p through the block table, one softmax over all of them (the Z / o
 * equations of [P5] section 二 restricted to u <= p), two-pass max-subtracted
 * form.  out: [num_tokens][num_q_heads][head_dim] doubles.  Returns 0, or -1
 * on a malformed size / table. */
static int prefill_one(const void* q, const void* kc, const void* vc, const int32_t* tables,
                       double scale, int bs, int hkv, int hq, int D, int maxb, int64_t nblocks,
                       int dtype, int64_t t, int last, int seq, int h, double* scores,
                       double* out) {
  int g = h / (hq / hkv);
  const int64_t qrow = (t * hq + h) * (int64_t)D;
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  if (last < 0) return 0;
  if (last / bs >= maxb) return -1;
  for (int u = 0; u <= last; ++u) {
    int64_t blk = tables[(int64_t)seq * maxb + u / bs];
    if (blk < 0 || blk >= nblocks) return -1;
    double dot = 0.0;
    for (int d = 0; d < D; ++d)
      dot += load_elem(q, dtype, qrow + d) *
             load_elem(kc, dtype, k_index(blk, g, u % bs, d, hkv, bs, D, k_piece(dtype)));
    scores[u] = scale * dot;
  }
  double m = -INFINITY;
  for (int u = 0; u <= last; ++u) m = scores[u] > m ? scores[u] : m;
  double z = 0.0;
  for (int u = 0; u <= last; ++u) {
    scores[u] = exp(scores[u] - m);
    z += scores[u];
  }
  for (int u = 0; u <= last; ++u) {
    int64_t blk = tables[(int64_t)seq * maxb + u / bs];
    for (int d = 0; d < D; ++d)
      out[d] += scores[u] * load_elem(vc, dtype, v_index(blk, g, u % bs, d, hkv, bs, D));
  }
  for (int d = 0; d < D; ++d) out[d] /= z;
  return 0;
}

int oracle_prefill(double* out, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* block_tables, const int32_t* context_lens,
                   const int32_t* query_start, double scale, int block_size, int num_kv_heads,
                   int num_seqs, int num_q_heads, int head_dim, int max_blocks_per_seq,
                   int64_t num_blocks, int dtype) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_q_heads % num_kv_heads != 0 || head_dim % k_piece(dtype) != 0)
    return -1;
  double* scores = (double*)malloc(sizeof(double) * ((size_t)max_blocks_per_seq * block_size + 1));
  if (!scores) return -2;
  int rc = 0;
  for (int i = 0; i < num_seqs && rc == 0; ++i) {
    int qs = query_start[i], ql = query_start[i + 1] - query_start[i], L = context_lens[i];
    if (ql < 0 || ql > L) {
      rc = -1;
      break;
    }
    for (int r = 0; r < ql && rc == 0; ++r) {
      int64_t t = (int64_t)qs + r;
      int pos = L - ql + r; /* the token's position in its sequence */
#if ORACLE_MUTANT == 8      /* mutant: no causal mask, every row sees the whole context */
      int last = L - 1;
#elif ORACLE_MUTANT == 9    /* mutant: causal mask off by one, own position excluded */
      int last = pos - 1;
#else
      int last = pos;
#endif
      for (int h = 0; h < num_q_heads && rc == 0; ++h)
        rc = prefill_one(q, k_cache, v_cache, block_tables, scale, block_size, num_kv_heads,
                         num_q_heads, head_dim, max_blocks_per_seq, num_blocks, dtype, t, last,
                         i, h, scores, out + (t * num_q_heads + h) * (int64_t)head_dim);
    }
  }
  free(scores);
  return rc;
}

/* Cache-write oracle: token t's K and V rows ([Hkv][D], token stride given in
 * elements) go to slot slot_mapping[t] = physical block * BS + offset ([P4]
 * pseudocode's flat slot numbering).  Bits are copied, no arithmetic.  A
 * negative slot is skipped.  Returns -1 for a slot beyond the pool. */
int oracle_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                             const int64_t* slot_mapping, int num_tokens, int64_t k_token_stride,
                             int64_t v_token_stride, int num_kv_heads, int head_dim, int block_size,
                             int64_t num_blocks, int dtype) {
  size_t es = elem_bytes(dtype);
  if (head_dim % k_piece(dtype) != 0) return -1;
  for (int t = 0; t < num_tokens; ++t) {
    int64_t slot = slot_mapping[t];
    if (slot < 0) continue;
    int64_t blk = slot / block_size;
    int off = (int)(slot % block_size);
    if (blk >= num_blocks) return -1;
    for (int h = 0; h < num_kv_heads; ++h)
      for (int d = 0; d < head_dim; ++d) {
        int64_t src_k = t * k_token_stride + (int64_t)h * head_dim + d;
        int64_t src_v = t * v_token_stride + (int64_t)h * head_dim + d;
        memcpy((char*)k_cache + es * k_index(blk, h, off, d, num_kv_heads, block_size, head_dim, k_piece(dtype)),
               (const char*)k + es * src_k, es);
        memcpy((char*)v_cache + es * v_index(blk, h, off, d, num_kv_heads, block_size, head_dim),
               (const char*)v + es * src_v, es);
      }
  }
  return 0;
}

/* Block-copy oracle for copy-on-write ([P5] section 二, "共享与写时复制"):
 * for each (src, dst) pair every element of block src is copied to block dst,
 * in both pools, in pair order.  Returns -1 for an id beyond the pool. */
int oracle_copy_blocks(void* k_cache, void* v_cache, const int64_t* src_dst_pairs, int num_pairs,
                       int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                       int dtype) {
  size_t es = elem_bytes(dtype);
  if (head_dim % k_piece(dtype) != 0) return -1;
  for (int p = 0; p < num_pairs; ++p) {
    int64_t src = src_dst_pairs[2 * p], dst = src_dst_pairs[2 * p + 1];
    if (src < 0 || dst < 0 || src >= num_blocks || dst >= num_blocks) return -1;
    for (int h = 0; h < num_kv_heads; ++h)
      for (int off = 0; off < block_size; ++off)
        for (int d = 0; d < head_dim; ++d) {
          int64_t ks = k_index(src, h, off, d, num_kv_heads, block_size, head_dim, k_piece(dtype));
          int64_t kd = k_index(dst, h, off, d, num_kv_heads, block_size, head_dim, k_piece(dtype));
          int64_t vs = v_index(src, h, off, d, num_kv_heads, block_size, head_dim);
          int64_t vd = v_index(dst, h, off, d, num_kv_heads, block_size, head_dim);
          memcpy((char*)k_cache + es * kd, (const char*)k_cache + es * ks, es);
          memcpy((char*)v_cache + es * vd, (const char*)v_cache + es * vs, es);
        }
  }
  return 0;
}

/* Swap oracle (deepinsea.top "PagedAttention 内存管理深度解析", "Swap 机制"):
 * for each (src, dst) pair every element of block src of the source pools is
 * copied to block dst of the destination pools, in pair order.  Bits only.
 * Returns -1 for an id beyond its pool. */
int oracle_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                       const int64_t* src_dst_pairs, int num_pairs, int64_t src_blocks,
                       int64_t dst_blocks, int num_kv_heads, int head_dim, int block_size,
                       int dtype) {
  size_t es = elem_bytes(dtype);
  if (head_dim % k_piece(dtype) != 0) return -1;
  for (int p = 0; p < num_pairs; ++p) {
    int64_t src = src_dst_pairs[2 * p], dst = src_dst_pairs[2 * p + 1];
    if (src < 0 || dst < 0 || src >= src_blocks || dst >= dst_blocks) return -1;
    for (int h = 0; h < num_kv_heads; ++h)
      for (int off = 0; off < block_size; ++off)
        for (int d = 0; d < head_dim; ++d) {
          int64_t ks = k_index(src, h, off, d, num_kv_heads, block_size, head_dim, k_piece(dtype));
          int64_t kd = k_index(dst, h, off, d, num_kv_heads, block_size, head_dim, k_piece(dtype));
          int64_t vs = v_index(src, h, off, d, num_kv_heads, block_size, head_dim);
          int64_t vd = v_index(dst, h, off, d, num_kv_heads, block_size, head_dim);
          memcpy((char*)dst_k + es * kd, (const char*)src_k + es * ks, es);
          memcpy((char*)dst_v + es * vd, (const char*)src_v + es * vs, es);
        }
  }
  return 0;
}

/* Exposed so tests can check the widening against numpy's own fp16 decode. */
double oracle_half_to_double(uint16_t h) { return half_bits_to_double(h); }
double oracle_bf16_to_double(uint16_t b) { return bf16_bits_to_double(b); }
