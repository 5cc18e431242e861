// Host-side ref-counted KV block allocator (pa_alloc_* in include/pa.h).
//
// Follows the block management the pages describe:
//  - gitcode.csdn.net "vLLM 推理引擎：PagedAttention 与 KVCache 管理",
//    section 1: a physical block has an id, a size and a reference count;
//    a block table maps logical to physical blocks, -1 when absent.
//  - deepinsea.top "PagedAttention 内存管理深度解析", "分页机制设计": a free
//    list popped from its end; ceil(tokens / block_size) blocks per request;
//    the free count is checked first so a failed request takes nothing.
//  - wq-win.github.io "079 | vLLM 与 PagedAttention", section 二 (sharing and
//    copy-on-write of a shared tail block, reclaim only at count zero) and
//    section 三 (per iteration: release finished sequences, give a sequence
//    a new block only when its next token crosses a block boundary, copy a
//    shared tail block before writing into it).
//
// Automatic prefix caching (zhy-blog.vercel.app vLLM post, section 2.2 (5);
// wq-win.github.io self-test question 2): a full block of a sequence whose
// tokens are known enters one table under the identity of its whole prefix
// (salt, tokens 0 .. end of the block), and a new request reuses the longest
// run of its leading full blocks found there.  The identity is a SHA-256
// chain, d_i = SHA-256(d_{i-1} | salt | tokens of block i) with d_{-1} = 0, so
// equal digests mean equal prefixes (short of a SHA-256 collision) and a
// lookup costs one block's worth of hashing, whatever the prefix length.
// Released entries stay in the table at count 0 (evictable) and are reused
// by later requests; free blocks are taken first and then the entry released
// longest ago is evicted.  A sequence is released from its last block to its
// first, so the deepest (least shared) blocks of a prefix go first.
#include <algorithm>
#include <array>
#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"
#include "sha256.h"

using Digest = std::array<uint8_t, 32>;

struct pa_alloc {
  int32_t block_size;
  std::vector<int32_t> free_list;  // LIFO: taken from / returned to the back
  std::vector<int32_t> ref;        // reference count per physical block
  struct Seq {
    std::vector<int32_t> blocks;
    int32_t len;
    // prefix caching: tokens known since the sequence was added
    bool tracked = false;
    uint64_t salt = 0;
    bool has_last = false;
    Digest last{};               // digest of the last full block
    std::vector<int32_t> tail;   // tokens of the partially filled block
    std::vector<int32_t> entered;  // blocks this sequence entered into the table
  };
  std::unordered_map<int64_t, Seq> seqs;

  // Prefix cache, allocated on first use.  table: open addressing with
  // linear probing over block ids (-1 empty), keyed by digest[b]; lru: the
  // entries at count 0, a doubly linked list through prev / next, oldest
  // release at the head.
  bool cache_ready = false;
  std::vector<Digest> digest;
  std::vector<uint8_t> is_entry;
  std::vector<int32_t> table;
  uint64_t mask = 0;
  int64_t n_entries = 0;
  std::vector<int32_t> prev, next;
  int32_t head = -1, tail_ = -1;
  int64_t n_evictable = 0;
  std::vector<Digest> scratch;  // per-request digests

  bool ensure_cache() {
    if (cache_ready) return true;
    try {
      const size_t nb = ref.size();
      size_t cap = 16;
      while (cap < 2 * nb) cap *= 2;
      digest.assign(nb, Digest{});
      is_entry.assign(nb, 0);
      table.assign(cap, -1);
      prev.assign(nb, -1);
      next.assign(nb, -1);
      mask = cap - 1;
    } catch (...) {
      digest.clear();
      is_entry.clear();
      table.clear();
      prev.clear();
      next.clear();
      return false;
    }
    cache_ready = true;
    return true;
  }

  uint64_t home(const Digest& d) const {
    uint64_t x;
    std::memcpy(&x, d.data(), 8);
    return x & mask;
  }
  int32_t find(const Digest& d) const {
    for (uint64_t i = home(d);; i = (i + 1) & mask) {
      const int32_t b = table[i];
      if (b < 0 || digest[b] == d) return b;
    }
  }
  void insert(int32_t b, const Digest& d) {
    digest[b] = d;
    is_entry[b] = 1;
    uint64_t i = home(d);
    while (table[i] >= 0) i = (i + 1) & mask;
    table[i] = b;
    ++n_entries;
  }
  void erase(int32_t b) {  // backward-shift deletion keeps probe runs intact
    uint64_t i = home(digest[b]);
    while (table[i] != b) i = (i + 1) & mask;
    for (uint64_t j = (i + 1) & mask; table[j] >= 0; j = (j + 1) & mask) {
      const uint64_t k = home(digest[table[j]]);
      // move table[j] back to the hole at i unless its home lies in (i, j]
      const bool in_range = i <= j ? (k > i && k <= j) : (k > i || k <= j);
      if (!in_range) {
        table[i] = table[j];
        i = j;
      }
    }
    table[i] = -1;
    is_entry[b] = 0;
    --n_entries;
  }
  void lru_push(int32_t b) {
    prev[b] = tail_;
    next[b] = -1;
    if (tail_ >= 0) next[tail_] = b; else head = b;
    tail_ = b;
    ++n_evictable;
  }
  void lru_remove(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else tail_ = prev[b];
    prev[b] = next[b] = -1;
    --n_evictable;
  }

  int64_t available() const { return (int64_t)free_list.size() + n_evictable; }

  int32_t take() {
    int32_t b;
    if (!free_list.empty()) {
      b = free_list.back();
      free_list.pop_back();
    } else {  // evict the entry released longest ago
      b = head;
      lru_remove(b);
      erase(b);
    }
    ref[b] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--ref[b] == 0) {
      if (cache_ready && is_entry[b]) lru_push(b); else free_list.push_back(b);
    }
  }
  void revive(int32_t b) {
    if (ref[b] == 0) lru_remove(b);
    ++ref[b];
  }
  // the block b has just become full with digest d: it enters the table
  // unless that prefix already has an entry (returns whether it did)
  bool offer(int32_t b, const Digest& d) {
    if (find(d) >= 0) return false;
    insert(b, d);
    return true;
  }
  int64_t blocks_for(int64_t n) const { return (n + block_size - 1) / block_size; }
};

namespace {

// splitmix64 (Steele, Lea, Flood 2014): a small seeded generator for the
// one-off shuffle of physical ids.
uint64_t splitmix64(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

Digest block_digest(const Digest* parent, uint64_t salt, const int32_t* tokens, int64_t n) {
  pa::Sha256 h;
  // the message: parent | salt (little-endian) | tokens (little-endian),
  // serialised a chunk at a time
  uint8_t b[1024];
  if (parent) std::memcpy(b, parent->data(), 32); else std::memset(b, 0, 32);
  for (int i = 0; i < 8; ++i) b[32 + i] = (uint8_t)(salt >> (8 * i));
  size_t len = 40;
  for (int64_t t = 0; t < n; ++t) {
    const uint32_t v = (uint32_t)tokens[t];
    for (int i = 0; i < 4; ++i) b[len + i] = (uint8_t)(v >> (8 * i));
    len += 4;
    if (len == sizeof b) {
      h.update(b, len);
      len = 0;
    }
  }
  h.update(b, len);
  return h.finish();
}

// Reserve slots for n_tokens more tokens of s (the copy-on-write and
// block-boundary rules of pa_alloc_append).
pa_status append_slots(pa_alloc* a, pa_alloc::Seq& s, int32_t n_tokens, int64_t* slots_out,
                       int64_t* cow_pairs_out, int32_t* n_cow_out) {
  const int32_t bs = a->block_size;
  const int64_t new_len = (int64_t)s.len + n_tokens;
  if (new_len > INT32_MAX) return PA_EINVAL;
  const int64_t need_new = a->blocks_for(new_len) - (int64_t)s.blocks.size();
  const bool cow = n_tokens > 0 && s.len % bs != 0 && a->ref[s.blocks.back()] > 1;
  if (cow && !cow_pairs_out) return PA_EINVAL;
  if (need_new + (cow ? 1 : 0) > a->available()) return PA_ENOMEM;
  try {
    s.blocks.reserve((size_t)a->blocks_for(new_len));
  } catch (...) {
    return PA_ENOMEM;
  }
  *n_cow_out = 0;
  if (cow) {
    const int32_t old = s.blocks.back();
    const int32_t fresh = a->take();
    a->drop(old);
    s.blocks.back() = fresh;
    cow_pairs_out[0] = old;
    cow_pairs_out[1] = fresh;
    *n_cow_out = 1;
  }
  for (int64_t pos = s.len; pos < new_len; ++pos) {
    const int64_t lb = pos / bs;
    if (lb == (int64_t)s.blocks.size()) s.blocks.push_back(a->take());
    slots_out[pos - s.len] = (int64_t)s.blocks[(size_t)lb] * bs + pos % bs;
  }
  s.len = (int32_t)new_len;
  return PA_OK;
}

}  // namespace

extern "C" {

pa_alloc* pa_alloc_create(int64_t num_blocks, int32_t block_size, uint64_t shuffle_seed) {
  if (num_blocks <= 0 || num_blocks > INT32_MAX || block_size <= 0) return nullptr;
  pa_alloc* a = new (std::nothrow) pa_alloc();
  if (!a) return nullptr;
  try {
    a->block_size = block_size;
    a->ref.assign((size_t)num_blocks, 0);
    a->free_list.resize((size_t)num_blocks);
    for (int64_t i = 0; i < num_blocks; ++i) a->free_list[(size_t)i] = (int32_t)i;
    if (shuffle_seed != 0) {  // Fisher-Yates
      uint64_t st = shuffle_seed;
      for (int64_t i = num_blocks - 1; i > 0; --i) {
        const int64_t j = (int64_t)(splitmix64(st) % (uint64_t)(i + 1));
        std::swap(a->free_list[(size_t)i], a->free_list[(size_t)j]);
      }
    }
  } catch (...) {
    delete a;
    return nullptr;
  }
  return a;
}

void pa_alloc_destroy(pa_alloc* a) { delete a; }

pa_status pa_alloc_add_seq(pa_alloc* a, int64_t seq_id, int32_t num_tokens) {
  if (!a || num_tokens < 0) return PA_EINVAL;
  if (a->seqs.count(seq_id)) return PA_ENOENT;
  const int64_t need = a->blocks_for(num_tokens);
  if (need > a->available()) return PA_ENOMEM;
  pa_alloc::Seq* s;
  try {  // everything that can throw comes before the first block is taken
    s = &a->seqs.emplace(seq_id, pa_alloc::Seq()).first->second;
    s->blocks.reserve((size_t)need);
  } catch (...) {
    a->seqs.erase(seq_id);
    return PA_ENOMEM;
  }
  s->len = num_tokens;
  for (int64_t i = 0; i < need; ++i) s->blocks.push_back(a->take());
  return PA_OK;
}

pa_status pa_alloc_fork(pa_alloc* a, int64_t parent_id, int64_t child_id) {
  if (!a) return PA_EINVAL;
  auto it = a->seqs.find(parent_id);
  if (it == a->seqs.end() || a->seqs.count(child_id)) return PA_ENOENT;
  try {
    pa_alloc::Seq child = it->second;
    child.entered.clear();  // entries belong to the sequence that created them
    if (child.tracked) child.tail.reserve((size_t)a->block_size);
    a->seqs.emplace(child_id, std::move(child));
  } catch (...) {
    a->seqs.erase(child_id);
    return PA_ENOMEM;
  }
  for (int32_t b : a->seqs.find(child_id)->second.blocks) ++a->ref[b];
  return PA_OK;
}

pa_status pa_alloc_append(pa_alloc* a, int64_t seq_id, int32_t n_tokens, int64_t* slots_out,
                          int64_t* cow_pairs_out, int32_t* n_cow_out) {
  if (!a || n_tokens < 0 || (n_tokens > 0 && !slots_out) || !n_cow_out) return PA_EINVAL;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PA_ENOENT;
  const pa_status st = append_slots(a, it->second, n_tokens, slots_out, cow_pairs_out, n_cow_out);
  if (st == PA_OK) {  // tokens unknown from here on: nothing more of it is cached
    it->second.tracked = false;
    std::vector<int32_t>().swap(it->second.tail);
  }
  return st;
}

pa_status pa_alloc_append_batch(pa_alloc* a, const int64_t* seq_ids, const int32_t* n_tokens,
                                int32_t n, int64_t* slots_out, int64_t* cow_pairs_out,
                                int32_t* n_cow_out, int32_t* n_done_out) {
  if (!a || n < 0 || (n > 0 && (!seq_ids || !n_tokens)) || !n_cow_out || !n_done_out)
    return PA_EINVAL;
  *n_cow_out = 0;
  *n_done_out = 0;
  int64_t total = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (n_tokens[i] < 0) return PA_EINVAL;
    total += n_tokens[i];
  }
  if (total > 0 && !slots_out) return PA_EINVAL;
  int64_t at = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t ncow = 0;
    const pa_status st =
        pa_alloc_append(a, seq_ids[i], n_tokens[i], n_tokens[i] > 0 ? slots_out + at : nullptr,
                        cow_pairs_out ? cow_pairs_out + 2 * (int64_t)*n_cow_out : nullptr, &ncow);
    if (st != PA_OK) return st;  // this sequence untouched (pa_alloc_append is all or nothing)
    *n_cow_out += ncow;
    at += n_tokens[i];
    *n_done_out = i + 1;
  }
  return PA_OK;
}

pa_status pa_alloc_add_seq_tokens(pa_alloc* a, int64_t seq_id, const int32_t* tokens,
                                  int32_t num_tokens, uint64_t salt, int32_t* num_cached_out) {
  if (!a || num_tokens < 0 || (num_tokens > 0 && !tokens) || !num_cached_out) return PA_EINVAL;
  if (a->seqs.count(seq_id)) return PA_ENOENT;
  if (!a->ensure_cache()) return PA_ENOMEM;
  const int32_t bs = a->block_size;
  const int64_t nfull = num_tokens / bs, nblocks = a->blocks_for(num_tokens);
  pa_alloc::Seq s;
  try {
    a->scratch.resize((size_t)nfull);
    s.blocks.reserve((size_t)nblocks);
    s.tail.reserve((size_t)bs);
    s.entered.reserve((size_t)nfull);
  } catch (...) {
    return PA_ENOMEM;
  }
  // digests of the full blocks; the hits are the longest run of leading
  // blocks whose digest is in the table
  int64_t hits = 0, revived = 0;
  bool hitting = true;
  for (int64_t i = 0; i < nfull; ++i) {
    a->scratch[(size_t)i] =
        block_digest(i ? &a->scratch[(size_t)i - 1] : nullptr, salt, tokens + i * bs, bs);
    if (hitting) {
      const int32_t b = a->find(a->scratch[(size_t)i]);
      if (b < 0) {
        hitting = false;
      } else {
        s.blocks.push_back(b);
        revived += a->ref[b] == 0;
        ++hits;
      }
    }
  }
  if (nblocks - hits > a->available() - revived) return PA_ENOMEM;
  try {
    a->seqs.emplace(seq_id, pa_alloc::Seq());
  } catch (...) {
    return PA_ENOMEM;
  }
  for (int32_t b : s.blocks) a->revive(b);
  for (int64_t i = hits; i < nblocks; ++i) {
    const int32_t b = a->take();
    s.blocks.push_back(b);
    if (i < nfull && a->offer(b, a->scratch[(size_t)i])) s.entered.push_back(b);
  }
  s.len = num_tokens;
  s.tracked = true;
  s.salt = salt;
  s.has_last = nfull > 0;
  if (nfull > 0) s.last = a->scratch[(size_t)nfull - 1];
  s.tail.assign(tokens + nfull * bs, tokens + num_tokens);
  a->seqs[seq_id] = std::move(s);
  *num_cached_out = (int32_t)(hits * bs);
  return PA_OK;
}

pa_status pa_alloc_append_tokens(pa_alloc* a, int64_t seq_id, const int32_t* tokens,
                                 int32_t n_tokens, int64_t* slots_out, int64_t* cow_pairs_out,
                                 int32_t* n_cow_out) {
  if (!a || n_tokens < 0 || (n_tokens > 0 && (!slots_out || !tokens)) || !n_cow_out)
    return PA_EINVAL;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PA_ENOENT;
  pa_alloc::Seq& s = it->second;
  const int64_t L = s.len;
  const pa_status st = append_slots(a, s, n_tokens, slots_out, cow_pairs_out, n_cow_out);
  if (st != PA_OK || !s.tracked) return st;
  const int32_t bs = a->block_size;
  for (int32_t t = 0; t < n_tokens; ++t) {  // tail has capacity bs: no allocation
    s.tail.push_back(tokens[t]);
    if ((int32_t)s.tail.size() == bs) {
      s.last = block_digest(s.has_last ? &s.last : nullptr, s.salt, s.tail.data(), bs);
      s.has_last = true;
      s.tail.clear();
      const int32_t b = s.blocks[(size_t)((L + t) / bs)];
      if (a->offer(b, s.last)) {
        try {
          s.entered.push_back(b);
        } catch (...) {  // cannot record it: keep the block out of the table instead
          a->erase(b);
        }
      }
    }
  }
  return PA_OK;
}

pa_status pa_alloc_free_seq(pa_alloc* a, int64_t seq_id) {
  if (!a) return PA_EINVAL;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PA_ENOENT;
  const std::vector<int32_t>& blocks = it->second.blocks;
  for (size_t i = blocks.size(); i-- > 0;) a->drop(blocks[i]);
  a->seqs.erase(it);
  return PA_OK;
}

pa_status pa_alloc_discard_seq(pa_alloc* a, int64_t seq_id) {
  if (!a) return PA_EINVAL;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PA_ENOENT;
  // the sequence still references every block it entered, so none of them
  // can have been evicted and re-entered by another sequence meanwhile
  for (int32_t b : it->second.entered)
    if (a->cache_ready && a->is_entry[b]) a->erase(b);
  return pa_alloc_free_seq(a, seq_id);
}

pa_status pa_alloc_share_groups(const pa_alloc* a, const int64_t* seq_ids, int32_t n,
                                int32_t max_members, int32_t* group_start_out,
                                int32_t* group_prefix_out, int32_t* num_groups_out) {
  if (!a || n < 0 || max_members < 1 || !num_groups_out || !group_start_out ||
      (n > 0 && (!seq_ids || !group_prefix_out)))
    return PA_EINVAL;
  std::vector<const pa_alloc::Seq*> seqs((size_t)n);
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return PA_ENOENT;
    seqs[(size_t)i] = &it->second;
  }
  const int32_t bs = a->block_size;
  // leading blocks two sequences hold in common and that are full in both
  auto common = [bs](const pa_alloc::Seq& x, const pa_alloc::Seq& y) {
    const size_t full = (size_t)(std::min(x.len, y.len) / bs);
    size_t j = 0;
    while (j < full && x.blocks[j] == y.blocks[j]) ++j;
    return (int32_t)j;
  };
  int32_t g = 0;
  for (int32_t i = 0; i < n;) {
    // group g starts at i; a later sequence joins while it shares the
    // group's whole prefix with the first member (the first joiner sets it)
    group_start_out[g] = i;
    int32_t prefix = 0, j = i + 1;
    for (; j < n && j - i < max_members; ++j) {
      const int32_t c = common(*seqs[(size_t)i], *seqs[(size_t)j]);
      if (c == 0 || (j > i + 1 && c < prefix)) break;
      if (j == i + 1) prefix = c;
    }
    group_prefix_out[g] = prefix * bs;
    ++g;
    i = j;
  }
  group_start_out[g] = n;
  *num_groups_out = g;
  return PA_OK;
}

pa_status pa_alloc_block_tables(const pa_alloc* a, const int64_t* seq_ids, int32_t n,
                                int32_t max_blocks, int32_t* tables_out, int32_t* lens_out) {
  if (!a || n < 0 || max_blocks < 0 || (n > 0 && (!seq_ids || !lens_out))) return PA_EINVAL;
  if (n > 0 && max_blocks > 0 && !tables_out) return PA_EINVAL;
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return PA_ENOENT;
    if ((int64_t)it->second.blocks.size() > max_blocks) return PA_EINVAL;
  }
  for (int32_t i = 0; i < n; ++i) {
    const pa_alloc::Seq& s = a->seqs.find(seq_ids[i])->second;
    int32_t* row = tables_out + (int64_t)i * max_blocks;
    int32_t j = 0;
    for (; j < (int32_t)s.blocks.size(); ++j) row[j] = s.blocks[(size_t)j];
    for (; j < max_blocks; ++j) row[j] = -1;
    lens_out[i] = s.len;
  }
  return PA_OK;
}

int64_t pa_alloc_num_free(const pa_alloc* a) { return a ? a->available() : -1; }

int64_t pa_alloc_num_cached(const pa_alloc* a) { return a ? a->n_entries : -1; }

int64_t pa_alloc_num_evictable(const pa_alloc* a) { return a ? a->n_evictable : -1; }

pa_status pa_alloc_reset_prefix_cache(pa_alloc* a) {
  if (!a) return PA_EINVAL;
  if (!a->cache_ready) return PA_OK;
  try {
    a->free_list.reserve(a->free_list.size() + (size_t)a->n_evictable);
  } catch (...) {
    return PA_ENOMEM;
  }
  for (int32_t b = a->head; b >= 0;) {
    const int32_t nx = a->next[b];
    a->prev[b] = a->next[b] = -1;
    a->free_list.push_back(b);
    b = nx;
  }
  a->head = a->tail_ = -1;
  a->n_evictable = 0;
  std::fill(a->table.begin(), a->table.end(), -1);
  std::fill(a->is_entry.begin(), a->is_entry.end(), 0);
  a->n_entries = 0;
  return PA_OK;
}

pa_status pa_prefix_block_hash(const uint8_t* parent, uint64_t salt, const int32_t* tokens,
                               int32_t num_tokens, uint8_t* digest_out) {
  if (num_tokens < 0 || (num_tokens > 0 && !tokens) || !digest_out) return PA_EINVAL;
  Digest p;
  if (parent) std::memcpy(p.data(), parent, 32);
  const Digest d = block_digest(parent ? &p : nullptr, salt, tokens, num_tokens);
  std::memcpy(digest_out, d.data(), 32);
  return PA_OK;
}

int32_t pa_alloc_refcount(const pa_alloc* a, int64_t block) {
  if (!a || block < 0 || block >= (int64_t)a->ref.size()) return -1;
  return a->ref[(size_t)block];
}

int32_t pa_alloc_seq_len(const pa_alloc* a, int64_t seq_id) {
  if (!a) return -1;
  auto it = a->seqs.find(seq_id);
  return it == a->seqs.end() ? -1 : it->second.len;
}

int32_t pa_alloc_seq_num_blocks(const pa_alloc* a, int64_t seq_id) {
  if (!a) return -1;
  auto it = a->seqs.find(seq_id);
  return it == a->seqs.end() ? -1 : (int32_t)it->second.blocks.size();
}

}  // extern "C"
