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
#include <cstdint>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"

struct pa_alloc {
  int32_t block_size;
  std::vector<int32_t> free_list;  // LIFO: taken from / returned to the back
  std::vector<int32_t> ref;        // reference count per physical block
  struct Seq {
    std::vector<int32_t> blocks;
    int32_t len;
  };
  std::unordered_map<int64_t, Seq> seqs;

  int32_t take() {
    const int32_t b = free_list.back();
    free_list.pop_back();
    ref[b] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--ref[b] == 0) free_list.push_back(b);
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
  if (need > (int64_t)a->free_list.size()) return PA_ENOMEM;
  try {
    pa_alloc::Seq s;
    s.len = num_tokens;
    s.blocks.reserve((size_t)need);
    for (int64_t i = 0; i < need; ++i) s.blocks.push_back(a->take());
    a->seqs.emplace(seq_id, std::move(s));
  } catch (...) {
    return PA_ENOMEM;
  }
  return PA_OK;
}

pa_status pa_alloc_fork(pa_alloc* a, int64_t parent_id, int64_t child_id) {
  if (!a) return PA_EINVAL;
  auto it = a->seqs.find(parent_id);
  if (it == a->seqs.end() || a->seqs.count(child_id)) return PA_ENOENT;
  try {
    pa_alloc::Seq child = it->second;
    for (int32_t b : child.blocks) ++a->ref[b];
    a->seqs.emplace(child_id, std::move(child));
  } catch (...) {
    return PA_ENOMEM;
  }
  return PA_OK;
}

pa_status pa_alloc_append(pa_alloc* a, int64_t seq_id, int32_t n_tokens, int64_t* slots_out,
                          int64_t* cow_pairs_out, int32_t* n_cow_out) {
  if (!a || n_tokens < 0 || (n_tokens > 0 && !slots_out) || !n_cow_out) return PA_EINVAL;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PA_ENOENT;
  pa_alloc::Seq& s = it->second;
  const int32_t bs = a->block_size;
  const int64_t new_len = (int64_t)s.len + n_tokens;
  if (new_len > INT32_MAX) return PA_EINVAL;
  const int64_t need_new = a->blocks_for(new_len) - (int64_t)s.blocks.size();
  const bool cow = n_tokens > 0 && s.len % bs != 0 && a->ref[s.blocks.back()] > 1;
  if (cow && !cow_pairs_out) return PA_EINVAL;
  if (need_new + (cow ? 1 : 0) > (int64_t)a->free_list.size()) return PA_ENOMEM;
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

pa_status pa_alloc_free_seq(pa_alloc* a, int64_t seq_id) {
  if (!a) return PA_EINVAL;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PA_ENOENT;
  for (int32_t b : it->second.blocks) a->drop(b);
  a->seqs.erase(it);
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

int64_t pa_alloc_num_free(const pa_alloc* a) { return a ? (int64_t)a->free_list.size() : -1; }

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
