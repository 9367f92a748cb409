// Host-side block bookkeeping of the paged KV cache: free list, reference
// counts, on-demand growth and the prefix cache (froggydisk "LLM에서 KV 캐시는
// 얼마나 생길까", section "KV 캐시를 줄이는 기법", PagedAttention and
// prefix-cache paragraphs).  Plain C++17, no HIP.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <list>
#include <new>
#include <set>
#include <unordered_map>
#include <vector>

#include "kvblocks.h"

namespace {

constexpr int32_t kBlock = 16;

// Lookup key of a full block: hash of every token before it, and its own tokens.
struct Key {
  uint64_t prefix;
  int32_t tok[kBlock];
  bool operator==(const Key& o) const {
    return prefix == o.prefix && std::memcmp(tok, o.tok, sizeof tok) == 0;
  }
};

// The SplitMix64 output function (Steele, Lea and Flood, "Fast splittable
// pseudorandom number generators", OOPSLA 2014; the published constants):
// a bijective 64-bit mix.
inline uint64_t mix64(uint64_t x) {
  x ^= x >> 30;
  x *= 0xBF58476D1CE4E5B9ull;
  x ^= x >> 27;
  x *= 0x94D049BB133111EBull;
  x ^= x >> 31;
  return x;
}

// Hash of a prefix extended by one block of tokens.
inline uint64_t extend(uint64_t h, const int32_t* tok) {
  for (int r = 0; r < kBlock; ++r) h = mix64(h + 0x9E3779B97F4A7C15ull + (uint32_t)tok[r]);
  return h;
}

constexpr uint64_t kRoot = 0x6A09E667F3BCC909ull;   // hash of the empty prefix

struct KeyHash {
  size_t operator()(const Key& k) const { return (size_t)extend(k.prefix, k.tok); }
};

struct Sequence {
  std::vector<int32_t> blocks;
  std::vector<uint64_t> prefix;     // prefix[k]: hash of the tokens before block k (tracked sequences)
  std::vector<int32_t> tail;        // tokens of the partly filled last block
  int32_t len = 0;
  bool tracked = false;             // token ids known from the start
};

}  // namespace

struct kvd_block_manager {
  int32_t num_blocks = 0;
  bool prefix_cache = false;
  std::vector<int32_t> ref;
  std::set<int32_t> free;                                  // lowest id first
  std::list<int32_t> evictable;                            // least recently released first
  std::vector<std::list<int32_t>::iterator> evict_pos;
  std::vector<char> registered;
  std::vector<Key> key_of;
  std::unordered_map<Key, int32_t, KeyHash> cache;
  std::unordered_map<int64_t, Sequence> seqs;
  int64_t next_id = 0;

  int32_t available() const { return (int32_t)free.size() + (int32_t)evictable.size(); }

  int32_t take() {
    int32_t b;
    if (!free.empty()) {
      b = *free.begin();
      free.erase(free.begin());
    } else {
      b = evictable.front();
      evictable.pop_front();
      cache.erase(key_of[b]);
      registered[b] = 0;
    }
    ref[b] = 1;
    return b;
  }

  void release(int32_t b) {
    if (--ref[b] == 0) {
      if (registered[b]) {
        evictable.push_back(b);
        evict_pos[b] = std::prev(evictable.end());
      } else {
        free.insert(b);
      }
    }
  }

  void reuse(int32_t b) {
    if (ref[b] == 0) evictable.erase(evict_pos[b]);
    ++ref[b];
  }

  // Block k of s has just become full with tokens tok: record the hash of the
  // prefix after it and register it unless its prefix is cached already.
  void block_filled(Sequence& s, int32_t k, const int32_t* tok) {
    const uint64_t before = s.prefix[k];
    s.prefix.push_back(extend(before, tok));
    if (!prefix_cache) return;
    const int32_t b = s.blocks[k];
    if (registered[b]) return;
    Key key;
    key.prefix = before;
    std::memcpy(key.tok, tok, sizeof key.tok);
    if (cache.find(key) != cache.end()) return;
    cache.emplace(key, b);
    registered[b] = 1;
    key_of[b] = key;
  }

  const Sequence* find(int64_t id) const {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
};

extern "C" {

kvd_status kvd_bm_create(int32_t num_blocks, int32_t prefix_cache, kvd_block_manager** out) {
  if (!out || num_blocks < 1 || (prefix_cache != 0 && prefix_cache != 1)) return KVD_ERR_INVALID_ARG;
  try {
    auto* bm = new kvd_block_manager();
    bm->num_blocks = num_blocks;
    bm->prefix_cache = prefix_cache == 1;
    bm->ref.assign(num_blocks, 0);
    bm->evict_pos.resize(num_blocks);
    bm->registered.assign(num_blocks, 0);
    bm->key_of.resize(num_blocks);
    for (int32_t b = 0; b < num_blocks; ++b) bm->free.insert(bm->free.end(), b);
    *out = bm;
    return KVD_OK;
  } catch (const std::bad_alloc&) {
    return KVD_ERR_CAPACITY;
  }
}

kvd_status kvd_bm_destroy(kvd_block_manager* bm) {
  if (!bm) return KVD_ERR_INVALID_ARG;
  delete bm;
  return KVD_OK;
}

kvd_status kvd_bm_add_sequence(kvd_block_manager* bm, const int32_t* tokens, int32_t n_tokens,
                               int64_t* seq_id, int32_t* n_cached) {
  if (!bm || !seq_id || n_tokens < 0) return KVD_ERR_INVALID_ARG;
  try {
    const int32_t full = n_tokens / kBlock;
    // Match full blocks from the front up to the first miss.
    std::vector<int32_t> found;
    int32_t reusable = 0;
    if (bm->prefix_cache && tokens) {
      uint64_t h = kRoot;
      for (int32_t k = 0; k < full; ++k) {
        Key key;
        key.prefix = h;
        std::memcpy(key.tok, tokens + (size_t)k * kBlock, sizeof key.tok);
        auto it = bm->cache.find(key);
        if (it == bm->cache.end()) break;
        found.push_back(it->second);
        reusable += bm->ref[it->second] == 0;
        h = extend(h, key.tok);
      }
    }
    const int32_t need = (n_tokens + kBlock - 1) / kBlock - (int32_t)found.size();
    if (need > bm->available() - reusable) return KVD_ERR_CAPACITY;

    Sequence s;
    s.blocks.reserve(found.size() + need);
    s.tracked = tokens != nullptr;
    for (int32_t b : found) bm->reuse(b);
    s.blocks = found;
    for (int32_t k = 0; k < need; ++k) s.blocks.push_back(bm->take());
    s.len = n_tokens;
    if (s.tracked) {
      s.prefix.push_back(kRoot);
      for (int32_t k = 0; k < full; ++k) bm->block_filled(s, k, tokens + (size_t)k * kBlock);
      s.tail.assign(tokens + (size_t)full * kBlock, tokens + n_tokens);
    }
    const int64_t id = bm->next_id++;
    bm->seqs.emplace(id, std::move(s));
    *seq_id = id;
    if (n_cached) *n_cached = (int32_t)found.size() * kBlock;
    return KVD_OK;
  } catch (const std::bad_alloc&) {
    return KVD_ERR_CAPACITY;
  }
}

kvd_status kvd_bm_append(kvd_block_manager* bm, int64_t seq_id, const int32_t* tokens, int32_t n,
                         int32_t* slots) {
  if (!bm || n < 0 || (n > 0 && !slots)) return KVD_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return KVD_ERR_INVALID_ARG;
  Sequence& s = it->second;
  if ((int64_t)s.len + n > INT32_MAX - kBlock) return KVD_ERR_INVALID_ARG;
  try {
    const int32_t need = (s.len + n + kBlock - 1) / kBlock - (int32_t)s.blocks.size();
    if (need > bm->available()) return KVD_ERR_CAPACITY;
    s.blocks.reserve(s.blocks.size() + std::max(need, 0));
    for (int32_t k = 0; k < need; ++k) s.blocks.push_back(bm->take());
    if (s.tracked && !tokens) {
      s.tracked = false;
      s.tail.clear();
    }
    for (int32_t r = 0; r < n; ++r) {
      const int32_t t = s.len + r;
      slots[r] = s.blocks[t / kBlock] * kBlock + t % kBlock;
      if (s.tracked) {
        s.tail.push_back(tokens[r]);
        if ((int32_t)s.tail.size() == kBlock) {
          bm->block_filled(s, t / kBlock, s.tail.data());
          s.tail.clear();
        }
      }
    }
    s.len += n;
    return KVD_OK;
  } catch (const std::bad_alloc&) {
    return KVD_ERR_CAPACITY;
  }
}

kvd_status kvd_bm_slots(const kvd_block_manager* bm, int64_t seq_id, int32_t first, int32_t n,
                        int32_t* slots) {
  if (!bm || first < 0 || n < 0 || (n > 0 && !slots)) return KVD_ERR_INVALID_ARG;
  const Sequence* s = bm->find(seq_id);
  if (!s || (int64_t)first + n > s->len) return KVD_ERR_INVALID_ARG;
  for (int32_t r = 0; r < n; ++r) {
    const int32_t t = first + r;
    slots[r] = s->blocks[t / kBlock] * kBlock + t % kBlock;
  }
  return KVD_OK;
}

kvd_status kvd_bm_length(const kvd_block_manager* bm, int64_t seq_id, int32_t* length) {
  if (!bm || !length) return KVD_ERR_INVALID_ARG;
  const Sequence* s = bm->find(seq_id);
  if (!s) return KVD_ERR_INVALID_ARG;
  *length = s->len;
  return KVD_OK;
}

kvd_status kvd_bm_block_table(const kvd_block_manager* bm, int64_t seq_id, int32_t* table,
                              int32_t capacity, int32_t* n_blocks) {
  if (!bm || !n_blocks || capacity < 0) return KVD_ERR_INVALID_ARG;
  const Sequence* s = bm->find(seq_id);
  if (!s) return KVD_ERR_INVALID_ARG;
  const int32_t nb = (int32_t)s->blocks.size();
  *n_blocks = nb;
  if (nb > capacity || (nb > 0 && !table)) return KVD_ERR_INVALID_ARG;
  std::copy(s->blocks.begin(), s->blocks.end(), table);
  return KVD_OK;
}

kvd_status kvd_bm_fill_tables(const kvd_block_manager* bm, const int64_t* seq_ids, int32_t b,
                              int32_t* table, int32_t max_blocks, int32_t* context_lens) {
  if (!bm || b < 0 || max_blocks < 1) return KVD_ERR_INVALID_ARG;
  if (b == 0) return KVD_OK;
  if (!seq_ids || !table || !context_lens) return KVD_ERR_INVALID_ARG;
  for (int32_t i = 0; i < b; ++i) {
    const Sequence* s = bm->find(seq_ids[i]);
    if (!s || (int32_t)s->blocks.size() > max_blocks) return KVD_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < b; ++i) {
    const Sequence* s = bm->find(seq_ids[i]);
    int32_t* row = table + (size_t)i * max_blocks;
    std::fill(row, row + max_blocks, -1);
    std::copy(s->blocks.begin(), s->blocks.end(), row);
    context_lens[i] = s->len;
  }
  return KVD_OK;
}

kvd_status kvd_bm_free_sequence(kvd_block_manager* bm, int64_t seq_id) {
  if (!bm) return KVD_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return KVD_ERR_INVALID_ARG;
  const std::vector<int32_t>& blocks = it->second.blocks;
  for (auto b = blocks.rbegin(); b != blocks.rend(); ++b) bm->release(*b);
  bm->seqs.erase(it);
  return KVD_OK;
}

kvd_status kvd_bm_counts(const kvd_block_manager* bm, int32_t* free_blocks, int32_t* cached_blocks,
                         int32_t* used_blocks) {
  if (!bm) return KVD_ERR_INVALID_ARG;
  const int32_t f = (int32_t)bm->free.size(), c = (int32_t)bm->evictable.size();
  if (free_blocks) *free_blocks = f;
  if (cached_blocks) *cached_blocks = c;
  if (used_blocks) *used_blocks = bm->num_blocks - f - c;
  return KVD_OK;
}

kvd_status kvd_bm_refcount(const kvd_block_manager* bm, int32_t block, int32_t* refcount) {
  if (!bm || !refcount || block < 0 || block >= bm->num_blocks) return KVD_ERR_INVALID_ARG;
  *refcount = bm->ref[block];
  return KVD_OK;
}

}  // extern "C"
