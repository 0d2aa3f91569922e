// Host-side block allocator: a free list of physical block ids, per-block
// reference counts and per-sequence block lists.  Produces block tables,
// context lengths and slots; never touches device memory.
//
// Paging semantics as on the vLLM page ("vLLM -- PagedAttention으로 LLM 추론 성능을
// 2~4배 끌어올린 서빙 엔진", section "PagedAttention -- OS 가상 메모리에서 영감":
// blocks taken only as tokens arrive, non-contiguous physical blocks behind a
// contiguous logical sequence, free blocks reusable by any request) and the
// Nano-vLLM page ("Nano-vLLM로 배우는 vLLM 추론 엔진 작동 원리 한눈에 정리",
// section "KV 캐시와 Block Manager": metadata on the CPU, shared prefix blocks
// found by hashing the blocks' tokens).
//
// Prefix caching: a full prompt block is registered under a hash chained over
// its tokens and every earlier block's, so a later prompt that starts with the
// same full blocks of tokens finds them and shares them.  A match is confirmed
// exactly (same tokens, same parent block in the same incarnation), so a hash
// collision can never share the wrong block.  A registered block whose last
// holder frees it keeps its K/V and stays findable: free blocks that hold
// nothing registered are handed out first, and registered ones only when no
// other block is free, least recently freed first (the block is then dropped
// from the registry before it is reused).
#include "pkv_alloc.h"

#include <algorithm>
#include <new>
#include <unordered_map>
#include <vector>

struct pkv_alloc {
  struct Seq {
    std::vector<int32_t> blocks;
    int32_t len = 0;
  };
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  // free blocks holding nothing registered; the next one handed out is
  // free_stack.back()
  std::vector<int32_t> free_stack;
  // free blocks still registered (their K/V still findable), least recently
  // freed at lru_head: a doubly linked list through lru_prev / lru_next (-1 ends)
  std::vector<int32_t> lru_prev, lru_next;
  int32_t lru_head = -1, lru_tail = -1, lru_size = 0;
  std::vector<int32_t> refcount;
  std::unordered_map<int64_t, Seq> seqs;
  // prefix registry: chained hash -> block; per block its hash (0: not
  // registered), parent block (-1: first block of a prompt), the parent's
  // incarnation when the block was registered, and tokens.  incarnation[b]
  // grows each time b is handed out, so a registered child whose parent block
  // was reused for other tokens can never be matched through it.
  std::unordered_map<uint64_t, int32_t> by_hash;
  std::vector<uint64_t> block_hash;
  std::vector<int32_t> block_parent;
  std::vector<uint32_t> parent_incarnation;
  std::vector<uint32_t> incarnation;
  std::vector<int32_t> block_tokens;

  int32_t num_free() const { return static_cast<int32_t>(free_stack.size()) + lru_size; }
  void lru_push(int32_t b) {
    lru_prev[b] = lru_tail;
    lru_next[b] = -1;
    (lru_tail >= 0 ? lru_next[lru_tail] : lru_head) = b;
    lru_tail = b;
    ++lru_size;
  }
  void lru_remove(int32_t b) {
    (lru_prev[b] >= 0 ? lru_next[lru_prev[b]] : lru_head) = lru_next[b];
    (lru_next[b] >= 0 ? lru_prev[lru_next[b]] : lru_tail) = lru_prev[b];
    lru_prev[b] = lru_next[b] = -1;
    --lru_size;
  }
  void unregister(int32_t b) {
    if (block_hash[b] == 0) return;
    auto it = by_hash.find(block_hash[b]);
    if (it != by_hash.end() && it->second == b) by_hash.erase(it);
    block_hash[b] = 0;
  }
  // A free block for new contents: an unregistered one if any, else the least
  // recently freed registered one, dropped from the registry.
  int32_t take() {
    int32_t b;
    if (!free_stack.empty()) {
      b = free_stack.back();
      free_stack.pop_back();
    } else {
      b = lru_head;
      lru_remove(b);
      unregister(b);
    }
    ++incarnation[b];
    refcount[b] = 1;
    return b;
  }
  // One more holder of block b, which may be a free registered block.
  void hold(int32_t b) {
    if (refcount[b]++ == 0) lru_remove(b);
  }
  void release(int32_t b) {
    if (--refcount[b] == 0) {
      if (block_hash[b] != 0)
        lru_push(b);
      else
        free_stack.push_back(b);
    }
  }
  int32_t blocks_for(int64_t tokens) const {
    return static_cast<int32_t>((tokens + block_size - 1) / block_size);
  }
};

namespace {

// SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014): the shuffle's random source.
uint64_t splitmix64(uint64_t& state) {
  uint64_t z = (state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// FNV-1a over the 32-bit tokens of one block, continuing from the previous
// block's hash (Fowler, Noll, Vo; 64-bit offset basis replaced by the chain
// value), then a SplitMix64 finaliser; never 0 (0 marks an unregistered block).
uint64_t chain_hash(uint64_t prev, const int32_t* tokens, int32_t n) {
  uint64_t h = prev ^ 0xcbf29ce484222325ull;
  for (int32_t i = 0; i < n; ++i) {
    const uint32_t t = static_cast<uint32_t>(tokens[i]);
    for (int k = 0; k < 4; ++k) {
      h ^= (t >> (8 * k)) & 0xffu;
      h *= 0x100000001b3ull;
    }
  }
  uint64_t s = h;
  uint64_t z = splitmix64(s);
#ifdef PKV_ALLOC_HASH_BITS
  // test builds only: a hash of a few bits, so that collisions are common and
  // the exact confirmation of every match is what keeps sharing correct
  z &= (uint64_t{1} << PKV_ALLOC_HASH_BITS) - 1;
#endif
  return z == 0 ? 1 : z;
}

}  // namespace

extern "C" {

pkv_alloc* pkv_alloc_create(int32_t num_blocks, int32_t block_size, uint64_t shuffle_seed) {
  if (num_blocks <= 0 || block_size <= 0) return nullptr;
  pkv_alloc* a = new (std::nothrow) pkv_alloc;
  if (!a) return nullptr;
  try {
    a->num_blocks = num_blocks;
    a->block_size = block_size;
    a->refcount.assign(num_blocks, 0);
    a->lru_prev.assign(num_blocks, -1);
    a->lru_next.assign(num_blocks, -1);
    a->block_hash.assign(num_blocks, 0);
    a->block_parent.assign(num_blocks, -1);
    a->parent_incarnation.assign(num_blocks, 0);
    a->incarnation.assign(num_blocks, 0);
    // hand-out order: order[0] first
    std::vector<int32_t> order(num_blocks);
    for (int32_t i = 0; i < num_blocks; ++i) order[i] = i;
    if (shuffle_seed != 0) {
      uint64_t s = shuffle_seed;
      for (int32_t i = num_blocks - 1; i > 0; --i) {
        const int32_t j = static_cast<int32_t>(splitmix64(s) % static_cast<uint64_t>(i + 1));
        std::swap(order[i], order[j]);
      }
    }
    a->free_stack.assign(order.rbegin(), order.rend());
  } catch (...) {
    delete a;
    return nullptr;
  }
  return a;
}

void pkv_alloc_destroy(pkv_alloc* a) { delete a; }

int pkv_alloc_add_seq(pkv_alloc* a, int64_t seq_id, int32_t num_tokens) {
  if (!a) return PKV_E_NULL;
  if (num_tokens < 0) return PKV_E_SHAPE;
  if (a->seqs.count(seq_id)) return PKV_E_EXISTS;
  const int32_t need = a->blocks_for(num_tokens);
  if (need > a->num_free()) return PKV_E_NOMEM;
  pkv_alloc::Seq s;
  s.len = num_tokens;
  s.blocks.reserve(need);
  for (int32_t i = 0; i < need; ++i) s.blocks.push_back(a->take());
  a->seqs.emplace(seq_id, std::move(s));
  return PKV_OK;
}

int pkv_alloc_add_seq_shared(pkv_alloc* a, int64_t seq_id, int32_t num_tokens, int64_t src_seq,
                             int32_t num_shared_blocks) {
  if (!a) return PKV_E_NULL;
  if (num_tokens < 0 || num_shared_blocks < 0) return PKV_E_SHAPE;
  if (a->seqs.count(seq_id)) return PKV_E_EXISTS;
  auto it = a->seqs.find(src_seq);
  if (it == a->seqs.end()) return PKV_E_NOSEQ;
  const int64_t shared_tokens = static_cast<int64_t>(num_shared_blocks) * a->block_size;
  if (shared_tokens > num_tokens || shared_tokens > it->second.len) return PKV_E_SHAPE;
  const int32_t need = a->blocks_for(num_tokens);
  const int32_t fresh = need - num_shared_blocks;
  if (fresh > a->num_free()) return PKV_E_NOMEM;
  pkv_alloc::Seq s;
  s.len = num_tokens;
  s.blocks.reserve(need);
  for (int32_t j = 0; j < num_shared_blocks; ++j) {
    const int32_t b = it->second.blocks[j];
    ++a->refcount[b];
    s.blocks.push_back(b);
  }
  for (int32_t j = 0; j < fresh; ++j) s.blocks.push_back(a->take());
  a->seqs.emplace(seq_id, std::move(s));
  return PKV_OK;
}

int pkv_alloc_share_prefix(pkv_alloc* a, int64_t dst_seq, int64_t src_seq, int32_t num_full_blocks) {
  if (!a) return PKV_E_NULL;
  auto d = a->seqs.find(dst_seq);
  auto s = a->seqs.find(src_seq);
  if (d == a->seqs.end() || s == a->seqs.end()) return PKV_E_NOSEQ;
  if (num_full_blocks < 0 || dst_seq == src_seq) return PKV_E_SHAPE;
  const int64_t tokens = static_cast<int64_t>(num_full_blocks) * a->block_size;
  if (tokens > s->second.len || tokens > d->second.len) return PKV_E_SHAPE;
  // take the new references before dropping the old ones, so a block that
  // dst_seq already shares with src_seq never reaches a zero count
  for (int32_t j = 0; j < num_full_blocks; ++j) {
    const int32_t b = s->second.blocks[j];
    const int32_t old = d->second.blocks[j];
    if (b == old) continue;
    ++a->refcount[b];
    d->second.blocks[j] = b;
    a->release(old);
  }
  return PKV_OK;
}

int pkv_alloc_add_seq_prefix(pkv_alloc* a, int64_t seq_id, const int32_t* token_ids, int32_t num_tokens,
                             int32_t* cached_tokens_out) {
  if (!a || !cached_tokens_out || (num_tokens > 0 && !token_ids)) return PKV_E_NULL;
  if (num_tokens < 0) return PKV_E_SHAPE;
  if (a->seqs.count(seq_id)) return PKV_E_EXISTS;
  const int32_t bs = a->block_size;
  const int32_t need = a->blocks_for(num_tokens), full = num_tokens / bs;
  // longest run of leading full blocks already registered (exact match), live
  // or free; the free ones matched leave the free pool
  std::vector<uint64_t> hashes(full);
  int32_t shared = 0, parent = -1, revived = 0;
  uint64_t h = 0x6a09e667f3bcc909ull;
  for (int32_t j = 0; j < full; ++j) {
    h = chain_hash(h, token_ids + static_cast<int64_t>(j) * bs, bs);
    hashes[j] = h;
    if (shared == j) {
      auto it = a->by_hash.find(h);
      if (it != a->by_hash.end()) {
        const int32_t c = it->second;
        if (a->block_parent[c] == parent &&
            (parent < 0 || a->parent_incarnation[c] == a->incarnation[parent]) &&
            std::equal(token_ids + static_cast<int64_t>(j) * bs, token_ids + static_cast<int64_t>(j + 1) * bs,
                       a->block_tokens.begin() + static_cast<int64_t>(c) * bs)) {
          parent = c;
          ++shared;
          revived += a->refcount[c] == 0;
        }
      }
    }
  }
  if (need - shared > a->num_free() - revived) return PKV_E_NOMEM;
  try {
    if (a->block_tokens.empty()) a->block_tokens.assign(static_cast<size_t>(a->num_blocks) * bs, 0);
    pkv_alloc::Seq s;
    s.len = num_tokens;
    s.blocks.reserve(need);
    parent = -1;
    // the shared blocks first, so that taking the fresh ones cannot reuse them
    for (int32_t j = 0; j < need; ++j) {
      int32_t b;
      if (j < shared) {
        b = a->by_hash.find(hashes[j])->second;
        a->hold(b);
      } else {
        b = a->take();
        if (j < full) {
          // register the new full block.  A block registered under the same
          // hash could not be matched (the chained hash fixes every earlier
          // token, so only a block whose ancestors are gone, or a collision,
          // stops the match before it): it leaves the registry, and if free it
          // holds nothing findable any more
          auto it = a->by_hash.find(hashes[j]);
          if (it != a->by_hash.end()) {
            const int32_t e = it->second;
            a->unregister(e);
            if (a->refcount[e] == 0) {
              a->lru_remove(e);
              a->free_stack.push_back(e);
            }
          }
          a->by_hash.emplace(hashes[j], b);
          a->block_hash[b] = hashes[j];
          a->block_parent[b] = parent;
          a->parent_incarnation[b] = parent >= 0 ? a->incarnation[parent] : 0;
          std::copy(token_ids + static_cast<int64_t>(j) * bs, token_ids + static_cast<int64_t>(j + 1) * bs,
                    a->block_tokens.begin() + static_cast<int64_t>(b) * bs);
        }
      }
      s.blocks.push_back(b);
      parent = b;
    }
    a->seqs.emplace(seq_id, std::move(s));
  } catch (...) {
    return PKV_E_NOMEM;
  }
  *cached_tokens_out = shared * bs;
  return PKV_OK;
}

int pkv_alloc_append_slot(pkv_alloc* a, int64_t seq_id, int64_t* slot_out) {
  return pkv_alloc_append_slots(a, &seq_id, 1, slot_out);
}

int pkv_alloc_append_slots(pkv_alloc* a, const int64_t* seq_ids, int32_t n, int64_t* slots_out) {
  if (!a || (n > 0 && (!seq_ids || !slots_out))) return PKV_E_NULL;
  if (n < 0) return PKV_E_SHAPE;
  // check first, so that failure changes nothing
  std::vector<pkv_alloc::Seq*> ss(n);
  int64_t fresh = 0;
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return PKV_E_NOSEQ;
    ss[i] = &it->second;
    for (int32_t k = 0; k < i; ++k)
      if (ss[k] == ss[i]) return PKV_E_SHAPE;  // one token per sequence per call
    if (ss[i]->len == static_cast<int64_t>(ss[i]->blocks.size()) * a->block_size) ++fresh;
  }
  if (fresh > a->num_free()) return PKV_E_NOMEM;
  for (int32_t i = 0; i < n; ++i) {
    pkv_alloc::Seq& s = *ss[i];
    const int32_t pos = s.len;
    if (pos == static_cast<int32_t>(s.blocks.size()) * a->block_size) s.blocks.push_back(a->take());
    slots_out[i] = static_cast<int64_t>(s.blocks[pos / a->block_size]) * a->block_size + pos % a->block_size;
    s.len = pos + 1;
  }
  return PKV_OK;
}

int pkv_alloc_free_seq(pkv_alloc* a, int64_t seq_id) {
  if (!a) return PKV_E_NULL;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PKV_E_NOSEQ;
  // release in reverse so the sequence's first block is the next one handed out
  for (auto b = it->second.blocks.rbegin(); b != it->second.blocks.rend(); ++b) a->release(*b);
  a->seqs.erase(it);
  return PKV_OK;
}

int pkv_alloc_block_tables(const pkv_alloc* a, const int64_t* seq_ids, int32_t n, int32_t max_blocks,
                           int32_t pad_value, int32_t* tables_out, int32_t* context_lens_out) {
  if (!a || (n > 0 && (!seq_ids || !tables_out || !context_lens_out))) return PKV_E_NULL;
  if (n < 0 || max_blocks <= 0) return PKV_E_SHAPE;
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return PKV_E_NOSEQ;
    if (static_cast<int32_t>(it->second.blocks.size()) > max_blocks) return PKV_E_SHAPE;
  }
  for (int32_t i = 0; i < n; ++i) {
    const pkv_alloc::Seq& s = a->seqs.find(seq_ids[i])->second;
    int32_t* row = tables_out + static_cast<int64_t>(i) * max_blocks;
    const int32_t nb = static_cast<int32_t>(s.blocks.size());
    std::copy(s.blocks.begin(), s.blocks.end(), row);
    std::fill(row + nb, row + max_blocks, pad_value);
    context_lens_out[i] = s.len;
  }
  return PKV_OK;
}

int32_t pkv_alloc_num_free(const pkv_alloc* a) {
  return a ? a->num_free() : 0;
}

int32_t pkv_alloc_num_cached(const pkv_alloc* a) { return a ? a->lru_size : 0; }

int32_t pkv_alloc_num_seqs(const pkv_alloc* a) {
  return a ? static_cast<int32_t>(a->seqs.size()) : 0;
}

int pkv_alloc_context_len(const pkv_alloc* a, int64_t seq_id, int32_t* len_out) {
  if (!a || !len_out) return PKV_E_NULL;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PKV_E_NOSEQ;
  *len_out = it->second.len;
  return PKV_OK;
}

int32_t pkv_alloc_refcount(const pkv_alloc* a, int32_t block) {
  if (!a || block < 0 || block >= a->num_blocks) return -1;
  return a->refcount[block];
}

}  // extern "C"
