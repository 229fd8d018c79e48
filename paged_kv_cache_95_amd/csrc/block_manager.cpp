// Host-side block manager: hands out the pool's 16-token blocks to sequences, keeps each
// sequence's block table, and shares full blocks with identical token prefixes.
//
// Follows the BlockManager / PagedKVCache of the koas-w "errors and solutions" post
// ("KV Cache management": one global pool of fixed 16-token blocks allocated up front,
// blocks allocated and recycled per request, a logical -> physical block_table per
// request whose lifetime is the request's) and the cross-request prefix sharing that
// PocketLLM "cpp_engine Batching Implementation (Phase 3.1)" plans after per-slot prefix
// caches (risk 3). Policy (this library's reading; the pages fix none of it):
//  * a new block is the lowest-numbered free block that holds no cached prefix; only
//    when none is left is a cached free block evicted, least recently released first
//    (ties: lowest number);
//  * a block that becomes full gets a chained hash of (previous block's hash, its
//    token ids) and is entered in the prefix index unless that hash is already there;
//  * a new sequence reuses indexed blocks for its leading full blocks while the hash
//    matches and the stored token ids are equal, but always leaves at least its last
//    token to be computed;
//  * appending to a shared partial block copies it first (copy-on-write; the caller
//    copies the device rows, e.g. with pa_copy_blocks);
//  * released blocks are returned tail first, so a sequence's prefix stays cached
//    longest.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <map>
#include <new>
#include <set>
#include <unordered_map>
#include <vector>

#include "internal.h"

namespace {

uint64_t mix64(uint64_t x) {  // splitmix64 finaliser
  x ^= x >> 30;
  x *= 0xbf58476d1ce4e5b9ULL;
  x ^= x >> 27;
  x *= 0x94d049bb133111ebULL;
  x ^= x >> 31;
  return x;
}

uint64_t block_hash(uint64_t parent, const int32_t* tokens, int n) {
  uint64_t h = mix64(parent ^ 0x9e3779b97f4a7c15ULL);
  for (int i = 0; i < n; ++i) h = mix64(h ^ (uint64_t)(uint32_t)tokens[i]);
  return h | 1;  // 0 means "no hash"
}

struct Seq {
  std::vector<int32_t> blocks;
  std::vector<uint64_t> hashes;  // per block; 0 while the block is not full
  std::vector<int32_t> tokens;
};

}  // namespace

struct pa_block_manager {
  int64_t num_blocks = 0;
  int block_size = 16;
  bool prefix_cache = true;
  std::vector<int32_t> refcount;
  std::vector<uint64_t> hash;             // hash of a block in the prefix index, else 0
  std::vector<uint64_t> parent;           // its parent's hash
  std::vector<std::vector<int32_t>> toks; // its token ids
  std::vector<int64_t> released_at;       // release time of a cached free block
  std::set<int32_t> free_plain;           // free, no cached prefix
  std::set<std::pair<int64_t, int32_t>> free_cached;  // (released_at, block)
  std::unordered_map<uint64_t, int32_t> index;         // hash -> block
  std::map<int64_t, Seq> seqs;
  int64_t clock = 0;

  int64_t num_free() const { return (int64_t)free_plain.size() + (int64_t)free_cached.size(); }

  // Take a free block (caller checked that one exists); it leaves with refcount 1.
  int32_t take() {
    int32_t b;
    if (!free_plain.empty()) {
      b = *free_plain.begin();
      free_plain.erase(free_plain.begin());
    } else {
      const auto it = free_cached.begin();
      b = it->second;
      free_cached.erase(it);
      index.erase(hash[b]);
      hash[b] = parent[b] = 0;
      toks[b].clear();
    }
    refcount[b] = 1;
    return b;
  }

  void release(int32_t b) {
    if (--refcount[b] > 0) return;
    if (hash[b] != 0) {
      released_at[b] = clock++;
      free_cached.insert({released_at[b], b});
    } else {
      free_plain.insert(b);
    }
  }

  // Enter full block b (tokens t[0..bs), parent hash p) in the prefix index.
  uint64_t publish(int32_t b, uint64_t p, const int32_t* t) {
    const uint64_t h = block_hash(p, t, block_size);
    if (prefix_cache && index.find(h) == index.end() && hash[b] == 0) {
      index[h] = b;
      hash[b] = h;
      parent[b] = p;
      toks[b].assign(t, t + block_size);
    }
    return h;
  }

  // Block holding exactly these tokens after parent hash p, or -1.
  int32_t lookup(uint64_t p, const int32_t* t) const {
    if (!prefix_cache) return -1;
    const auto it = index.find(block_hash(p, t, block_size));
    if (it == index.end()) return -1;
    const int32_t b = it->second;
    if (parent[b] != p || !std::equal(toks[b].begin(), toks[b].end(), t)) return -1;
    return b;
  }
};

extern "C" {

pa_block_manager_t* pa_bm_create(int64_t num_blocks, int32_t block_size,
                                 int32_t prefix_caching) {
  if (num_blocks <= 0 || num_blocks > INT32_MAX || block_size <= 0) return nullptr;
  pa_block_manager_t* m = new (std::nothrow) pa_block_manager_t();
  if (!m) return nullptr;
  m->num_blocks = num_blocks;
  m->block_size = block_size;
  m->prefix_cache = prefix_caching != 0;
  m->refcount.assign(num_blocks, 0);
  m->hash.assign(num_blocks, 0);
  m->parent.assign(num_blocks, 0);
  m->toks.assign(num_blocks, {});
  m->released_at.assign(num_blocks, 0);
  for (int64_t b = 0; b < num_blocks; ++b) m->free_plain.insert((int32_t)b);
  return m;
}

void pa_bm_destroy(pa_block_manager_t* m) { delete m; }

int64_t pa_bm_num_free_blocks(const pa_block_manager_t* m) { return m ? m->num_free() : -1; }

int pa_bm_add_sequence(pa_block_manager_t* m, int64_t seq_id, const int32_t* token_ids,
                       int64_t num_tokens, int64_t* cached_tokens) {
  if (!m || num_tokens < 0 || (num_tokens > 0 && !token_ids)) return PA_ERR_INVALID_ARG;
  if (m->seqs.count(seq_id)) return PA_ERR_INVALID_ARG;
  const int bs = m->block_size;
  const int64_t nblocks = (num_tokens + bs - 1) / bs;
  // leading full blocks found in the prefix index (never the block of the last token)
  const int64_t reusable = num_tokens > 0 ? (num_tokens - 1) / bs : 0;
  std::vector<int32_t> hit;
  std::vector<uint64_t> hit_hash;
  uint64_t p = 0;
  for (int64_t i = 0; i < reusable; ++i) {
    const int32_t b = m->lookup(p, token_ids + i * bs);
    if (b < 0) break;
    hit.push_back(b);
    p = m->hash[b];
    hit_hash.push_back(p);
  }
  int64_t from_free = 0;  // matched blocks that currently sit in the free (cached) set
  for (const int32_t b : hit) from_free += m->refcount[b] == 0;
  if ((int64_t)(nblocks - hit.size()) > m->num_free() - from_free) return PA_ERR_WORKSPACE;
  Seq s;
  for (size_t i = 0; i < hit.size(); ++i) {
    const int32_t b = hit[i];
    if (m->refcount[b] == 0) m->free_cached.erase({m->released_at[b], b});
    ++m->refcount[b];
    s.blocks.push_back(b);
    s.hashes.push_back(hit_hash[i]);
  }
  for (int64_t i = (int64_t)hit.size(); i < nblocks; ++i) {
    const int32_t b = m->take();
    s.blocks.push_back(b);
    uint64_t h = 0;
    if ((i + 1) * bs <= num_tokens) h = m->publish(b, p, token_ids + i * bs);
    s.hashes.push_back(h);
    p = h;
  }
  s.tokens.assign(token_ids, token_ids + num_tokens);
  m->seqs.emplace(seq_id, std::move(s));
  if (cached_tokens) *cached_tokens = (int64_t)hit.size() * bs;
  return PA_OK;
}

int pa_bm_append_token(pa_block_manager_t* m, int64_t seq_id, int32_t token_id, int64_t* slot,
                       int32_t* copy_src, int32_t* copy_dst) {
  if (!m || !slot || !copy_src || !copy_dst) return PA_ERR_INVALID_ARG;
  const auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PA_ERR_INVALID_ARG;
  Seq& s = it->second;
  const int bs = m->block_size;
  const int64_t pos = (int64_t)s.tokens.size();
  *copy_src = *copy_dst = -1;
  if (pos % bs == 0) {
    if (m->num_free() < 1) return PA_ERR_WORKSPACE;
    s.blocks.push_back(m->take());
    s.hashes.push_back(0);
  } else if (m->refcount[s.blocks.back()] > 1) {
    // the partial last block is shared (after a fork): copy it first
    if (m->num_free() < 1) return PA_ERR_WORKSPACE;
    const int32_t old = s.blocks.back();
    const int32_t b = m->take();
    m->release(old);
    s.blocks.back() = b;
    *copy_src = old;
    *copy_dst = b;
  }
  s.tokens.push_back(token_id);
  if ((pos + 1) % bs == 0) {
    const size_t i = s.blocks.size() - 1;
    const uint64_t p = i > 0 ? s.hashes[i - 1] : 0;
    s.hashes[i] = m->publish(s.blocks[i], p, s.tokens.data() + i * bs);
  }
  *slot = (int64_t)s.blocks.back() * bs + pos % bs;
  return PA_OK;
}

int pa_bm_fork(pa_block_manager_t* m, int64_t parent_id, int64_t child_id) {
  if (!m) return PA_ERR_INVALID_ARG;
  const auto it = m->seqs.find(parent_id);
  if (it == m->seqs.end() || m->seqs.count(child_id)) return PA_ERR_INVALID_ARG;
  Seq c = it->second;
  for (const int32_t b : c.blocks) ++m->refcount[b];
  m->seqs.emplace(child_id, std::move(c));
  return PA_OK;
}

int pa_bm_free_sequence(pa_block_manager_t* m, int64_t seq_id) {
  if (!m) return PA_ERR_INVALID_ARG;
  const auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PA_ERR_INVALID_ARG;
  const std::vector<int32_t>& bl = it->second.blocks;
  for (auto b = bl.rbegin(); b != bl.rend(); ++b) m->release(*b);  // tail first
  m->seqs.erase(it);
  return PA_OK;
}

int64_t pa_bm_context_len(const pa_block_manager_t* m, int64_t seq_id) {
  if (!m) return -1;
  const auto it = m->seqs.find(seq_id);
  return it == m->seqs.end() ? -1 : (int64_t)it->second.tokens.size();
}

int pa_bm_block_tables(const pa_block_manager_t* m, const int64_t* seq_ids, int32_t num_seqs,
                       int32_t max_blocks_per_seq, int32_t* block_tables,
                       int32_t* context_lens) {
  if (!m || num_seqs < 0 || max_blocks_per_seq <= 0 || (num_seqs > 0 && (!seq_ids || !block_tables)))
    return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const auto it = m->seqs.find(seq_ids[i]);
    if (it == m->seqs.end() || (int64_t)it->second.blocks.size() > max_blocks_per_seq)
      return PA_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Seq& s = m->seqs.find(seq_ids[i])->second;
    int32_t* row = block_tables + (int64_t)i * max_blocks_per_seq;
    std::fill(row, row + max_blocks_per_seq, -1);
    std::copy(s.blocks.begin(), s.blocks.end(), row);
    if (context_lens) context_lens[i] = (int32_t)s.tokens.size();
  }
  return PA_OK;
}

int pa_bm_slots(const pa_block_manager_t* m, int64_t seq_id, int64_t first_pos, int64_t count,
                int64_t* slots) {
  if (!m || count < 0 || first_pos < 0 || (count > 0 && !slots)) return PA_ERR_INVALID_ARG;
  const auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end() || first_pos + count > (int64_t)it->second.tokens.size())
    return PA_ERR_INVALID_ARG;
  const Seq& s = it->second;
  const int bs = m->block_size;
  for (int64_t j = 0; j < count; ++j) {
    const int64_t p = first_pos + j;
    slots[j] = (int64_t)s.blocks[p / bs] * bs + p % bs;
  }
  return PA_OK;
}

int32_t pa_bm_block_refcount(const pa_block_manager_t* m, int32_t block) {
  if (!m || block < 0 || block >= m->num_blocks) return -1;
  return m->refcount[block];
}

}  // extern "C"
