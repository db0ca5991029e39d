// block_manager.cpp -- the host-side block manager of include/pa_block_manager.h:
// a FIFO free queue of pool blocks, per-block reference counts, per-sequence
// block tables, copy-on-write of shared partial blocks, and a prefix cache of
// full blocks keyed by their content.
//
// Content keys are interned: a key is (parent key, the block's token ids),
// and equal keys get the same id, so two keys are equal exactly when the
// whole token prefixes they stand for are.  Keys are reference counted by the
// cached block that holds them, by sequences whose last full block they
// describe, and by their child keys, and are dropped at zero.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <deque>
#include <list>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "pa_block_manager.h"

namespace {

constexpr int64_t kNoKey = -1;

struct Key {
  int64_t parent;
  std::vector<int32_t> tokens;
  int32_t block = -1;  // cached block holding this content, -1 if none
  int32_t refs = 0;
};

struct Sequence {
  std::vector<int32_t> blocks;
  int64_t len = 0;
  std::vector<int32_t> tail;  // token ids of the partly filled last block
  int64_t last_key = kNoKey;  // key of the last full block
  uint64_t stamp = 0;         // last batched call that named this sequence
};

uint64_t mix(uint64_t h, uint64_t v) {  // splitmix64 step over h ^ v
  uint64_t z = h ^ (v + 0x9e3779b97f4a7c15ull + (h << 6) + (h >> 2));
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

}  // namespace

struct pa_bm {
  int32_t nb, bs;
  std::deque<int32_t> free_q;
  std::vector<int32_t> refs;       // per block: sequences referencing it
  std::vector<int64_t> key_of;     // per block: registered key, kNoKey if none
  std::list<int32_t> evictable;    // cached blocks nobody uses, oldest first
  std::vector<std::list<int32_t>::iterator> ev_pos;
  std::vector<char> in_ev;
  std::unordered_map<int64_t, Key> keys;
  std::unordered_multimap<uint64_t, int64_t> key_index;  // content hash -> key id
  int64_t next_key = 0;
  std::unordered_map<int64_t, Sequence> seqs;
  uint64_t calls = 0;              // batched calls so far (duplicate-id check)
  std::vector<Sequence*> picked;   // sequences of the current batched call
  mutable std::mutex mu;

  // ---- keys
  static uint64_t content_hash(int64_t parent, const int32_t* t, int n) {
    uint64_t h = mix(0x243f6a8885a308d3ull, (uint64_t)parent);
    for (int i = 0; i < n; ++i) h = mix(h, (uint64_t)(uint32_t)t[i]);
    return h;
  }
  int64_t find_key(int64_t parent, const int32_t* t) const {
    auto r = key_index.equal_range(content_hash(parent, t, bs));
    for (auto it = r.first; it != r.second; ++it) {
      const Key& k = keys.at(it->second);
      if (k.parent == parent && std::equal(k.tokens.begin(), k.tokens.end(), t)) return it->second;
    }
    return kNoKey;
  }
  int64_t intern(int64_t parent, const int32_t* t) {
    int64_t id = find_key(parent, t);
    if (id != kNoKey) return id;
    id = next_key++;
    Key k;
    k.parent = parent;
    k.tokens.assign(t, t + bs);
    keys.emplace(id, std::move(k));
    key_index.emplace(content_hash(parent, t, bs), id);
    ref_key(parent);
    return id;
  }
  void ref_key(int64_t id) {
    if (id != kNoKey) ++keys.at(id).refs;
  }
  void unref_key(int64_t id) {
    while (id != kNoKey) {
      Key& k = keys.at(id);
      if (--k.refs > 0) return;
      const int64_t parent = k.parent;
      auto r = key_index.equal_range(content_hash(parent, k.tokens.data(), bs));
      for (auto it = r.first; it != r.second; ++it)
        if (it->second == id) {
          key_index.erase(it);
          break;
        }
      keys.erase(id);
      id = parent;  // the child's reference to its parent goes too
    }
  }

  // ---- pool
  int32_t num_free() const { return (int32_t)(free_q.size() + evictable.size()); }

  int32_t take() {  // caller has checked num_free() > 0
    int32_t b;
    if (!free_q.empty()) {
      b = free_q.front();
      free_q.pop_front();
    } else {
      b = evictable.front();
      evictable.pop_front();
      in_ev[b] = 0;
      Key& k = keys.at(key_of[b]);
      k.block = -1;
      const int64_t id = key_of[b];
      key_of[b] = kNoKey;
      unref_key(id);
    }
    refs[b] = 1;
    return b;
  }
  void release(int32_t b) {
    if (--refs[b] > 0) return;
    if (key_of[b] != kNoKey) {
      evictable.push_back(b);
      ev_pos[b] = std::prev(evictable.end());
      in_ev[b] = 1;
    } else {
      free_q.push_back(b);
    }
  }
  void use_cached(int32_t b) {
    if (refs[b] == 0 && in_ev[b]) {
      evictable.erase(ev_pos[b]);
      in_ev[b] = 0;
    }
    ++refs[b];
  }

  // After a token lands: a block that just filled joins the cache.
  void register_if_full(Sequence& q) {
    if (q.len % bs != 0) return;
    const int32_t blk = q.blocks.back();
    const int64_t id = intern(q.last_key, q.tail.data());
    ref_key(id);             // the sequence now describes its prefix by id
    unref_key(q.last_key);   // ... instead of by the previous key
    q.last_key = id;
    q.tail.clear();
    Key& k = keys.at(id);
    if (k.block == -1 && key_of[blk] == kNoKey) {
      k.block = blk;
      key_of[blk] = id;
      ++k.refs;
    }
  }

  void push_token(Sequence& q, int32_t tok, int32_t* slot) {
    *slot = (int32_t)(q.blocks.back() * (int64_t)bs + q.len % bs);
    q.tail.push_back(tok);
    ++q.len;
    register_if_full(q);
  }
};

extern "C" {

pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                       pa_bm** out) {
  if (!out) return PA_ERR_NULL;
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0) return PA_ERR_SHAPE;
  pa_bm* bm = new pa_bm();
  bm->nb = num_blocks;
  bm->bs = block_size;
  bm->refs.assign(num_blocks, 0);
  bm->key_of.assign(num_blocks, kNoKey);
  bm->ev_pos.resize(num_blocks);
  bm->in_ev.assign(num_blocks, 0);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete bm;
        return PA_ERR_SHAPE;
      }
      seen[b] = 1;
      bm->free_q.push_back(b);
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) bm->free_q.push_back(i);
  }
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_bm* bm) { delete bm; }

int32_t pa_bm_num_free(const pa_bm* bm) {
  if (!bm) return -1;
  std::lock_guard<std::mutex> lock(bm->mu);
  return bm->num_free();
}

pa_status pa_bm_add_sequence(pa_bm* bm, int64_t seq_id, const int32_t* tokens,
                             int32_t num_tokens, int32_t* slots, int32_t* num_cached) {
  if (!bm || !num_cached || (num_tokens > 0 && (!tokens || !slots))) return PA_ERR_NULL;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  std::lock_guard<std::mutex> lock(bm->mu);
  if (bm->seqs.count(seq_id)) return PA_ERR_SHAPE;
  const int32_t bs = bm->bs;
  // cached prefix: whole blocks, stopping at the first miss
  std::vector<int32_t> hits;
  int64_t key = kNoKey;
  for (int32_t j = 0; j < num_tokens / bs; ++j) {
    const int64_t k = bm->find_key(key, tokens + (int64_t)j * bs);
    if (k == kNoKey || bm->keys.at(k).block < 0) break;
    hits.push_back(bm->keys.at(k).block);
    key = k;
  }
  const int32_t n_cached = (int32_t)hits.size() * bs;
  const int64_t need = (num_tokens + bs - 1) / bs - (int64_t)hits.size();
  int64_t revive = 0;
  for (int32_t b : hits) revive += bm->refs[b] == 0;
  if (need > bm->num_free() - revive) return PA_ERR_NO_BLOCKS;
  for (int32_t b : hits) bm->use_cached(b);
  Sequence& q = bm->seqs[seq_id];
  q.blocks = hits;
  q.len = n_cached;
  q.last_key = key;
  bm->ref_key(key);
  for (int32_t i = 0; i < n_cached; ++i) slots[i] = -1;
  for (int32_t i = n_cached; i < num_tokens; ++i) {
    if (q.len % bs == 0) q.blocks.push_back(bm->take());
    bm->push_token(q, tokens[i], &slots[i]);
  }
  *num_cached = n_cached;
  return PA_OK;
}

pa_status pa_bm_append(pa_bm* bm, int64_t seq_id, const int32_t* tokens, int32_t num_tokens,
                       int32_t* slots, int32_t* cow_pairs, int32_t cow_capacity,
                       int32_t* num_cow) {
  if (!bm || !num_cow || (num_tokens > 0 && (!tokens || !slots)) ||
      (cow_capacity > 0 && !cow_pairs))
    return PA_ERR_NULL;
  if (num_tokens < 0 || cow_capacity < 0) return PA_ERR_SHAPE;
  std::lock_guard<std::mutex> lock(bm->mu);
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_SHAPE;
  Sequence& q = it->second;
  const int32_t bs = bm->bs;
  *num_cow = 0;
  const bool cow = num_tokens > 0 && q.len % bs != 0 && bm->refs[q.blocks.back()] > 1;
  if (cow && cow_capacity < 1) return PA_ERR_SHAPE;
  const int64_t need = (cow ? 1 : 0) + (q.len + num_tokens + bs - 1) / bs - (q.len + bs - 1) / bs;
  if (need > bm->num_free()) return PA_ERR_NO_BLOCKS;
  for (int32_t i = 0; i < num_tokens; ++i) {
    if (q.len % bs == 0) {
      q.blocks.push_back(bm->take());
    } else if (bm->refs[q.blocks.back()] > 1) {
      const int32_t src = q.blocks.back();
      const int32_t dst = bm->take();
      bm->release(src);
      q.blocks.back() = dst;
      cow_pairs[2 * *num_cow] = src;
      cow_pairs[2 * *num_cow + 1] = dst;
      ++*num_cow;
    }
    bm->push_token(q, tokens[i], &slots[i]);
  }
  return PA_OK;
}

pa_status pa_bm_append_batch(pa_bm* bm, const int64_t* seq_ids, const int32_t* tokens,
                             int32_t num_seqs, int32_t* slots, int32_t* cow_pairs,
                             int32_t cow_capacity, int32_t* num_cow) {
  if (!bm || !num_cow || (num_seqs > 0 && (!seq_ids || !tokens || !slots)) ||
      (cow_capacity > 0 && !cow_pairs))
    return PA_ERR_NULL;
  if (num_seqs < 0 || cow_capacity < 0) return PA_ERR_SHAPE;
  std::lock_guard<std::mutex> lock(bm->mu);
  *num_cow = 0;
  const int32_t bs = bm->bs;
  // Validate and count the blocks the step needs before changing anything.
  // A copy lowers the shared block's count, which can spare a later sequence
  // of the same step its own copy: track those drops.
  std::vector<Sequence*>& qs = bm->picked;
  qs.resize(num_seqs);
  const uint64_t stamp = ++bm->calls;
  std::unordered_map<int32_t, int32_t> dropped;
  int64_t need = 0, copies = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end() || it->second.stamp == stamp) return PA_ERR_SHAPE;
    Sequence& q = it->second;
    q.stamp = stamp;
    qs[i] = &q;
    if (q.len % bs == 0) {
      ++need;
      continue;
    }
    const int32_t b = q.blocks.back();
    auto d = dropped.find(b);
    const int32_t r = bm->refs[b] - (d == dropped.end() ? 0 : d->second);
    if (r > 1) {
      ++need;
      ++copies;
      ++dropped[b];
    }
  }
  if (copies > cow_capacity) return PA_ERR_SHAPE;
  if (need > bm->num_free()) return PA_ERR_NO_BLOCKS;
  for (int32_t i = 0; i < num_seqs; ++i) {
    Sequence& q = *qs[i];
    if (q.len % bs == 0) {
      q.blocks.push_back(bm->take());
    } else if (bm->refs[q.blocks.back()] > 1) {
      const int32_t src = q.blocks.back();
      const int32_t dst = bm->take();
      bm->release(src);
      q.blocks.back() = dst;
      cow_pairs[2 * *num_cow] = src;
      cow_pairs[2 * *num_cow + 1] = dst;
      ++*num_cow;
    }
    bm->push_token(q, tokens[i], &slots[i]);
  }
  return PA_OK;
}

pa_status pa_bm_fork(pa_bm* bm, int64_t parent_id, int64_t child_id) {
  if (!bm) return PA_ERR_NULL;
  std::lock_guard<std::mutex> lock(bm->mu);
  auto it = bm->seqs.find(parent_id);
  if (it == bm->seqs.end() || bm->seqs.count(child_id)) return PA_ERR_SHAPE;
  Sequence child = it->second;
  for (int32_t b : child.blocks) ++bm->refs[b];
  bm->ref_key(child.last_key);
  bm->seqs.emplace(child_id, std::move(child));
  return PA_OK;
}

pa_status pa_bm_free(pa_bm* bm, int64_t seq_id) {
  if (!bm) return PA_ERR_NULL;
  std::lock_guard<std::mutex> lock(bm->mu);
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_SHAPE;
  for (int32_t b : it->second.blocks) bm->release(b);
  bm->unref_key(it->second.last_key);
  bm->seqs.erase(it);
  return PA_OK;
}

pa_status pa_bm_tables(pa_bm* bm, const int64_t* seq_ids, int32_t num_seqs,
                       int32_t max_blocks_per_seq, int32_t pad_block, int32_t* tables,
                       int32_t* seq_lens) {
  if (!bm || (num_seqs > 0 && (!seq_ids || !tables || !seq_lens))) return PA_ERR_NULL;
  if (num_seqs < 0 || max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  std::lock_guard<std::mutex> lock(bm->mu);
  std::vector<Sequence*>& qs = bm->picked;
  qs.resize(num_seqs);
  for (int32_t s = 0; s < num_seqs; ++s) {
    auto it = bm->seqs.find(seq_ids[s]);
    if (it == bm->seqs.end() || (int64_t)it->second.blocks.size() > max_blocks_per_seq ||
        it->second.len > INT32_MAX)
      return PA_ERR_SHAPE;
    qs[s] = &it->second;
  }
  for (int32_t s = 0; s < num_seqs; ++s) {
    const Sequence& q = *qs[s];
    int32_t* row = tables + (int64_t)s * max_blocks_per_seq;
    const int32_t n = (int32_t)q.blocks.size();
    std::copy(q.blocks.begin(), q.blocks.end(), row);
    std::fill(row + n, row + max_blocks_per_seq, pad_block);
    seq_lens[s] = (int32_t)q.len;
  }
  return PA_OK;
}

int32_t pa_bm_block_refs(const pa_bm* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->nb) return -1;
  std::lock_guard<std::mutex> lock(bm->mu);
  return bm->refs[block];
}

}  // extern "C"
