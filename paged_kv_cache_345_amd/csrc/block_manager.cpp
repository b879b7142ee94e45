// Host block manager of the paged KV cache.
//
// Mechanism from page "vLLM 部署与 PagedAttention 原理 · 检索整理（CSDN 频道批次）",
// item 2 (the 2023 vLLM blog) and page "vLLM：从 PagedAttention 长出来的开源服务栈",
// section "把显存当虚拟内存管": fixed-size blocks, a per-sequence block table,
// on-demand allocation, per-block reference counts and copy-on-write for
// parallel samples.  The exact policy (free-list order, which sharer copies) is
// documented with the declarations in pagedkv.h.
//
// State is a ring-buffer free list (front = next block handed out, back = where
// freed blocks go), a refcount per block and, per sequence, its block list and
// token count.  Every public call validates and counts what it needs first, and
// only then mutates, so failures leave the state unchanged.
//
// Prefix caching (page "vLLM 深度解析：以 PagedAttention 与内核生态构建高吞吐 LLM
// 推理引擎", §2.2: the KV cache of an identical prefix, such as a system prompt,
// is computed once and reused by later requests).  A full block whose token ids
// are known is registered under the key (node id of the block before it in its
// chain, its block_size token ids); node ids are handed out once and never
// reused, so a key names one exact token prefix.  A registered block whose
// refcount drops to zero becomes evictable instead of free: still found by its
// key, revived by a hit, and taken (least recently freed first, its key dropped)
// only when the free list is empty.  With no registered block every call
// behaves exactly as without prefix caching.

#include <cstdint>
#include <cstring>
#include <list>
#include <new>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"

namespace {

// Key of a registered block: parent node id (two int32 halves), then the tokens.
struct KeyHash {
  size_t operator()(const std::vector<int32_t>& k) const {
    uint64_t h = 1469598103934665603ull;  // FNV-1a over the words
    for (int32_t w : k) {
      h ^= static_cast<uint32_t>(w);
      h *= 1099511628211ull;
    }
    return static_cast<size_t>(h);
  }
};

}  // namespace

struct pkv_block_manager {
  struct Seq {
    std::vector<int32_t> blocks;
    int32_t length = 0;
    int64_t chain = -1;           // node of the last full block, 0 = none yet; -1: token ids unknown
    std::vector<int32_t> tail;    // token ids of the partial last block (chain >= 0)
  };

  int32_t num_blocks = 0;
  int32_t block_size = 0;
  // free list as a ring buffer of capacity num_blocks
  std::vector<int32_t> ring;
  int64_t head = 0;  // index of the front element
  int32_t count = 0; // number of free blocks
  std::vector<int32_t> ref;
  std::unordered_map<int32_t, Seq> seqs;
  // prefix cache
  std::unordered_map<std::vector<int32_t>, int32_t, KeyHash> cache;  // key -> block
  std::vector<int64_t> node;                  // node id of a registered block, -1 if none
  std::vector<std::vector<int32_t>> key_of;   // key of a registered block
  std::list<int32_t> evictable;               // front = least recently freed
  std::vector<std::list<int32_t>::iterator> ev_pos;
  std::vector<char> in_ev;
  int64_t next_node = 1;

  int32_t available() const { return count + static_cast<int32_t>(evictable.size()); }

  void unregister(int32_t b) {
    cache.erase(key_of[static_cast<size_t>(b)]);
    key_of[static_cast<size_t>(b)].clear();
    node[static_cast<size_t>(b)] = -1;
  }
  void leave_evictable(int32_t b) {
    evictable.erase(ev_pos[static_cast<size_t>(b)]);
    in_ev[static_cast<size_t>(b)] = 0;
  }
  int32_t take() {
    int32_t b;
    if (count > 0) {
      b = ring[static_cast<size_t>(head)];
      head = (head + 1) % num_blocks;
      --count;
    } else {  // the caller checked available(): evict the least recently freed block
      b = evictable.front();
      leave_evictable(b);
      unregister(b);
    }
    ref[static_cast<size_t>(b)] = 1;
    return b;
  }
  void give_back(int32_t b) {
    if (node[static_cast<size_t>(b)] >= 0) {  // keep its content findable
      ev_pos[static_cast<size_t>(b)] = evictable.insert(evictable.end(), b);
      in_ev[static_cast<size_t>(b)] = 1;
      return;
    }
    ring[static_cast<size_t>((head + count) % num_blocks)] = b;
    ++count;
  }
  std::vector<int32_t> key(int64_t parent, const int32_t* tokens) const {
    std::vector<int32_t> k(static_cast<size_t>(block_size) + 2);
    k[0] = static_cast<int32_t>(parent & 0xffffffff);
    k[1] = static_cast<int32_t>(parent >> 32);
    std::memcpy(k.data() + 2, tokens, sizeof(int32_t) * static_cast<size_t>(block_size));
    return k;
  }
  // a sequence's block b just became full with token ids `tokens`: register it
  // (or, if its content is registered already, follow that block's node)
  void on_full(Seq& s, int32_t b, const int32_t* tokens) {
    if (s.chain < 0) return;
    std::vector<int32_t> k = key(s.chain, tokens);
    auto it = cache.find(k);
    if (it != cache.end()) {
      s.chain = node[static_cast<size_t>(it->second)];
      return;
    }
    const int64_t id = next_node++;
    node[static_cast<size_t>(b)] = id;
    key_of[static_cast<size_t>(b)] = k;
    cache.emplace(std::move(k), b);
    s.chain = id;
  }
  int32_t slot(const Seq& s, int32_t pos) const {
    return s.blocks[static_cast<size_t>(pos / block_size)] * block_size + pos % block_size;
  }
};

namespace {

bool valid_block_size(int32_t bs) { return bs > 0 && bs <= (1 << 20); }

}  // namespace

extern "C" {

pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order) {
  if (num_blocks <= 0 || !valid_block_size(block_size)) return nullptr;
  if (static_cast<int64_t>(num_blocks) * block_size > INT32_MAX) return nullptr;  // slots are int32
  pkv_block_manager* bm = new (std::nothrow) pkv_block_manager();
  if (!bm) return nullptr;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->ring.resize(static_cast<size_t>(num_blocks));
  bm->ref.assign(static_cast<size_t>(num_blocks), 0);
  bm->node.assign(static_cast<size_t>(num_blocks), -1);
  bm->key_of.resize(static_cast<size_t>(num_blocks));
  bm->ev_pos.resize(static_cast<size_t>(num_blocks));
  bm->in_ev.assign(static_cast<size_t>(num_blocks), 0);
  std::vector<char> seen(static_cast<size_t>(num_blocks), 0);
  for (int32_t i = 0; i < num_blocks; ++i) {
    int32_t b = free_order ? free_order[i] : i;
    if (b < 0 || b >= num_blocks || seen[static_cast<size_t>(b)]) {
      delete bm;
      return nullptr;
    }
    seen[static_cast<size_t>(b)] = 1;
    bm->ring[static_cast<size_t>(i)] = b;
  }
  bm->head = 0;
  bm->count = num_blocks;
  return bm;
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

pkv_status pkv_bm_add(pkv_block_manager* bm, int32_t seq, int32_t num_tokens, int32_t* slots_out) {
  if (!bm || num_tokens < 0) return PKV_ERR_INVALID;
  if (bm->seqs.count(seq)) return PKV_ERR_INVALID;
  int64_t need = (static_cast<int64_t>(num_tokens) + bm->block_size - 1) / bm->block_size;
  if (need > bm->available()) return PKV_ERR_OUT_OF_BLOCKS;
  pkv_block_manager::Seq s;
  s.blocks.reserve(static_cast<size_t>(need));
  for (int64_t i = 0; i < need; ++i) s.blocks.push_back(bm->take());
  s.length = num_tokens;
  if (slots_out)
    for (int32_t t = 0; t < num_tokens; ++t) slots_out[t] = bm->slot(s, t);
  bm->seqs.emplace(seq, std::move(s));
  return PKV_OK;
}

pkv_status pkv_bm_fork(pkv_block_manager* bm, int32_t parent, int32_t child) {
  if (!bm || parent == child) return PKV_ERR_INVALID;
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end() || bm->seqs.count(child)) return PKV_ERR_INVALID;
  pkv_block_manager::Seq c = it->second;  // copy of the block list and length
  for (int32_t b : c.blocks) ++bm->ref[static_cast<size_t>(b)];
  bm->seqs.emplace(child, std::move(c));
  return PKV_OK;
}

namespace {

// Appends one token to `s`; the caller has checked that a free block exists if
// one is needed.  Returns the slot; writes the copy pair or (-1, -1).
int32_t append_one(pkv_block_manager* bm, pkv_block_manager::Seq& s, int32_t* cow) {
  const int32_t bs = bm->block_size;
  const int32_t pos = s.length;
  cow[0] = cow[1] = -1;
  s.chain = -1;  // a token without an id: this sequence's later blocks stay unregistered
  s.tail.clear();
  if (pos % bs == 0) {
    s.blocks.push_back(bm->take());
  } else {
    int32_t& last = s.blocks[static_cast<size_t>(pos / bs)];
    if (bm->ref[static_cast<size_t>(last)] > 1) {
      const int32_t fresh = bm->take();
      --bm->ref[static_cast<size_t>(last)];
      cow[0] = last;
      cow[1] = fresh;
      last = fresh;
    }
  }
  s.length = pos + 1;
  return bm->slot(s, pos);
}

// Blocks one append to `s` would take, given the refcounts in `pending` (a
// sparse override of bm->ref for blocks already touched in this batch).
bool append_needs_block(const pkv_block_manager* bm, const pkv_block_manager::Seq& s,
                        std::unordered_map<int32_t, int32_t>& pending) {
  const int32_t pos = s.length;
  if (pos % bm->block_size == 0) return true;
  const int32_t last = s.blocks[static_cast<size_t>(pos / bm->block_size)];
  auto it = pending.find(last);
  int32_t r = it == pending.end() ? bm->ref[static_cast<size_t>(last)] : it->second;
  if (r > 1) {
    pending[last] = r - 1;
    return true;
  }
  return false;
}

}  // namespace

pkv_status pkv_bm_append_slot(pkv_block_manager* bm, int32_t seq, int32_t* slot_out, int32_t* cow_pair_out) {
  if (!bm || !slot_out || !cow_pair_out) return PKV_ERR_INVALID;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PKV_ERR_INVALID;
  if (it->second.length == INT32_MAX) return PKV_ERR_INVALID;
  std::unordered_map<int32_t, int32_t> pending;
  if (append_needs_block(bm, it->second, pending) && bm->available() < 1) return PKV_ERR_OUT_OF_BLOCKS;
  *slot_out = append_one(bm, it->second, cow_pair_out);
  return PKV_OK;
}

pkv_status pkv_bm_step(pkv_block_manager* bm, const int32_t* seqs, int32_t n,
                       int32_t* slot_mapping_out, int32_t* pairs_out, int32_t* num_pairs_out) {
  if (!bm || n < 0 || (n > 0 && (!seqs || !slot_mapping_out || !pairs_out)) || !num_pairs_out)
    return PKV_ERR_INVALID;
  std::vector<pkv_block_manager::Seq*> targets;
  targets.reserve(static_cast<size_t>(n));
  std::unordered_map<int32_t, int32_t> seen;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end() || seen.count(seqs[i]) || it->second.length == INT32_MAX)
      return PKV_ERR_INVALID;
    seen[seqs[i]] = 1;
    targets.push_back(&it->second);
  }
  std::unordered_map<int32_t, int32_t> pending;
  int64_t need = 0;
  for (auto* s : targets) need += append_needs_block(bm, *s, pending) ? 1 : 0;
  if (need > bm->available()) return PKV_ERR_OUT_OF_BLOCKS;
  int32_t np = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t cow[2];
    slot_mapping_out[i] = append_one(bm, *targets[static_cast<size_t>(i)], cow);
    if (cow[0] >= 0) {
      pairs_out[2 * np] = cow[0];
      pairs_out[2 * np + 1] = cow[1];
      ++np;
    }
  }
  *num_pairs_out = np;
  return PKV_OK;
}

pkv_status pkv_bm_free(pkv_block_manager* bm, int32_t seq) {
  if (!bm) return PKV_ERR_INVALID;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PKV_ERR_INVALID;
  for (int32_t b : it->second.blocks) {
    if (--bm->ref[static_cast<size_t>(b)] == 0) bm->give_back(b);
  }
  bm->seqs.erase(it);
  return PKV_OK;
}

pkv_status pkv_bm_block_table(const pkv_block_manager* bm, const int32_t* seqs, int32_t n,
                              int32_t max_blocks, int32_t* table_out, int32_t* context_lens_out) {
  if (!bm || n < 0 || max_blocks < 0 || (n > 0 && (!seqs || !table_out))) return PKV_ERR_INVALID;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return PKV_ERR_INVALID;
    if (static_cast<int64_t>(it->second.blocks.size()) > max_blocks) return PKV_ERR_INVALID;
  }
  for (int32_t i = 0; i < n; ++i) {
    const auto& s = bm->seqs.find(seqs[i])->second;
    int32_t* row = table_out + static_cast<int64_t>(i) * max_blocks;
    const int32_t nb = static_cast<int32_t>(s.blocks.size());
    for (int32_t j = 0; j < max_blocks; ++j) row[j] = j < nb ? s.blocks[static_cast<size_t>(j)] : -1;
    if (context_lens_out) context_lens_out[i] = s.length;
  }
  return PKV_OK;
}

int32_t pkv_bm_num_free(const pkv_block_manager* bm) { return bm ? bm->available() : -1; }

int32_t pkv_bm_refcount(const pkv_block_manager* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->ref[static_cast<size_t>(block)];
}

int32_t pkv_bm_length(const pkv_block_manager* bm, int32_t seq) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -1 : it->second.length;
}

int32_t pkv_bm_num_seq_blocks(const pkv_block_manager* bm, int32_t seq) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -1 : static_cast<int32_t>(it->second.blocks.size());
}

int32_t pkv_bm_waste(const pkv_block_manager* bm, int32_t seq) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return -1;
  return static_cast<int32_t>(static_cast<int64_t>(it->second.blocks.size()) * bm->block_size -
                              it->second.length);
}

pkv_status pkv_bm_add_cached(pkv_block_manager* bm, int32_t seq, int32_t num_tokens, const int32_t* token_ids,
                             int32_t* slots_out, int32_t* num_cached_out) {
  if (!bm || num_tokens < 0 || (num_tokens > 0 && !token_ids) || !num_cached_out) return PKV_ERR_INVALID;
  if (bm->seqs.count(seq)) return PKV_ERR_INVALID;
  const int32_t bs = bm->block_size;
  const int32_t full = num_tokens / bs;
  // longest run of registered full blocks matching the prompt
  std::vector<int32_t> hits;
  int64_t parent = 0;
  int32_t revived = 0;
  for (int32_t j = 0; j < full; ++j) {
    auto it = bm->cache.find(bm->key(parent, token_ids + static_cast<int64_t>(j) * bs));
    if (it == bm->cache.end()) break;
    hits.push_back(it->second);
    revived += bm->in_ev[static_cast<size_t>(it->second)] ? 1 : 0;
    parent = bm->node[static_cast<size_t>(it->second)];
  }
  const int64_t need = (static_cast<int64_t>(num_tokens) + bs - 1) / bs - static_cast<int64_t>(hits.size());
  if (need > bm->available() - revived) return PKV_ERR_OUT_OF_BLOCKS;

  pkv_block_manager::Seq s;
  s.blocks.reserve(hits.size() + static_cast<size_t>(need));
  for (int32_t b : hits) {
    if (bm->in_ev[static_cast<size_t>(b)]) {
      bm->leave_evictable(b);
      bm->ref[static_cast<size_t>(b)] = 1;
    } else {
      ++bm->ref[static_cast<size_t>(b)];
    }
    s.blocks.push_back(b);
  }
  s.chain = parent;
  for (int64_t i = 0; i < need; ++i) {
    const int32_t j = static_cast<int32_t>(hits.size() + i);
    const int32_t b = bm->take();
    s.blocks.push_back(b);
    if (j < full) bm->on_full(s, b, token_ids + static_cast<int64_t>(j) * bs);
  }
  s.length = num_tokens;
  s.tail.assign(token_ids + static_cast<int64_t>(full) * bs, token_ids + num_tokens);
  if (slots_out)
    for (int32_t t = 0; t < num_tokens; ++t) slots_out[t] = bm->slot(s, t);
  *num_cached_out = static_cast<int32_t>(hits.size()) * bs;
  bm->seqs.emplace(seq, std::move(s));
  return PKV_OK;
}

pkv_status pkv_bm_append_token(pkv_block_manager* bm, int32_t seq, int32_t token_id, int32_t* slot_out,
                               int32_t* cow_pair_out) {
  if (!bm || !slot_out || !cow_pair_out) return PKV_ERR_INVALID;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PKV_ERR_INVALID;
  pkv_block_manager::Seq& s = it->second;
  if (s.length == INT32_MAX) return PKV_ERR_INVALID;
  std::unordered_map<int32_t, int32_t> pending;
  if (append_needs_block(bm, s, pending) && bm->available() < 1) return PKV_ERR_OUT_OF_BLOCKS;
  const int64_t chain = s.chain;
  std::vector<int32_t> tail = std::move(s.tail);
  *slot_out = append_one(bm, s, cow_pair_out);  // clears chain and tail
  if (chain < 0) return PKV_OK;
  s.chain = chain;
  s.tail = std::move(tail);
  s.tail.push_back(token_id);
  if (static_cast<int32_t>(s.tail.size()) == bm->block_size) {
    bm->on_full(s, s.blocks.back(), s.tail.data());
    s.tail.clear();
  }
  return PKV_OK;
}

int32_t pkv_bm_num_evictable(const pkv_block_manager* bm) {
  return bm ? static_cast<int32_t>(bm->evictable.size()) : -1;
}

int32_t pkv_bm_free_list(const pkv_block_manager* bm, int32_t* out, int32_t capacity) {
  if (!bm) return -1;
  const int32_t n = bm->count < capacity ? bm->count : capacity;
  for (int32_t i = 0; out && i < n; ++i) out[i] = bm->ring[static_cast<size_t>((bm->head + i) % bm->num_blocks)];
  return bm->count;
}

}  // extern "C"
