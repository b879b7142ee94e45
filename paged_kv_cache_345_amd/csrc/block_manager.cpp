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

#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"

struct pkv_block_manager {
  struct Seq {
    std::vector<int32_t> blocks;
    int32_t length = 0;
  };

  int32_t num_blocks = 0;
  int32_t block_size = 0;
  // free list as a ring buffer of capacity num_blocks
  std::vector<int32_t> ring;
  int64_t head = 0;  // index of the front element
  int32_t count = 0; // number of free blocks
  std::vector<int32_t> ref;
  std::unordered_map<int32_t, Seq> seqs;

  int32_t take() {
    int32_t b = ring[static_cast<size_t>(head)];
    head = (head + 1) % num_blocks;
    --count;
    ref[static_cast<size_t>(b)] = 1;
    return b;
  }
  void give_back(int32_t b) {
    ring[static_cast<size_t>((head + count) % num_blocks)] = b;
    ++count;
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
  if (need > bm->count) return PKV_ERR_OUT_OF_BLOCKS;
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
  if (append_needs_block(bm, it->second, pending) && bm->count < 1) return PKV_ERR_OUT_OF_BLOCKS;
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
  if (need > bm->count) return PKV_ERR_OUT_OF_BLOCKS;
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

int32_t pkv_bm_num_free(const pkv_block_manager* bm) { return bm ? bm->count : -1; }

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

int32_t pkv_bm_free_list(const pkv_block_manager* bm, int32_t* out, int32_t capacity) {
  if (!bm) return -1;
  const int32_t n = bm->count < capacity ? bm->count : capacity;
  for (int32_t i = 0; out && i < n; ++i) out[i] = bm->ring[static_cast<size_t>((bm->head + i) % bm->num_blocks)];
  return bm->count;
}

}  // extern "C"
