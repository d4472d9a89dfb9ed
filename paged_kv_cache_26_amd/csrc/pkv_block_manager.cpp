// Host block manager (allocation, sharing, copy-on-write) and the batch grouping by shared
// leading blocks; host C++ only (the GPU block copy is in pkv_append.hip, its entry point
// in pkv_capi.cpp). The behaviour and its sources are documented in
// include/pkv_block_manager.h.

#include "../../include/pkv_block_manager.h"

#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pkv_internal.h"

struct pkv_block_manager {
  int32_t num_blocks;
  int32_t block_size;
  std::vector<int32_t> fresh;        // never-used blocks, in hand-out order
  size_t next_fresh = 0;
  std::deque<int32_t> returned;      // freed blocks, first in first out
  std::vector<int32_t> ref;          // reference count per block
  std::unordered_map<int64_t, std::vector<int32_t>> tables;

  int32_t num_free() const {
    return (int32_t)(fresh.size() - next_fresh) + (int32_t)returned.size();
  }
  // Caller checks num_free() first.
  int32_t take() {
    int32_t blk;
    if (next_fresh < fresh.size()) {
      blk = fresh[next_fresh++];
    } else {
      blk = returned.front();
      returned.pop_front();
    }
    ref[blk] = 1;
    return blk;
  }
  void release(int32_t blk) {
    if (--ref[blk] == 0) returned.push_back(blk);
  }
  int32_t blocks_for(int64_t n_tokens) const {
    return (int32_t)((n_tokens + block_size - 1) / block_size);
  }
};

extern "C" {

pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size,
                                 const int32_t* free_order) {
  if (num_blocks <= 0 || block_size <= 0) return nullptr;
  pkv_block_manager* bm = new (std::nothrow) pkv_block_manager();
  if (!bm) return nullptr;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->ref.assign(num_blocks, 0);
  bm->fresh.resize(num_blocks);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {   // not a permutation
        delete bm;
        return nullptr;
      }
      seen[b] = 1;
      bm->fresh[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) bm->fresh[i] = i;
  }
  return bm;
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int32_t pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id) {
  if (!bm) return PKV_ERR_NULL;
  if (bm->tables.count(seq_id)) return PKV_ERR_SEQUENCE_EXISTS;
  bm->tables.emplace(seq_id, std::vector<int32_t>());
  return PKV_OK;
}

int32_t pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child) {
  if (!bm) return PKV_ERR_NULL;
  auto it = bm->tables.find(parent);
  if (it == bm->tables.end()) return PKV_ERR_NO_SEQUENCE;
  if (bm->tables.count(child)) return PKV_ERR_SEQUENCE_EXISTS;
  std::vector<int32_t> copy = it->second;
  for (int32_t b : copy) ++bm->ref[b];
  bm->tables.emplace(child, std::move(copy));
  return PKV_OK;
}

int32_t pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq_id) {
  if (!bm) return PKV_ERR_NULL;
  auto it = bm->tables.find(seq_id);
  if (it == bm->tables.end()) return PKV_ERR_NO_SEQUENCE;
  for (int32_t b : it->second) bm->release(b);
  bm->tables.erase(it);
  return PKV_OK;
}

int32_t pkv_bm_grow(pkv_block_manager* bm, int64_t seq_id, int32_t n_tokens) {
  if (!bm) return PKV_ERR_NULL;
  if (n_tokens < 0) return PKV_ERR_SHAPE;
  auto it = bm->tables.find(seq_id);
  if (it == bm->tables.end()) return PKV_ERR_NO_SEQUENCE;
  std::vector<int32_t>& t = it->second;
  const int32_t need = bm->blocks_for(n_tokens) - (int32_t)t.size();
  if (need <= 0) return PKV_OK;
  if (need > bm->num_free()) return PKV_ERR_OUT_OF_BLOCKS;
  for (int32_t i = 0; i < need; ++i) t.push_back(bm->take());
  return PKV_OK;
}

int32_t pkv_bm_append_slot(pkv_block_manager* bm, int64_t seq_id, int32_t token_index,
                           int32_t* phys_block, int32_t* slot, int32_t* copy_src,
                           int32_t* copy_dst) {
  if (!bm) return PKV_ERR_NULL;
  if (token_index < 0) return PKV_ERR_SHAPE;
  auto it = bm->tables.find(seq_id);
  if (it == bm->tables.end()) return PKV_ERR_NO_SEQUENCE;
  std::vector<int32_t>& t = it->second;
  const int32_t logical = token_index / bm->block_size;
  const int32_t grow = logical + 1 - (int32_t)t.size();
  // A block reached without growing may be shared: it then needs one more block.
  const bool cow = grow <= 0 && bm->ref[t[logical]] > 1;
  const int32_t need = (grow > 0 ? grow : 0) + (cow ? 1 : 0);
  if (need > bm->num_free()) return PKV_ERR_OUT_OF_BLOCKS;
  for (int32_t i = 0; i < grow; ++i) t.push_back(bm->take());
  int32_t src = -1, dst = -1;
  if (cow) {
    src = t[logical];
    dst = bm->take();
    bm->release(src);
    t[logical] = dst;
  }
  if (phys_block) *phys_block = t[logical];
  if (slot) *slot = token_index % bm->block_size;
  if (copy_src) *copy_src = src;
  if (copy_dst) *copy_dst = dst;
  return PKV_OK;
}

int32_t pkv_bm_append_slots(pkv_block_manager* bm, const int64_t* seq_ids,
                            const int32_t* token_index, int32_t n, int32_t* phys_block,
                            int32_t* slot, int32_t* copy_pairs, int32_t* n_done) {
  if (n_done) *n_done = 0;
  if (!bm || (n > 0 && (!seq_ids || !token_index))) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  for (int32_t i = 0; i < n; ++i) {
    int32_t pb, sl, src, dst;
    const int32_t st = pkv_bm_append_slot(bm, seq_ids[i], token_index[i], &pb, &sl, &src, &dst);
    if (st != PKV_OK) return st;
    if (phys_block) phys_block[i] = pb;
    if (slot) slot[i] = sl;
    if (copy_pairs) {
      copy_pairs[2 * i] = src;
      copy_pairs[2 * i + 1] = dst;
    }
    if (n_done) *n_done = i + 1;
  }
  return PKV_OK;
}

int32_t pkv_bm_num_free(const pkv_block_manager* bm) {
  return bm ? bm->num_free() : PKV_ERR_NULL;
}

int32_t pkv_bm_refcount(const pkv_block_manager* bm, int32_t block) {
  if (!bm) return PKV_ERR_NULL;
  if (block < 0 || block >= bm->num_blocks) return PKV_ERR_BAD_BLOCK;
  return bm->ref[block];
}

int32_t pkv_bm_num_blocks_of(const pkv_block_manager* bm, int64_t seq_id) {
  if (!bm) return PKV_ERR_NULL;
  auto it = bm->tables.find(seq_id);
  return it == bm->tables.end() ? PKV_ERR_NO_SEQUENCE : (int32_t)it->second.size();
}

int32_t pkv_bm_tables(const pkv_block_manager* bm, const int64_t* seq_ids, int32_t n,
                      int32_t max_blocks, int32_t* out) {
  if (!bm || (n > 0 && (!seq_ids || !out))) return PKV_ERR_NULL;
  if (n < 0 || max_blocks < 0) return PKV_ERR_SHAPE;
  for (int32_t i = 0; i < n; ++i) {          // check everything before writing
    auto it = bm->tables.find(seq_ids[i]);
    if (it == bm->tables.end()) return PKV_ERR_NO_SEQUENCE;
    if ((int32_t)it->second.size() > max_blocks) return PKV_ERR_SHAPE;
  }
  for (int32_t i = 0; i < n; ++i) {
    const std::vector<int32_t>& t = bm->tables.find(seq_ids[i])->second;
    int32_t* row = out + (size_t)i * max_blocks;
    for (int32_t k = 0; k < max_blocks; ++k) row[k] = k < (int32_t)t.size() ? t[k] : -1;
  }
  return PKV_OK;
}

int32_t pkv_find_shared_prefixes(const int32_t* tables, int32_t num_seqs, int32_t max_blocks,
                                 const int32_t* context_lens, int32_t block_size,
                                 int32_t min_members, int32_t* seq_group, int32_t* group_blocks,
                                 int32_t* n_groups, int32_t* max_group_size,
                                 int32_t* max_shared_blocks) {
  if (!n_groups || !max_group_size || !max_shared_blocks) return PKV_ERR_NULL;
  if (num_seqs > 0 && (!tables || !context_lens || !seq_group || !group_blocks))
    return PKV_ERR_NULL;
  if (num_seqs < 0 || max_blocks < 0 || block_size <= 0 || min_members < 2) return PKV_ERR_SHAPE;
  *n_groups = 0;
  *max_group_size = 0;
  *max_shared_blocks = 0;
  // candidates: sequences with at least one whole block before their last token, keyed by
  // their first physical block, in order of first appearance
  std::unordered_map<int32_t, int32_t> slot_of;
  std::vector<std::vector<int32_t>> sets;
  for (int32_t b = 0; b < num_seqs; ++b) {
    seq_group[b] = -1;
    const int32_t n = context_lens[b];
    if (n <= block_size || max_blocks == 0) continue;
    const int32_t first = tables[(size_t)b * max_blocks];
    if (first < 0) continue;
    auto ins = slot_of.emplace(first, (int32_t)sets.size());
    if (ins.second) sets.emplace_back();
    sets[ins.first->second].push_back(b);
  }
  for (const std::vector<int32_t>& m : sets) {
    if ((int32_t)m.size() < min_members) continue;
    const int32_t* lead = tables + (size_t)m[0] * max_blocks;
    int32_t sb = max_blocks;
    for (int32_t b : m) {
      const int32_t* row = tables + (size_t)b * max_blocks;
      int32_t k = 0;
      const int32_t own = (context_lens[b] - 1) / block_size;   // blocks before the last token
      const int32_t lim = own < sb ? own : sb;
      while (k < lim && row[k] == lead[k] && row[k] >= 0) ++k;
      sb = k;
    }
    if (sb == 0) continue;
    const int32_t g = (*n_groups)++;
    group_blocks[g] = sb;
    for (int32_t b : m) seq_group[b] = g;
    if ((int32_t)m.size() > *max_group_size) *max_group_size = (int32_t)m.size();
    if (sb > *max_shared_blocks) *max_shared_blocks = sb;
  }
  return PKV_OK;
}

}  // extern "C"
