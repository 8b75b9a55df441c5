// Host-side block manager of a paged KV cache (C ABI in include/pa.h).
//
// The pages describe the bookkeeping around the kernels ("vLLM 前世今生" §3.2
// and §3.3; "vLLM" note, section "PagedAttention"): a sequence's cache grows in
// fixed-size blocks taken from a shared pool on demand and returned when the
// sequence finishes; free blocks are kept in a list so both take O(1); a block
// may be shared by several sequences (forked decoding, shared prompt prefixes)
// and is copied before a sequence writes into it while it is shared
// (copy-on-write). This file keeps that state and emits what the device side
// needs: the slot of each appended token, the (source, destination) block
// pairs to copy, and dense block tables.
//
// Data layout: the free list is a stack of block ids; every block has a
// reference count; every live sequence has its block list and its length.
// Nothing here touches device memory.
#include <algorithm>
#include <cstdint>
#include <unordered_map>
#include <vector>

#include "pa.h"
#include "pa_error.h"

namespace {

struct Seq {
  std::vector<int32_t> blocks;
  int64_t len = 0;
};

}  // namespace

struct pa_block_manager {
  int block_size = 16;
  int max_blocks_per_seq = 0;
  std::vector<int32_t> free_list;  // stack: allocate from the back, free onto the back
  std::vector<int32_t> refcount;
  std::unordered_map<int64_t, Seq> seqs;

  int32_t take() {
    const int32_t b = free_list.back();
    free_list.pop_back();
    refcount[b] = 1;
    return b;
  }
  void release(int32_t b) {
    if (--refcount[b] == 0) free_list.push_back(b);
  }
};

extern "C" {

pa_block_manager* pa_bm_create(int64_t num_blocks, int block_size, int max_blocks_per_seq) {
  if (num_blocks < 1 || num_blocks > INT32_MAX || block_size != 16 || max_blocks_per_seq < 1) {
    pa::fail(PA_ERR_SHAPE, "bm_create: need num_blocks in [1, 2^31), block_size 16, max_blocks_per_seq >= 1");
    return nullptr;
  }
  auto* bm = new pa_block_manager;
  bm->block_size = block_size;
  bm->max_blocks_per_seq = max_blocks_per_seq;
  bm->refcount.assign((size_t)num_blocks, 0);
  bm->free_list.reserve((size_t)num_blocks);
  for (int64_t b = num_blocks - 1; b >= 0; --b) bm->free_list.push_back((int32_t)b);  // block 0 is taken first
  return bm;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int64_t pa_bm_num_free_blocks(const pa_block_manager* bm) { return bm ? (int64_t)bm->free_list.size() : -1; }

int pa_bm_add_sequence(pa_block_manager* bm, int64_t seq_id) {
  if (!bm) return pa::fail(PA_ERR_NULL, "bm_add_sequence: NULL manager");
  if (!bm->seqs.emplace(seq_id, Seq{}).second)
    return pa::fail(PA_ERR_STATE, "bm_add_sequence: sequence %lld already exists", (long long)seq_id);
  return pa::ok();
}

int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child) {
  if (!bm) return pa::fail(PA_ERR_NULL, "bm_fork: NULL manager");
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return pa::fail(PA_ERR_STATE, "bm_fork: no sequence %lld", (long long)parent);
  if (bm->seqs.count(child)) return pa::fail(PA_ERR_STATE, "bm_fork: sequence %lld already exists", (long long)child);
  Seq s = it->second;  // copy: same blocks, same length
  for (int32_t b : s.blocks) ++bm->refcount[b];
  bm->seqs.emplace(child, std::move(s));
  return pa::ok();
}

int pa_bm_free_sequence(pa_block_manager* bm, int64_t seq_id) {
  if (!bm) return pa::fail(PA_ERR_NULL, "bm_free_sequence: NULL manager");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return pa::fail(PA_ERR_STATE, "bm_free_sequence: no sequence %lld", (long long)seq_id);
  for (int32_t b : it->second.blocks) bm->release(b);
  bm->seqs.erase(it);
  return pa::ok();
}

int pa_bm_append_slots(pa_block_manager* bm, const int64_t* seq_ids, int n, int64_t* slots_out, int32_t* cow_src,
                       int32_t* cow_dst, int* num_cow) {
  if (!bm || (n > 0 && (!seq_ids || !slots_out || !cow_src || !cow_dst)) || !num_cow)
    return pa::fail(PA_ERR_NULL, "bm_append_slots: NULL argument");
  *num_cow = 0;
  // Check everything first so that a failing call changes nothing. The block
  // count is exact: when several listed sequences share a last block, every
  // one but the last writer to reach it copies it (its count drops as they go).
  int64_t need = 0;
  std::unordered_map<int32_t, int32_t> shared_left;  // remaining holders of shared last blocks
  for (int i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return pa::fail(PA_ERR_STATE, "bm_append_slots: no sequence %lld", (long long)seq_ids[i]);
    for (int k = 0; k < i; ++k)
      if (seq_ids[k] == seq_ids[i])
        return pa::fail(PA_ERR_STATE, "bm_append_slots: sequence %lld listed twice", (long long)seq_ids[i]);
    const Seq& s = it->second;
    if (s.len % bm->block_size == 0) {
      if ((int64_t)s.blocks.size() >= bm->max_blocks_per_seq)
        return pa::fail(PA_ERR_CAPACITY, "bm_append_slots: sequence %lld would exceed %d blocks",
                       (long long)seq_ids[i], bm->max_blocks_per_seq);
      ++need;
    } else {
      const int32_t last = s.blocks.back();
      auto sl = shared_left.emplace(last, bm->refcount[last]).first;
      if (sl->second > 1) {
        ++need;
        --sl->second;
      }
    }
  }
  if (need > (int64_t)bm->free_list.size())
    return pa::fail(PA_ERR_CAPACITY, "bm_append_slots: %lld free blocks needed, %zu left", (long long)need,
                   bm->free_list.size());
  for (int i = 0; i < n; ++i) {
    Seq& s = bm->seqs[seq_ids[i]];
    const int64_t off = s.len % bm->block_size;
    if (off == 0) {
      s.blocks.push_back(bm->take());
    } else if (bm->refcount[s.blocks.back()] > 1) {
      // The last block is shared and this sequence is about to write into it:
      // give the sequence its own copy first.
      const int32_t src = s.blocks.back();
      const int32_t dst = bm->take();
      bm->release(src);
      s.blocks.back() = dst;
      cow_src[*num_cow] = src;
      cow_dst[*num_cow] = dst;
      ++*num_cow;
    }
    slots_out[i] = (int64_t)s.blocks.back() * bm->block_size + off;
    ++s.len;
  }
  return pa::ok();
}

int pa_bm_block_tables(const pa_block_manager* bm, const int64_t* seq_ids, int n, int32_t* tables_out,
                       int max_blocks, int32_t* lens_out) {
  if (!bm || (n > 0 && (!seq_ids || !tables_out || !lens_out)))
    return pa::fail(PA_ERR_NULL, "bm_block_tables: NULL argument");
  for (int i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return pa::fail(PA_ERR_STATE, "bm_block_tables: no sequence %lld", (long long)seq_ids[i]);
    const Seq& s = it->second;
    if ((int64_t)s.blocks.size() > max_blocks)
      return pa::fail(PA_ERR_SHAPE, "bm_block_tables: sequence %lld holds %zu blocks, table rows hold %d",
                     (long long)seq_ids[i], s.blocks.size(), max_blocks);
    int32_t* row = tables_out + (int64_t)i * max_blocks;
    for (int j = 0; j < max_blocks; ++j) row[j] = j < (int)s.blocks.size() ? s.blocks[j] : -1;
    lens_out[i] = (int32_t)s.len;
  }
  return pa::ok();
}

int pa_bm_shared_prefix(const pa_block_manager* bm, const int64_t* seq_ids, int n, int min_blocks,
                        int32_t* groups_out, int max_groups, int* num_groups) {
  if (!bm || (n > 0 && !seq_ids) || (max_groups > 0 && !groups_out) || !num_groups)
    return pa::fail(PA_ERR_NULL, "bm_shared_prefix: NULL argument");
  if (min_blocks < 1 || max_groups < 0)
    return pa::fail(PA_ERR_SHAPE, "bm_shared_prefix: min_blocks must be >= 1 and max_groups >= 0");
  *num_groups = 0;
  std::vector<const Seq*> list((size_t)(n > 0 ? n : 0));
  for (int i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end())
      return pa::fail(PA_ERR_STATE, "bm_shared_prefix: no sequence %lld", (long long)seq_ids[i]);
    list[(size_t)i] = &it->second;
  }
  // Leading blocks two sequences hold in common, counting only blocks full in
  // both (a shared block is never written again once full, so those stay
  // shared; a shared partial block is copied before either writes into it).
  auto common = [&](const Seq& a, const Seq& b) {
    const int64_t full = std::min(a.len, b.len) / bm->block_size;
    int64_t j = 0;
    while (j < full && a.blocks[(size_t)j] == b.blocks[(size_t)j]) ++j;
    return j;
  };
  // A group: a maximal run of consecutive listed sequences that each share at
  // least min_blocks leading blocks with the run's first; its count of shared
  // blocks is the smallest of those.
  for (int i = 0; i < n;) {
    int end = i + 1;
    int64_t shared = INT64_MAX;
    while (end < n) {
      const int64_t c = common(*list[(size_t)i], *list[(size_t)end]);
      if (c < min_blocks) break;
      shared = std::min(shared, c);
      ++end;
    }
    if (end - i >= 2 && *num_groups < max_groups) {
      int32_t* g = groups_out + 3 * (int64_t)*num_groups;
      g[0] = i;
      g[1] = end - i;
      g[2] = (int32_t)shared;
      ++*num_groups;
    }
    i = end;
  }
  return pa::ok();
}

int pa_bm_block_refcount(const pa_block_manager* bm, int32_t block) {
  if (!bm || block < 0 || block >= (int32_t)bm->refcount.size()) return -1;
  return bm->refcount[block];
}

}  // extern "C"
