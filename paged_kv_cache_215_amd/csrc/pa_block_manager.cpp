// Host-side block manager of the paged KV cache (declared in
// include/pa_blocks.h): a stack of free blocks, per-block reference counts,
// per-sequence tables, and a queue of copy-on-write block copies.
//
// What it follows: blocks are taken only as tokens arrive and return to the
// pool as soon as a sequence ends (How vLLM gets real throughput on H100s,
// "PagedAttention borrows from operating systems" and "Continuous batching
// removes straggler bubbles"); sequences forked from one prompt share its
// blocks and a shared block is copied only when one of them writes into it
// (Dissecting vLLM, "PagedAttention: Virtual Memory for KV Cache").
//
// Every operation is O(tokens touched + blocks touched); an append first
// counts the blocks it needs, so a failing call leaves the state unchanged.

#include "pa_blocks.h"

#include <algorithm>
#include <cstdint>
#include <unordered_map>
#include <unordered_set>
#include <vector>

struct pa_block_manager {
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t length = 0;
  };
  int64_t num_blocks = 0;
  int32_t block_size = 0;
  int32_t capacity = 0;
  std::vector<int32_t> free_stack;  // top = back
  std::vector<int32_t> refcount;
  std::unordered_map<int64_t, Seq> seqs;
  std::vector<int64_t> copies;      // queued (src, dst) pairs, flattened
  size_t copies_head = 0;           // first pair not yet taken (in pairs)

  int32_t take() {
    const int32_t b = free_stack.back();
    free_stack.pop_back();
    refcount[b] = 1;
    return b;
  }

  int64_t needed(const Seq& s, int64_t k) const {
    if (k <= 0) return 0;
    const int64_t n = s.length, bs = block_size;
    // positions p in [n, n + k) with p % bs == 0
    const int64_t first = (n + bs - 1) / bs * bs;
    const int64_t fresh = first < n + k ? (n + k - 1 - first) / bs + 1 : 0;
    const bool cow = (n % bs) != 0 && refcount[s.blocks.back()] > 1;
    return fresh + (cow ? 1 : 0);
  }
};

extern "C" {

pa_status_t pa_bm_create(int64_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                         pa_block_manager** out) {
  if (!out) return PA_ERR_NULL;
  *out = nullptr;
  if (num_blocks <= 0 || num_blocks > INT32_MAX || block_size <= 0 || max_blocks_per_seq <= 0)
    return PA_ERR_SHAPE;
  auto* bm = new pa_block_manager();
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->capacity = max_blocks_per_seq;
  bm->free_stack.resize((size_t)num_blocks);
  for (int64_t i = 0; i < num_blocks; ++i) bm->free_stack[(size_t)i] = (int32_t)(num_blocks - 1 - i);
  bm->refcount.assign((size_t)num_blocks, 0);
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

pa_status_t pa_bm_add(pa_block_manager* bm, int64_t seq) {
  if (!bm) return PA_ERR_NULL;
  if (bm->seqs.count(seq)) return PA_ERR_STATE;
  bm->seqs.emplace(seq, pa_block_manager::Seq{});
  return PA_OK;
}

pa_status_t pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end() || bm->seqs.count(child)) return PA_ERR_STATE;
  pa_block_manager::Seq copy = it->second;
  for (int32_t b : copy.blocks) ++bm->refcount[(size_t)b];
  bm->seqs.emplace(child, std::move(copy));
  return PA_OK;
}

pa_status_t pa_bm_append(pa_block_manager* bm, int64_t seq, int32_t num_tokens, int64_t* slots) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_ERR_STATE;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!slots) return PA_ERR_NULL;
  auto& s = it->second;
  const int64_t bs = bm->block_size;
  const int64_t n = s.length, end = n + num_tokens;
  if ((end + bs - 1) / bs > bm->capacity) return PA_ERR_SHAPE;
  if (bm->needed(s, num_tokens) > (int64_t)bm->free_stack.size()) return PA_ERR_OUT_OF_BLOCKS;
  if (n % bs != 0 && bm->refcount[(size_t)s.blocks.back()] > 1) {  // copy-on-write
    const int32_t src = s.blocks.back();
    const int32_t dst = bm->take();
    --bm->refcount[(size_t)src];
    s.blocks.back() = dst;
    bm->copies.push_back(src);
    bm->copies.push_back(dst);
  }
  for (int64_t p = n; p < end; ++p) {
    if (p % bs == 0) s.blocks.push_back(bm->take());
    slots[p - n] = (int64_t)s.blocks[(size_t)(p / bs)] * bs + p % bs;
  }
  s.length = end;
  return PA_OK;
}

pa_status_t pa_bm_free(pa_block_manager* bm, int64_t seq) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_ERR_STATE;
  const auto& blocks = it->second.blocks;
  for (auto b = blocks.rbegin(); b != blocks.rend(); ++b)
    if (--bm->refcount[(size_t)*b] == 0) bm->free_stack.push_back(*b);
  bm->seqs.erase(it);
  return PA_OK;
}

int64_t pa_bm_num_free(const pa_block_manager* bm) {
  return bm ? (int64_t)bm->free_stack.size() : -1;
}

int64_t pa_bm_length(const pa_block_manager* bm, int64_t seq) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -1 : it->second.length;
}

int64_t pa_bm_blocks_needed(const pa_block_manager* bm, int64_t seq, int32_t num_tokens) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -1 : bm->needed(it->second, num_tokens);
}

int32_t pa_bm_refcount(const pa_block_manager* bm, int64_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->refcount[(size_t)block];
}

int32_t pa_bm_table(const pa_block_manager* bm, int64_t seq, int32_t* out, int32_t capacity) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return -1;
  const auto& blocks = it->second.blocks;
  if (out) {
    for (int32_t i = 0; i < capacity; ++i)
      out[i] = (size_t)i < blocks.size() ? blocks[(size_t)i] : -1;
  }
  return (int32_t)blocks.size();
}

pa_status_t pa_bm_tables(const pa_block_manager* bm, const int64_t* seqs, int32_t num_seqs,
                         int32_t* tables, int32_t row_stride, int32_t* context_lens) {
  if (!bm) return PA_ERR_NULL;
  if (num_seqs < 0 || row_stride < bm->capacity) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!seqs || !tables || !context_lens) return PA_ERR_NULL;
  for (int32_t i = 0; i < num_seqs; ++i)
    if (!bm->seqs.count(seqs[i])) return PA_ERR_STATE;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const auto& s = bm->seqs.at(seqs[i]);
    int32_t* row = tables + (int64_t)i * row_stride;
    const size_t nb = s.blocks.size();
    std::copy(s.blocks.begin(), s.blocks.end(), row);
    std::fill(row + nb, row + row_stride, -1);
    context_lens[i] = (int32_t)s.length;
  }
  return PA_OK;
}

int64_t pa_bm_take_copies(pa_block_manager* bm, int64_t* pairs, int64_t max_pairs) {
  if (!bm || !pairs || max_pairs <= 0) return 0;
  std::unordered_set<int64_t> written, read;
  int64_t taken = 0;
  size_t i = bm->copies_head;
  while (i + 1 < bm->copies.size() && taken < max_pairs) {
    const int64_t src = bm->copies[i], dst = bm->copies[i + 1];
    if (written.count(src) || written.count(dst) || read.count(dst)) break;
    written.insert(dst);
    read.insert(src);
    pairs[2 * taken] = src;
    pairs[2 * taken + 1] = dst;
    ++taken;
    i += 2;
  }
  bm->copies_head = i;
  if (bm->copies_head == bm->copies.size()) {
    bm->copies.clear();
    bm->copies_head = 0;
  }
  return taken;
}

}  // extern "C"
