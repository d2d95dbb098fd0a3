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
//
// The pool is held lazily, so that creating a manager costs O(1) memory
// whatever num_blocks is: blocks that were never handed out are the range
// [fresh, num_blocks), taken in increasing order, and only returned blocks
// sit on an explicit stack above it. That is the same order as a stack
// initialised to num_blocks - 1 .. 0 (top = 0). Reference counts exist for
// blocks below `fresh` only.
//
// No C++ exception leaves this file: every entry point catches them and
// returns PA_ERR_NOMEM. Each mutating call reserves the memory it may need
// before it changes anything, so a failed allocation leaves the manager as it
// was.

#include "pa_blocks.h"

#include <algorithm>
#include <cstdint>
#include <new>
#include <unordered_map>
#include <vector>

struct pa_block_manager {
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t length = 0;
  };
  int64_t num_blocks = 0;
  int32_t block_size = 0;
  int32_t capacity = 0;
  int64_t fresh = 0;                // blocks [fresh, num_blocks) were never taken
  std::vector<int32_t> free_stack;  // returned blocks, top = back
  std::vector<int32_t> refcount;    // [fresh]
  std::unordered_map<int64_t, Seq> seqs;
  std::vector<int64_t> copies;      // queued (src, dst) pairs, flattened
  size_t copies_head = 0;           // first pair not yet taken (in pairs)

  int64_t num_free() const { return (int64_t)free_stack.size() + (num_blocks - fresh); }

  // Needs refcount capacity for one more fresh block (reserved by the caller).
  int32_t take() {
    if (!free_stack.empty()) {
      const int32_t b = free_stack.back();
      free_stack.pop_back();
      refcount[(size_t)b] = 1;
      return b;
    }
    const int32_t b = (int32_t)fresh++;
    refcount.push_back(1);
    return b;
  }

  int64_t needed(const Seq& s, int64_t k) const {
    if (k <= 0) return 0;
    const int64_t n = s.length, bs = block_size;
    // positions p in [n, n + k) with p % bs == 0
    const int64_t first = (n + bs - 1) / bs * bs;
    const int64_t fresh_blocks = first < n + k ? (n + k - 1 - first) / bs + 1 : 0;
    const bool cow = (n % bs) != 0 && refcount[(size_t)s.blocks.back()] > 1;
    return fresh_blocks + (cow ? 1 : 0);
  }
};

namespace {

// Capacity for n elements, growing geometrically (so that reserving before
// every mutation keeps appends amortised O(1)); may throw.
template <typename V>
void room_for(V& v, size_t n) {
  if (v.capacity() < n) v.reserve(std::max(n, 2 * v.capacity()));
}

// Runs f and turns any C++ exception into a status (none crosses the C ABI).
template <typename F>
pa_status_t guarded(F&& f) noexcept {
  try {
    return f();
  } catch (...) {
    return PA_ERR_NOMEM;
  }
}

}  // namespace

extern "C" {

pa_status_t pa_bm_create(int64_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                         pa_block_manager** out) {
  if (!out) return PA_ERR_NULL;
  *out = nullptr;
  if (num_blocks <= 0 || num_blocks > INT32_MAX || block_size <= 0 || max_blocks_per_seq <= 0)
    return PA_ERR_SHAPE;
  return guarded([&] {
    auto* bm = new pa_block_manager();
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->capacity = max_blocks_per_seq;
    *out = bm;
    return PA_OK;
  });
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

pa_status_t pa_bm_add(pa_block_manager* bm, int64_t seq) {
  if (!bm) return PA_ERR_NULL;
  return guarded([&] {
    if (bm->seqs.count(seq)) return PA_ERR_STATE;
    bm->seqs.emplace(seq, pa_block_manager::Seq{});  // unchanged if it throws
    return PA_OK;
  });
}

pa_status_t pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child) {
  if (!bm) return PA_ERR_NULL;
  return guarded([&] {
    auto it = bm->seqs.find(parent);
    if (it == bm->seqs.end() || bm->seqs.count(child)) return PA_ERR_STATE;
    pa_block_manager::Seq copy = it->second;
    // insert first (it may throw), then count the references (it cannot)
    auto& added = bm->seqs.emplace(child, std::move(copy)).first->second;
    for (int32_t b : added.blocks) ++bm->refcount[(size_t)b];
    return PA_OK;
  });
}

pa_status_t pa_bm_append(pa_block_manager* bm, int64_t seq, int32_t num_tokens, int64_t* slots) {
  if (!bm) return PA_ERR_NULL;
  return guarded([&] {
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end()) return PA_ERR_STATE;
    if (num_tokens < 0) return PA_ERR_SHAPE;
    if (num_tokens == 0) return PA_OK;
    if (!slots) return PA_ERR_NULL;
    auto& s = it->second;
    const int64_t bs = bm->block_size;
    const int64_t n = s.length, end = n + num_tokens;
    const int64_t nb_end = (end + bs - 1) / bs;
    if (nb_end > bm->capacity) return PA_ERR_SHAPE;
    const int64_t need = bm->needed(s, num_tokens);
    if (need > bm->num_free()) return PA_ERR_OUT_OF_BLOCKS;
    const bool cow = n % bs != 0 && bm->refcount[(size_t)s.blocks.back()] > 1;
    // everything that may allocate, before anything changes
    room_for(s.blocks, (size_t)nb_end);
    room_for(bm->refcount, (size_t)(bm->fresh + need));
    if (cow) room_for(bm->copies, bm->copies.size() + 2);
    if (cow) {  // copy-on-write of the shared, partly filled last block
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
  });
}

pa_status_t pa_bm_free(pa_block_manager* bm, int64_t seq) {
  if (!bm) return PA_ERR_NULL;
  return guarded([&] {
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end()) return PA_ERR_STATE;
    const auto& blocks = it->second.blocks;
    room_for(bm->free_stack, bm->free_stack.size() + blocks.size());
    for (auto b = blocks.rbegin(); b != blocks.rend(); ++b)
      if (--bm->refcount[(size_t)*b] == 0) bm->free_stack.push_back(*b);
    bm->seqs.erase(it);
    return PA_OK;
  });
}

int64_t pa_bm_num_free(const pa_block_manager* bm) { return bm ? bm->num_free() : -1; }

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
  return block < bm->fresh ? bm->refcount[(size_t)block] : 0;
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
    if (bm->seqs.find(seqs[i]) == bm->seqs.end()) return PA_ERR_STATE;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const auto& s = bm->seqs.find(seqs[i])->second;
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
  // The run's earlier pairs are in pairs[] already; a pair joins the run only
  // if it neither reads nor writes a block an earlier pair writes, and does
  // not write a block an earlier pair reads. (A linear scan: runs are as long
  // as one step's copy-on-write events, and nothing here allocates.)
  int64_t taken = 0;
  size_t i = bm->copies_head;
  while (i + 1 < bm->copies.size() && taken < max_pairs) {
    const int64_t src = bm->copies[i], dst = bm->copies[i + 1];
    bool clash = false;
    for (int64_t k = 0; k < taken && !clash; ++k) {
      const int64_t rs = pairs[2 * k], wd = pairs[2 * k + 1];
      clash = src == wd || dst == wd || dst == rs;
    }
    if (clash) break;
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

int32_t pa_find_shared_prefixes(const int32_t* block_tables, const int32_t* context_lens,
                                int32_t num_seqs, int32_t max_blocks_per_seq,
                                int32_t block_size, int32_t min_blocks, int32_t* cu_groups,
                                int32_t* prefix_lens, int32_t* max_group_size,
                                int32_t* max_prefix_len) {
  if (!block_tables || !context_lens || !cu_groups || !prefix_lens || !max_group_size ||
      !max_prefix_len || num_seqs < 0 || max_blocks_per_seq <= 0 || block_size <= 0 ||
      min_blocks < 1)
    return -1;
  *max_group_size = 0;
  *max_prefix_len = 0;
  auto blocks_of = [&](int32_t b) -> int64_t {  // table entries within the context
    const int64_t n = context_lens[b] < 0 ? 0 : context_lens[b];
    const int64_t nb = (n + block_size - 1) / block_size;
    return nb < max_blocks_per_seq ? nb : max_blocks_per_seq;
  };
  auto common = [&](int32_t a, int32_t b) -> int64_t {  // leading blocks a and b share
    const int32_t* ta = block_tables + (int64_t)a * max_blocks_per_seq;
    const int32_t* tb = block_tables + (int64_t)b * max_blocks_per_seq;
    const int64_t lim = std::min(blocks_of(a), blocks_of(b));
    int64_t k = 0;
    while (k < lim && ta[k] >= 0 && ta[k] == tb[k]) ++k;
    return k;
  };
  // group g spans cu_groups[g] .. cu_groups[g + 1] - 1
  int32_t groups = 0, last_end = -1;
  for (int32_t b = 0; b < num_seqs;) {
    int64_t shared = blocks_of(b);
    int32_t end = b + 1;
    while (end < num_seqs) {
      const int64_t k = common(b, end);
      if (k < min_blocks) break;
      shared = std::min(shared, k);
      ++end;
    }
    if (end - b < 2 || shared < min_blocks) {
      ++b;
      continue;
    }
    if (groups == 0) {
      cu_groups[0] = b;
    } else if (last_end < b) {  // the unshared sequences since the last run
      prefix_lens[groups] = 0;
      cu_groups[groups + 1] = b;
      ++groups;
    }
    prefix_lens[groups] = (int32_t)std::min<int64_t>(shared * block_size, INT32_MAX);
    cu_groups[groups + 1] = end;
    ++groups;
    *max_group_size = std::max(*max_group_size, end - b);
    *max_prefix_len = std::max(*max_prefix_len, prefix_lens[groups - 1]);
    last_end = end;
    b = end;
  }
  return groups;
}

}  // extern "C"
