// Iteration-level batching scheduler (declared in include/pa_sched.h): the
// host side of a continuous-batching step. It drives a native block manager
// for the device pool and a stack of host blocks for the swap space, and
// writes each iteration's plan (decode batch, prefill chunks, swap copies)
// into buffers it owns.
//
// The host swap space is held lazily, like the block manager's pool: blocks
// [host_fresh, num_host_blocks) were never handed out and are taken in
// increasing order, below the stack of returned ones. No C++ exception leaves
// this file: an allocation that fails inside pa_sched_step leaves the
// scheduler unusable (every later step returns PA_ERR_STATE), and one inside
// pa_sched_create frees what was made; both return PA_ERR_NOMEM.

#include "pa_sched.h"

#include <algorithm>
#include <cstdint>
#include <deque>
#include <vector>

namespace {

enum class State : uint8_t { Waiting, Prefilling, Running, Swapped, Finished };

}  // namespace

struct pa_scheduler {
  pa_sched_config cfg{};
  pa_block_manager* bm = nullptr;
  std::vector<int32_t> prompt, output, prefilled, generated;
  std::vector<State> state;
  std::vector<int64_t> batch;                 // admission order
  std::deque<int64_t> swapped;                // oldest preemption first
  std::vector<std::vector<int64_t>> host_of;  // host blocks of a swapped sequence
  std::vector<int64_t> host_free;             // returned host blocks, top = back
  int64_t host_fresh = 0;                     // host blocks [host_fresh, num_host_blocks) never used
  int64_t next_waiting = 0;
  int64_t finished_count = 0;
  int32_t iteration = 0;
  bool broken = false;                        // a step failed half way
  std::vector<int32_t> table_buf;

  // plan buffers
  std::vector<int64_t> d_seqs, d_slots, p_seqs, p_slots, s_out, s_in, fin, adm, pre, res;
  std::vector<int32_t> d_ctx, p_start, p_cu;

  int64_t blocks_for(int64_t tokens) const {
    return (tokens + cfg.block_size - 1) / cfg.block_size;
  }
  int64_t host_free_count() const {
    return (int64_t)host_free.size() + (cfg.num_host_blocks - host_fresh);
  }
  int64_t take_host() {
    if (host_free.empty()) return host_fresh++;
    const int64_t h = host_free.back();
    host_free.pop_back();
    return h;
  }
  // seq's table in table_buf (grown to the table's length); its block count
  int32_t table(int64_t seq) {
    const int32_t nb = pa_bm_table(bm, seq, nullptr, 0);
    if (nb > (int32_t)table_buf.size()) table_buf.resize((size_t)nb);
    return pa_bm_table(bm, seq, table_buf.data(), (int32_t)table_buf.size());
  }
};

namespace {

// A block-manager call the plan relies on. The scheduler's own checks rule
// out every failure but a failed allocation; any failure abandons the step.
void must(pa_status_t st) {
  if (st != PA_OK) throw st;
}

pa_status_t step_impl(pa_scheduler* s, pa_step_plan* plan);

}  // namespace

extern "C" {

pa_status_t pa_sched_create(const pa_sched_config* cfg, const int32_t* prompt_lens,
                            const int32_t* output_lens, int32_t num_requests,
                            pa_scheduler** out) {
  if (!out) return PA_ERR_NULL;
  *out = nullptr;
  if (!cfg) return PA_ERR_NULL;
  if (num_requests < 0 || cfg->num_blocks <= 0 || cfg->num_host_blocks < 0 ||
      cfg->num_host_blocks > INT32_MAX || cfg->block_size <= 0 || cfg->max_blocks_per_seq <= 0 ||
      cfg->max_batch <= 0 || cfg->chunk_tokens <= 0)
    return PA_ERR_SHAPE;
  if (num_requests > 0 && (!prompt_lens || !output_lens)) return PA_ERR_NULL;
  for (int32_t i = 0; i < num_requests; ++i)
    if (prompt_lens[i] < 1 || output_lens[i] < 1) return PA_ERR_SHAPE;
  pa_scheduler* s = nullptr;
  try {
    s = new pa_scheduler();
    s->cfg = *cfg;
    const pa_status_t st =
        pa_bm_create(cfg->num_blocks, cfg->block_size, cfg->max_blocks_per_seq, &s->bm);
    if (st != PA_OK) {
      delete s;
      return st;
    }
    s->prompt.assign(prompt_lens, prompt_lens + num_requests);
    s->output.assign(output_lens, output_lens + num_requests);
    s->prefilled.assign((size_t)num_requests, 0);
    s->generated.assign((size_t)num_requests, 0);
    s->state.assign((size_t)num_requests, State::Waiting);
    s->host_of.resize((size_t)num_requests);
  } catch (...) {
    pa_sched_destroy(s);
    return PA_ERR_NOMEM;
  }
  *out = s;
  return PA_OK;
}

void pa_sched_destroy(pa_scheduler* s) {
  if (!s) return;
  pa_bm_destroy(s->bm);
  delete s;
}

int32_t pa_sched_done(const pa_scheduler* s) {
  return s && s->finished_count == (int64_t)s->state.size() ? 1 : 0;
}

const pa_block_manager* pa_sched_blocks(const pa_scheduler* s) { return s ? s->bm : nullptr; }

pa_status_t pa_sched_step(pa_scheduler* s, pa_step_plan* plan) {
  if (!s || !plan) return PA_ERR_NULL;
  if (s->broken) return PA_ERR_STATE;
  try {
    return step_impl(s, plan);
  } catch (pa_status_t st) {
    s->broken = true;
    return st;
  } catch (...) {
    s->broken = true;
    return PA_ERR_NOMEM;
  }
}

}  // extern "C"

namespace {

pa_status_t step_impl(pa_scheduler* s, pa_step_plan* plan) {
  for (auto* v : {&s->d_seqs, &s->d_slots, &s->p_seqs, &s->p_slots, &s->s_out, &s->s_in,
                  &s->fin, &s->adm, &s->pre, &s->res})
    v->clear();
  s->d_ctx.clear();
  s->p_start.clear();
  s->p_cu.assign(1, 0);
  pa_block_manager* bm = s->bm;
  const int64_t bs = s->cfg.block_size;
  pa_status_t status = PA_OK;

  // 1. eject finished sequences
  for (size_t i = 0; i < s->batch.size();) {
    const int64_t q = s->batch[i];
    if (s->state[q] == State::Running && s->generated[q] == s->output[q]) {
      must(pa_bm_free(bm, q));
      s->state[q] = State::Finished;
      ++s->finished_count;
      s->fin.push_back(q);
      s->batch.erase(s->batch.begin() + (ptrdiff_t)i);
    } else {
      ++i;
    }
  }

  // 2. resume swapped sequences, oldest preemption first
  std::vector<int64_t> slots_tmp;
  while (!s->swapped.empty() && (int64_t)s->batch.size() < s->cfg.max_batch) {
    const int64_t q = s->swapped.front();
    const int64_t length = (int64_t)s->prompt[q] + s->generated[q];
    if (pa_bm_num_free(bm) < s->blocks_for(length) + 1) break;
    s->swapped.pop_front();
    must(pa_bm_add(bm, q));
    slots_tmp.resize((size_t)length);
    must(pa_bm_append(bm, q, (int32_t)length, slots_tmp.data()));
    const int32_t nb = s->table(q);
    auto& hosts = s->host_of[q];
    for (int32_t j = 0; j < nb; ++j) {
      s->s_in.push_back(hosts[(size_t)j]);
      s->s_in.push_back(s->table_buf[(size_t)j]);
    }
    for (auto h = hosts.rbegin(); h != hosts.rend(); ++h) s->host_free.push_back(*h);
    hosts.clear();
    s->state[q] = State::Running;
    s->batch.push_back(q);
    s->res.push_back(q);
  }

  // 3. admit waiting requests (not while anything is swapped out)
  while (s->swapped.empty() && s->next_waiting < (int64_t)s->state.size() &&
         (int64_t)s->batch.size() < s->cfg.max_batch) {
    const int64_t q = s->next_waiting;
    if (pa_bm_num_free(bm) < s->blocks_for((int64_t)s->prompt[q] + 1)) break;
    must(pa_bm_add(bm, q));
    slots_tmp.resize((size_t)s->prompt[q]);
    must(pa_bm_append(bm, q, s->prompt[q], slots_tmp.data()));
    s->state[q] = State::Prefilling;
    s->batch.push_back(q);
    ++s->next_waiting;
    s->adm.push_back(q);
  }

  // 4. prefill chunks within the row budget, admission order
  int64_t budget = s->cfg.chunk_tokens;
  std::vector<int64_t> became_running;
  for (const int64_t q : s->batch) {
    if (budget == 0) break;
    if (s->state[q] != State::Prefilling) continue;
    const int64_t start = s->prefilled[q];
    const int64_t take = std::min<int64_t>(budget, (int64_t)s->prompt[q] - start);
    s->table(q);
    s->p_seqs.push_back(q);
    s->p_start.push_back((int32_t)start);
    for (int64_t p = start; p < start + take; ++p)
      s->p_slots.push_back((int64_t)s->table_buf[(size_t)(p / bs)] * bs + p % bs);
    s->p_cu.push_back(s->p_cu.back() + (int32_t)take);
    s->prefilled[q] += (int32_t)take;
    budget -= take;
    if (s->prefilled[q] == s->prompt[q]) became_running.push_back(q);
  }

  // 5. decode one token per running sequence; preempt the latest admitted
  //    while the pool cannot hold them all
  std::vector<int64_t> runners;
  for (const int64_t q : s->batch)
    if (s->state[q] == State::Running) runners.push_back(q);
  auto need = [&]() {
    int64_t n = 0;
    for (const int64_t q : runners) n += pa_bm_blocks_needed(bm, q, 1);
    return n;
  };
  while (!runners.empty() && need() > pa_bm_num_free(bm)) {
    const int64_t v = runners.back();
    runners.pop_back();
    const int32_t nb = s->table(v);
    if (s->host_free_count() < nb) {
      status = PA_ERR_OUT_OF_BLOCKS;
      break;
    }
    auto& hosts = s->host_of[v];
    for (int32_t j = 0; j < nb; ++j) {
      const int64_t h = s->take_host();
      hosts.push_back(h);
      s->s_out.push_back(s->table_buf[(size_t)j]);
      s->s_out.push_back(h);
    }
    must(pa_bm_free(bm, v));
    s->state[v] = State::Swapped;
    s->batch.erase(std::find(s->batch.begin(), s->batch.end(), v));
    s->swapped.push_back(v);
    s->pre.push_back(v);
  }
  if (status == PA_OK) {
    for (const int64_t q : runners) {
      int64_t slot = 0;
      must(pa_bm_append(bm, q, 1, &slot));
      ++s->generated[q];
      s->d_seqs.push_back(q);
      s->d_slots.push_back(slot);
      s->d_ctx.push_back(s->prompt[q] + s->generated[q]);
    }
  }
  for (const int64_t q : became_running) s->state[q] = State::Running;

  plan->iteration = s->iteration++;
  plan->num_decode = (int32_t)s->d_seqs.size();
  plan->decode_seqs = s->d_seqs.data();
  plan->decode_slots = s->d_slots.data();
  plan->decode_context = s->d_ctx.data();
  plan->num_prefill = (int32_t)s->p_seqs.size();
  plan->prefill_seqs = s->p_seqs.data();
  plan->prefill_start = s->p_start.data();
  plan->prefill_cu = s->p_cu.data();
  plan->prefill_slots = s->p_slots.data();
  plan->num_swap_out = (int32_t)(s->s_out.size() / 2);
  plan->swap_out = s->s_out.data();
  plan->num_swap_in = (int32_t)(s->s_in.size() / 2);
  plan->swap_in = s->s_in.data();
  plan->num_finished = (int32_t)s->fin.size();
  plan->finished = s->fin.data();
  plan->num_admitted = (int32_t)s->adm.size();
  plan->admitted = s->adm.data();
  plan->num_preempted = (int32_t)s->pre.size();
  plan->preempted = s->pre.data();
  plan->num_resumed = (int32_t)s->res.size();
  plan->resumed = s->res.data();
  return status;
}

}  // namespace
