/*
 * pa_sched.h - iteration-level (continuous) batching scheduler over the
 * paged KV cache (host C++ in libpa.so).
 *
 * The scheduler decides at every forward pass (one token per running
 * sequence): a sequence that has produced its last token gives its blocks
 * back at once and a waiting request takes the freed slot in the same
 * iteration (How vLLM gets real throughput on H100s, "Continuous batching
 * removes straggler bubbles"; vLLM architecture, memory and benchmarks deep
 * dive, "Continuous batching and the straggler problem"). When memory runs
 * short a running sequence is preempted: its blocks are swapped to host
 * memory and freed, and it resumes later with its context intact (Dissecting
 * vLLM, "Continuous Batching: Breaking the Sequence Barrier"). Long prompts
 * are processed in chunks interleaved with decode tokens (vLLM
 * architecture... deep dive, "Hardware-level optimizations").
 *
 * Requests are an offline batch served first come, first served; request i
 * has prompt_lens[i] prompt tokens and is finished after output_lens[i]
 * generated tokens. Iteration t does, in order:
 *   1. eject running sequences that have generated all their tokens;
 *   2. resume swapped sequences (oldest preemption first) while the batch has
 *      room and the pool holds their length plus one block: fresh blocks for
 *      the whole length, host blocks copied back (swap_in) and released;
 *   3. admit waiting requests (only while nothing is swapped out) while the
 *      batch has room and the pool holds prompt_len + 1 tokens; the whole
 *      prompt's blocks are reserved;
 *   4. prefill up to chunk_tokens prompt rows, from the prefilling sequences
 *      in admission order, a run of consecutive rows each; a sequence whose
 *      prompt completes decodes from the next iteration;
 *   5. decode: every running sequence appends one token; while the pool is
 *      short, the running sequence admitted last is preempted (swap_out of
 *      its blocks to host blocks, in table order, then freed).
 * The device work of a plan runs in this order: swap_in copies, swap_out
 * copies, then the iteration's token writes (prefill rows, decode tokens) and
 * the attention. Device and host pools use the block manager's stack policy
 * (pa_blocks.h).
 */
#ifndef PA_SCHED_H
#define PA_SCHED_H

#include "pa_blocks.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_scheduler pa_scheduler;

typedef struct {
  int64_t num_blocks;         /* device pool */
  int64_t num_host_blocks;    /* host swap pool */
  int32_t block_size;
  int32_t max_blocks_per_seq;
  int32_t max_batch;          /* sequences prefilling or running at once */
  int32_t chunk_tokens;       /* prompt rows prefilled per iteration */
} pa_sched_config;

/*
 * One iteration's plan. Every pointer stays valid until the next
 * pa_sched_step or pa_sched_destroy. Sequence ids are request indices.
 */
typedef struct {
  int32_t iteration;
  int32_t num_decode;              /* decode batch, admission order */
  const int64_t* decode_seqs;      /* [num_decode] */
  const int64_t* decode_slots;     /* [num_decode] slot of the new token */
  const int32_t* decode_context;   /* [num_decode] context incl. the new token */
  int32_t num_prefill;             /* prefill chunks */
  const int64_t* prefill_seqs;     /* [num_prefill] */
  const int32_t* prefill_start;    /* [num_prefill] first prompt row of the chunk */
  const int32_t* prefill_cu;       /* [num_prefill + 1] chunk offsets in rows */
  const int64_t* prefill_slots;    /* [prefill_cu[num_prefill]] slots of the rows */
  int32_t num_swap_out;
  const int64_t* swap_out;         /* [num_swap_out][2] (device block, host block) */
  int32_t num_swap_in;
  const int64_t* swap_in;          /* [num_swap_in][2] (host block, device block) */
  int32_t num_finished;
  const int64_t* finished;
  int32_t num_admitted;
  const int64_t* admitted;
  int32_t num_preempted;
  const int64_t* preempted;
  int32_t num_resumed;
  const int64_t* resumed;
} pa_step_plan;

/* PA_ERR_SHAPE for non-positive sizes, num_host_blocks above 2^31 - 1, or a
 * request with prompt_len < 1 or output_len < 1; PA_ERR_NOMEM if host memory
 * runs out (nothing is leaked); *out is NULL on error. Host swap blocks are
 * handed out lazily, so creation costs no memory per host block. */
pa_status_t pa_sched_create(const pa_sched_config* cfg, const int32_t* prompt_lens,
                            const int32_t* output_lens, int32_t num_requests,
                            pa_scheduler** out);
void pa_sched_destroy(pa_scheduler* s);

/* 1 once every request is finished. */
int32_t pa_sched_done(const pa_scheduler* s);

/* Plan the next iteration. PA_ERR_OUT_OF_BLOCKS if a preemption needs more
 * host blocks than are free (the plan is then incomplete and the scheduler
 * should be discarded). PA_ERR_NOMEM if host memory runs out half way: the
 * scheduler is then unusable and every later step returns PA_ERR_STATE
 * (destroy it). No C++ exception leaves any pa_sched_* call. */
pa_status_t pa_sched_step(pa_scheduler* s, pa_step_plan* plan);

/* The device pool's manager, for block tables (pa_bm_tables) and queries. */
const pa_block_manager* pa_sched_blocks(const pa_scheduler* s);

#ifdef __cplusplus
}
#endif

#endif /* PA_SCHED_H */
