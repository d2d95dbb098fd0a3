/*
 * pa_engine.h - continuous-batching step driver in C++ (libpa.so): runs the
 * scheduler's plans (pa_sched.h) on the GPU through the library's own entry
 * points, with decode-only iterations replayed from a captured HIP graph.
 *
 * An iteration is planned on the host, then executed: swapped blocks come
 * back from the pinned host pool and preempted ones go out (pa_swap_in,
 * pa_swap_out), then for every layer the iteration's new K/V rows are written
 * through the slot mapping (pa_reshape_and_cache), the prefill chunks attend
 * to their prefix (pa_prefill_chunk) and the decode batch attends to its
 * context (pa_decode) (How vLLM gets real throughput on H100s, "Continuous
 * batching removes straggler bubbles"; Dissecting vLLM, "Continuous
 * Batching: Breaking the Sequence Barrier"; vLLM architecture, memory and
 * benchmarks deep dive, "Hardware-level optimizations"). Launch overhead is
 * what the graph removes: a decode-only iteration is two copies of slots,
 * tables and lengths from pinned staging and one graph launch that runs
 * every layer's scatter and decode for max_batch rows (rows past the batch
 * have context 0 and slot -1).
 *
 * The model is outside: between pa_engine_plan and pa_engine_execute the
 * caller writes the iteration's inputs into the buffers it registered - for
 * layer l, decode row i (the plan's i-th decode sequence) of q_dec[l],
 * k_dec[l], v_dec[l], and prefill row r (rows of the plan's chunks, in order)
 * of q_pre[l], k_pre[l], v_pre[l]. Outputs land in out_dec[l] (decode rows)
 * and out_pre[l] (prefill rows) when the stream reaches them.
 *
 * Ownership: the caller owns every registered buffer and keeps it alive;
 * the engine allocates its own index buffers, staging (pinned) and
 * workspaces at creation and frees them in pa_engine_destroy. All work is
 * enqueued on the stream given at creation.
 *
 * Caches: BF16, or FP8 (E4M3 codes, kv_fp8 = 1) with one float32 K and one V
 * scale per KV head and layer. The model's inputs (queries, new K/V rows) are
 * BF16 either way; an FP8 engine quantizes the new rows as it writes them
 * (pa_reshape_and_cache_fp8) and attends with pa_prefill_chunk_fp8 and
 * pa_decode_fp8; the host pools then hold codes too.
 */
#ifndef PA_ENGINE_H
#define PA_ENGINE_H

#include "pa_sched.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_engine pa_engine;

typedef struct {
  int32_t num_layers;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  float scale;
  int32_t use_graph;              /* replay decode-only iterations from graphs */
  pa_sched_config sched;          /* pools, block size, batch, chunk budget */
  int32_t kv_fp8;                 /* 1: E4M3 caches with per-head scales; 0: BF16 */
} pa_engine_config;

/* Arrays of num_layers pointers each (copied at creation). */
typedef struct {
  void* const* key_caches;        /* device [num_blocks, Hkv, bs, d], BF16 or E4M3 */
  void* const* value_caches;
  void* const* host_keys;         /* pinned [num_host_blocks, Hkv, bs, d], as the caches */
  void* const* host_values;
  void* const* q_dec;             /* device BF16 [max_batch, Hq, d] */
  void* const* k_dec;             /* device BF16 [max_batch, Hkv, d] */
  void* const* v_dec;
  void* const* q_pre;             /* device BF16 [chunk_tokens, Hq, d] */
  void* const* k_pre;             /* device BF16 [chunk_tokens, Hkv, d] */
  void* const* v_pre;
  float* const* out_dec;          /* device float32 [max_batch, Hq, d] */
  float* const* out_pre;          /* device float32 [chunk_tokens, Hq, d] */
  const float* const* k_scales;   /* kv_fp8: device float32 [Hkv] per layer (else NULL) */
  const float* const* v_scales;
} pa_engine_buffers;

/* Creates the engine: its scheduler, index buffers, pinned staging and
 * workspaces, and (use_graph) the captured decode-only graph. Returns
 * PA_ERR_NULL for a NULL cfg, bufs, out or pointer array (the scale arrays
 * only with kv_fp8); PA_ERR_SHAPE for
 * non-positive head counts or sizes, and the scheduler's own errors
 * (pa_sched_create); PA_ERR_UNSUPPORTED when pa_decode has no kernel for the
 * head shape or block size; PA_ERR_HIP when an allocation or the capture
 * fails. The pointers in the arrays are not dereferenced here. *out is NULL
 * on error and nothing stays allocated. */
pa_status_t pa_engine_create(const pa_engine_config* cfg, const pa_engine_buffers* bufs,
                             const int32_t* prompt_lens, const int32_t* output_lens,
                             int32_t num_requests, void* stream, pa_engine** out);
void pa_engine_destroy(pa_engine* e);

int32_t pa_engine_done(const pa_engine* e);

/* Plan the next iteration (the scheduler's step). The plan's arrays stay
 * valid until the next pa_engine_plan. PA_ERR_NULL for NULL arguments, else
 * the status of pa_sched_step (PA_ERR_OUT_OF_BLOCKS: the host pool cannot
 * take a preemption; the engine should then be destroyed). */
pa_status_t pa_engine_plan(pa_engine* e, pa_step_plan* plan);

/* Enqueue the device work of the last plan. Returns after enqueueing; it
 * waits only for the staging set it reuses (written two iterations ago).
 * PA_ERR_NULL for NULL; PA_ERR_STATE when no plan is pending (each plan is
 * executed once); PA_ERR_SHAPE when the plan exceeds the registered buffers
 * (cannot happen with the engine's own scheduler); otherwise the first error
 * of the entry points it calls (PA_ERR_HIP for a failed launch or copy), in
 * which case part of the iteration may have been enqueued. */
pa_status_t pa_engine_execute(pa_engine* e);

/* Iterations executed so far and how many of them were graph launches. */
int64_t pa_engine_iterations(const pa_engine* e);
int64_t pa_engine_graph_launches(const pa_engine* e);

#ifdef __cplusplus
}
#endif

#endif /* PA_ENGINE_H */
