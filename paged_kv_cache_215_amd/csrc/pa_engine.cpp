// Continuous-batching step driver (declared in include/pa_engine.h): plans an
// iteration with the native scheduler and enqueues its device work through
// the library's own entry points; decode-only iterations are one launch of a
// captured HIP graph. No C++ exception leaves an entry point: a failed host
// allocation is PA_ERR_NOMEM.

#include "pa_engine.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <vector>

namespace {

// One set of pinned staging buffers.
struct Stage {
  int64_t* slots = nullptr;   // [B | C]: decode slots, then prefill slots
  int32_t* meta = nullptr;    // decode tables, decode lens, prefill tables, ctx, cu
  int64_t* pairs = nullptr;   // swap-in pairs, then swap-out pairs
  hipEvent_t done = nullptr;  // recorded after the last work that read this set
  bool used = false;
};

}  // namespace

struct pa_engine {
  pa_engine_config cfg{};
  std::vector<void*> kc, vc, hk, hv, qd, kd, vd, qp, kp, vp;
  std::vector<float*> od, op;
  std::vector<const float*> ks, vs;   // E4M3 caches: per-layer K / V scales
  pa_scheduler* sched = nullptr;
  hipStream_t stream = nullptr;
  int32_t B = 0, MB = 0, C = 0, capacity = 0;
  size_t meta_len = 0, pair_len = 0;
  Stage stage[2];
  int next = 0;
  hipGraphExec_t graph = nullptr;
  int64_t* d_slots = nullptr;
  int32_t* d_meta = nullptr;
  void* dec_ws = nullptr;
  size_t dec_ws_bytes = 0;
  void* pf_ws = nullptr;
  size_t pf_ws_bytes = 0;
  pa_step_plan plan{};
  bool planned = false;
  int64_t iterations = 0, graph_launches = 0;

  // offsets into meta (int32 elements)
  size_t o_dec_tab() const { return 0; }
  size_t o_dec_len() const { return (size_t)B * MB; }
  size_t o_pre_tab() const { return (size_t)B * MB + B; }
  size_t o_pre_ctx() const { return 2 * (size_t)B * MB + B; }
  size_t o_pre_cu() const { return 2 * (size_t)B * MB + 2 * (size_t)B; }
};

namespace {

pa_status_t hip_ok(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

#define PA_TRY(x)                        \
  do {                                   \
    const pa_status_t st_ = (x);         \
    if (st_ != PA_OK) return st_;        \
  } while (0)

// The library calls of one layer, for the engine's cache type (BF16, or E4M3
// codes with the layer's scales; inputs are BF16 either way).
pa_status_t write_rows(pa_engine* e, int l, const void* k, const void* v, const int64_t* slots,
                       int32_t rows) {
  const auto& c = e->cfg;
  const auto& s = c.sched;
  if (c.kv_fp8)
    return pa_reshape_and_cache_fp8(k, v, e->kc[l], e->vc[l], slots, e->ks[l], e->vs[l], rows,
                                    c.num_kv_heads, c.head_dim, s.block_size, s.num_blocks,
                                    PA_DTYPE_BF16, e->stream);
  return pa_reshape_and_cache(k, v, e->kc[l], e->vc[l], slots, rows, c.num_kv_heads, c.head_dim,
                              s.block_size, s.num_blocks, PA_DTYPE_BF16, e->stream);
}

pa_status_t decode_layer(pa_engine* e, int l, int32_t rows, int32_t max_ctx) {
  const auto& c = e->cfg;
  const auto& s = c.sched;
  const int32_t* tab = e->d_meta + e->o_dec_tab();
  const int32_t* len = e->d_meta + e->o_dec_len();
  if (c.kv_fp8)
    return pa_decode_fp8(e->od[l], e->qd[l], e->kc[l], e->vc[l], e->ks[l], e->vs[l], tab, len,
                         rows, c.num_q_heads, c.num_kv_heads, c.head_dim, s.block_size, e->MB,
                         s.num_blocks, max_ctx, c.scale, PA_DTYPE_BF16, e->dec_ws,
                         e->dec_ws_bytes, e->stream);
  return pa_decode(e->od[l], e->qd[l], e->kc[l], e->vc[l], tab, len, rows, c.num_q_heads,
                   c.num_kv_heads, c.head_dim, s.block_size, e->MB, s.num_blocks, max_ctx,
                   c.scale, PA_DTYPE_BF16, e->dec_ws, e->dec_ws_bytes, e->stream);
}

pa_status_t prefill_layer(pa_engine* e, int l, int32_t n_pre, int32_t rows, int32_t max_q,
                          int32_t max_ctx) {
  const auto& c = e->cfg;
  const auto& s = c.sched;
  const int32_t* tab = e->d_meta + e->o_pre_tab();
  const int32_t* ctx = e->d_meta + e->o_pre_ctx();
  const int32_t* cu = e->d_meta + e->o_pre_cu();
  if (c.kv_fp8)
    return pa_prefill_chunk_fp8(e->op[l], e->qp[l], e->kc[l], e->vc[l], e->ks[l], e->vs[l], tab,
                                ctx, cu, n_pre, rows, max_q, c.num_q_heads, c.num_kv_heads,
                                c.head_dim, s.block_size, e->MB, s.num_blocks, max_ctx, c.scale,
                                PA_DTYPE_BF16, e->pf_ws, e->pf_ws_bytes, e->stream);
  return pa_prefill_chunk(e->op[l], e->qp[l], e->kc[l], e->vc[l], tab, ctx, cu, n_pre, rows,
                          max_q, c.num_q_heads, c.num_kv_heads, c.head_dim, s.block_size, e->MB,
                          s.num_blocks, max_ctx, c.scale, PA_DTYPE_BF16, e->pf_ws,
                          e->pf_ws_bytes, e->stream);
}

pa_dtype_t cache_dtype(const pa_engine* e) {
  return e->cfg.kv_fp8 ? PA_DTYPE_FP8_E4M3 : PA_DTYPE_BF16;
}

// Decode scatter + attention of every layer for B rows, reading slots and
// tables from the device index buffers: the body of the decode-only graph.
pa_status_t decode_body(pa_engine* e, int32_t rows, int32_t max_ctx) {
  for (int l = 0; l < e->cfg.num_layers; ++l) {
    PA_TRY(write_rows(e, l, e->kd[l], e->vd[l], e->d_slots, rows));
    PA_TRY(decode_layer(e, l, rows, max_ctx));
  }
  return PA_OK;
}

// The decode-only graph: the decode body for B rows at full capacity, reading
// the device index buffers. The copies from pinned staging into those buffers
// are issued before each launch, outside the graph: as memcpy nodes inside it
// they made every replay slower than the eager launches it replaces.
pa_status_t capture(pa_engine* e) {
  hipGraph_t g = nullptr;
  if (hipStreamBeginCapture(e->stream, hipStreamCaptureModeThreadLocal) != hipSuccess)
    return PA_ERR_HIP;
  pa_status_t status = decode_body(e, e->B, e->capacity);
  const hipError_t end = hipStreamEndCapture(e->stream, &g);
  if (status != PA_OK || end != hipSuccess) {
    if (g) (void)hipGraphDestroy(g);
    return status != PA_OK ? status : PA_ERR_HIP;
  }
  status = hip_ok(hipGraphInstantiate(&e->graph, g, nullptr, nullptr, 0));
  (void)hipGraphDestroy(g);
  return status;
}

void release(pa_engine* e) {
  if (e->graph) (void)hipGraphExecDestroy(e->graph);
  for (Stage& st : e->stage) {
    if (st.done) (void)hipEventDestroy(st.done);
    if (st.slots) (void)hipHostFree(st.slots);
    if (st.meta) (void)hipHostFree(st.meta);
    if (st.pairs) (void)hipHostFree(st.pairs);
  }
  if (e->d_slots) (void)hipFree(e->d_slots);
  if (e->d_meta) (void)hipFree(e->d_meta);
  if (e->dec_ws) (void)hipFree(e->dec_ws);
  if (e->pf_ws) (void)hipFree(e->pf_ws);
  if (e->sched) pa_sched_destroy(e->sched);
}

// Fills a new engine e; on failure the caller releases and deletes it.
pa_status_t create_impl(const pa_engine_config* cfg, const pa_engine_buffers* b,
                        const int32_t* prompt_lens, const int32_t* output_lens,
                        int32_t num_requests, void* stream, pa_engine* e) {
  const int L = cfg->num_layers;
  if (L <= 0 || cfg->num_q_heads <= 0 || cfg->num_kv_heads <= 0 || cfg->head_dim <= 0)
    return PA_ERR_SHAPE;
  for (void* const* a : {b->key_caches, b->value_caches, b->host_keys, b->host_values, b->q_dec,
                         b->k_dec, b->v_dec, b->q_pre, b->k_pre, b->v_pre})
    if (!a) return PA_ERR_NULL;
  if (!b->out_dec || !b->out_pre) return PA_ERR_NULL;
  if (cfg->kv_fp8 && (!b->k_scales || !b->v_scales)) return PA_ERR_NULL;
  e->cfg = *cfg;
  e->stream = static_cast<hipStream_t>(stream);
  auto take = [L](void* const* a, std::vector<void*>& v) { v.assign(a, a + L); };
  take(b->key_caches, e->kc);
  take(b->value_caches, e->vc);
  take(b->host_keys, e->hk);
  take(b->host_values, e->hv);
  take(b->q_dec, e->qd);
  take(b->k_dec, e->kd);
  take(b->v_dec, e->vd);
  take(b->q_pre, e->qp);
  take(b->k_pre, e->kp);
  take(b->v_pre, e->vp);
  e->od.assign(b->out_dec, b->out_dec + L);
  e->op.assign(b->out_pre, b->out_pre + L);
  if (cfg->kv_fp8) {
    e->ks.assign(b->k_scales, b->k_scales + L);
    e->vs.assign(b->v_scales, b->v_scales + L);
  }
  const pa_sched_config& s = cfg->sched;
  pa_status_t status = pa_sched_create(&s, prompt_lens, output_lens, num_requests, &e->sched);
  if (status != PA_OK) return status;
  e->B = s.max_batch;
  e->MB = s.max_blocks_per_seq;
  e->C = s.chunk_tokens;
  e->capacity = (int32_t)std::min<int64_t>((int64_t)s.max_blocks_per_seq * s.block_size, INT32_MAX);
  e->meta_len = e->o_pre_cu() + e->B + 1;
  e->pair_len = 4 * (size_t)s.num_blocks;  // swap-in and swap-out pairs
  e->dec_ws_bytes = pa_decode_workspace_size(e->B, cfg->num_q_heads, cfg->num_kv_heads,
                                             cfg->head_dim, s.block_size, e->capacity);
  e->pf_ws_bytes = pa_prefill_chunk_workspace_size(1, e->C, e->C, cfg->num_q_heads,
                                                   cfg->num_kv_heads, cfg->head_dim,
                                                   s.block_size, e->capacity);
  if (e->dec_ws_bytes == 0) status = PA_ERR_UNSUPPORTED;
  for (Stage& st : e->stage) {
    if (status != PA_OK) break;
    status = hip_ok(hipHostMalloc((void**)&st.slots, ((size_t)e->B + e->C) * sizeof(int64_t)));
    if (status == PA_OK) status = hip_ok(hipHostMalloc((void**)&st.meta, e->meta_len * sizeof(int32_t)));
    if (status == PA_OK) status = hip_ok(hipHostMalloc((void**)&st.pairs, e->pair_len * sizeof(int64_t)));
    if (status == PA_OK) status = hip_ok(hipEventCreateWithFlags(&st.done, hipEventDisableTiming));
  }
  if (status == PA_OK)
    status = hip_ok(hipMalloc((void**)&e->d_slots, ((size_t)e->B + e->C) * sizeof(int64_t)));
  if (status == PA_OK) status = hip_ok(hipMalloc((void**)&e->d_meta, e->meta_len * sizeof(int32_t)));
  if (status == PA_OK) status = hip_ok(hipMalloc(&e->dec_ws, e->dec_ws_bytes));
  if (status == PA_OK && e->pf_ws_bytes) status = hip_ok(hipMalloc(&e->pf_ws, e->pf_ws_bytes));
  if (status == PA_OK) status = pa_decode_workspace_init(e->dec_ws, e->dec_ws_bytes, stream);
  if (status == PA_OK && cfg->use_graph) {
    // the graphs start from staging that writes nothing (slots -1, lengths
    // 0); the body runs once outside capture first, so that the library's
    // one-time set-up (occupancy and device queries) never runs captured
    for (int k = 0; k < 2; ++k) {
      std::fill(e->stage[k].slots, e->stage[k].slots + e->B + e->C, (int64_t)-1);
      std::fill(e->stage[k].meta, e->stage[k].meta + e->meta_len, 0);
    }
    status = hip_ok(hipMemcpyAsync(e->d_slots, e->stage[0].slots, e->B * sizeof(int64_t),
                                   hipMemcpyHostToDevice, e->stream));
    if (status == PA_OK)
      status = hip_ok(hipMemcpyAsync(e->d_meta, e->stage[0].meta, e->meta_len * sizeof(int32_t),
                                     hipMemcpyHostToDevice, e->stream));
    if (status == PA_OK) status = decode_body(e, e->B, e->capacity);
    if (status == PA_OK) status = hip_ok(hipStreamSynchronize(e->stream));
    if (status == PA_OK) status = capture(e);
  }
  if (status == PA_OK) status = hip_ok(hipStreamSynchronize(e->stream));
  return status;
}


// The device work of the pending plan.
pa_status_t execute_impl(pa_engine* e) {
  const pa_step_plan& p = e->plan;
  const auto& c = e->cfg;
  const auto& s = c.sched;
  const int n_dec = p.num_decode, n_pre = p.num_prefill;
  const int rows = p.prefill_cu[n_pre];
  if (n_dec > e->B || rows > e->C || n_pre > e->B) return PA_ERR_SHAPE;

  // this iteration's staging set, free once its last reader has run
  Stage& st = e->stage[e->next];
  e->next ^= 1;
  if (st.used) PA_TRY(hip_ok(hipEventSynchronize(st.done)));
  const pa_block_manager* bm = pa_sched_blocks(e->sched);

  // decode rows: slots, tables, lengths (padded to B rows in graph mode)
  const bool graph = c.use_graph && rows == 0 && n_dec > 0;
  const int pad = graph ? e->B : n_dec;
  std::copy(p.decode_slots, p.decode_slots + n_dec, st.slots);
  std::fill(st.slots + n_dec, st.slots + pad, (int64_t)-1);
  if (n_dec)
    PA_TRY(pa_bm_tables(bm, p.decode_seqs, n_dec, st.meta + e->o_dec_tab(), e->MB,
                        st.meta + e->o_dec_len()));
  std::fill(st.meta + e->o_dec_tab() + (size_t)n_dec * e->MB,
            st.meta + e->o_dec_tab() + (size_t)pad * e->MB, -1);
  std::fill(st.meta + e->o_dec_len() + n_dec, st.meta + e->o_dec_len() + pad, 0);
  int32_t max_dec_ctx = 0;
  for (int i = 0; i < n_dec; ++i) max_dec_ctx = std::max(max_dec_ctx, st.meta[e->o_dec_len() + i]);

  // swaps: in, then out (pairs read from pinned staging by the kernels)
  if (p.num_swap_in > (int64_t)s.num_blocks || p.num_swap_out > (int64_t)s.num_blocks)
    return PA_ERR_SHAPE;
  int64_t* in_pairs = st.pairs;
  int64_t* out_pairs = st.pairs + 2 * (size_t)s.num_blocks;
  std::copy(p.swap_in, p.swap_in + 2 * (size_t)p.num_swap_in, in_pairs);
  std::copy(p.swap_out, p.swap_out + 2 * (size_t)p.num_swap_out, out_pairs);
  for (int l = 0; l < c.num_layers && p.num_swap_in; ++l)
    PA_TRY(pa_swap_in(e->kc[l], e->vc[l], e->hk[l], e->hv[l], in_pairs, p.num_swap_in,
                      c.num_kv_heads, c.head_dim, s.block_size, s.num_blocks, s.num_host_blocks,
                      cache_dtype(e), e->stream));
  for (int l = 0; l < c.num_layers && p.num_swap_out; ++l)
    PA_TRY(pa_swap_out(e->kc[l], e->vc[l], e->hk[l], e->hv[l], out_pairs, p.num_swap_out,
                       c.num_kv_heads, c.head_dim, s.block_size, s.num_blocks, s.num_host_blocks,
                       cache_dtype(e), e->stream));

  if (graph) {
    PA_TRY(hip_ok(hipMemcpyAsync(e->d_slots, st.slots, e->B * sizeof(int64_t),
                                 hipMemcpyHostToDevice, e->stream)));
    PA_TRY(hip_ok(hipMemcpyAsync(e->d_meta, st.meta, (e->o_dec_len() + e->B) * sizeof(int32_t),
                                 hipMemcpyHostToDevice, e->stream)));
    PA_TRY(hip_ok(hipGraphLaunch(e->graph, e->stream)));
    PA_TRY(hip_ok(hipEventRecord(st.done, e->stream)));
    st.used = true;
    ++e->iterations;
    ++e->graph_launches;
    return PA_OK;
  }

  // prefill chunks: slots after the decode region, tables, contexts, offsets
  int32_t max_q = 0, max_pre_ctx = 0;
  if (n_pre) {
    std::copy(p.prefill_slots, p.prefill_slots + rows, st.slots + e->B);
    PA_TRY(pa_bm_tables(bm, p.prefill_seqs, n_pre, st.meta + e->o_pre_tab(), e->MB,
                        st.meta + e->o_pre_ctx()));  // lengths overwritten below
    for (int i = 0; i < n_pre; ++i) {
      const int32_t q = p.prefill_cu[i + 1] - p.prefill_cu[i];
      st.meta[e->o_pre_ctx() + i] = p.prefill_start[i] + q;
      st.meta[e->o_pre_cu() + i] = p.prefill_cu[i];
      max_q = std::max(max_q, q);
      max_pre_ctx = std::max(max_pre_ctx, p.prefill_start[i] + q);
    }
    st.meta[e->o_pre_cu() + n_pre] = rows;
  }
  PA_TRY(hip_ok(hipMemcpyAsync(e->d_slots, st.slots, ((size_t)e->B + e->C) * sizeof(int64_t),
                               hipMemcpyHostToDevice, e->stream)));
  PA_TRY(hip_ok(hipMemcpyAsync(e->d_meta, st.meta, e->meta_len * sizeof(int32_t),
                               hipMemcpyHostToDevice, e->stream)));

  // prefill workspace for this plan (grown when a plan needs more)
  if (n_pre) {
    const size_t need = pa_prefill_chunk_workspace_size(n_pre, rows, max_q, c.num_q_heads,
                                                        c.num_kv_heads, c.head_dim,
                                                        s.block_size, max_pre_ctx);
    if (need > e->pf_ws_bytes) {
      PA_TRY(hip_ok(hipStreamSynchronize(e->stream)));
      if (e->pf_ws) (void)hipFree(e->pf_ws);
      e->pf_ws = nullptr;
      e->pf_ws_bytes = 0;
      PA_TRY(hip_ok(hipMalloc(&e->pf_ws, need)));
      e->pf_ws_bytes = need;
    }
  }

  for (int l = 0; l < c.num_layers; ++l) {
    if (n_dec) PA_TRY(write_rows(e, l, e->kd[l], e->vd[l], e->d_slots, n_dec));
    if (rows) PA_TRY(write_rows(e, l, e->kp[l], e->vp[l], e->d_slots + e->B, rows));
    if (n_pre) PA_TRY(prefill_layer(e, l, n_pre, rows, max_q, max_pre_ctx));
    if (n_dec) PA_TRY(decode_layer(e, l, n_dec, max_dec_ctx));
  }
  PA_TRY(hip_ok(hipEventRecord(st.done, e->stream)));
  st.used = true;
  ++e->iterations;
  return PA_OK;
}


}  // namespace

extern "C" {

pa_status_t pa_engine_create(const pa_engine_config* cfg, const pa_engine_buffers* b,
                             const int32_t* prompt_lens, const int32_t* output_lens,
                             int32_t num_requests, void* stream, pa_engine** out) {
  if (!out) return PA_ERR_NULL;
  *out = nullptr;
  if (!cfg || !b) return PA_ERR_NULL;
  pa_engine* e = nullptr;
  pa_status_t status = PA_OK;
  try {
    e = new pa_engine();
    status = create_impl(cfg, b, prompt_lens, output_lens, num_requests, stream, e);
  } catch (...) {
    status = PA_ERR_NOMEM;
  }
  if (status != PA_OK) {
    if (e) {
      release(e);
      delete e;
    }
    return status;
  }
  *out = e;
  return PA_OK;
}

void pa_engine_destroy(pa_engine* e) {
  if (!e) return;
  (void)hipStreamSynchronize(e->stream);
  release(e);
  delete e;
}

int32_t pa_engine_done(const pa_engine* e) { return e ? pa_sched_done(e->sched) : 0; }
int64_t pa_engine_iterations(const pa_engine* e) { return e ? e->iterations : -1; }
int64_t pa_engine_graph_launches(const pa_engine* e) { return e ? e->graph_launches : -1; }

pa_status_t pa_engine_plan(pa_engine* e, pa_step_plan* plan) {
  if (!e || !plan) return PA_ERR_NULL;
  PA_TRY(pa_sched_step(e->sched, &e->plan));
  e->planned = true;
  *plan = e->plan;
  return PA_OK;
}

pa_status_t pa_engine_execute(pa_engine* e) {
  if (!e) return PA_ERR_NULL;
  if (!e->planned) return PA_ERR_STATE;
  e->planned = false;
  try {
    return execute_impl(e);
  } catch (...) {
    return PA_ERR_NOMEM;
  }
}

}  // extern "C"
