"""Continuous-batching step driver: runs the native scheduler's plans on the
GPU through the C ABI.

Each iteration (How vLLM gets real throughput on H100s, "Continuous batching
removes straggler bubbles"; Dissecting vLLM, "Continuous Batching: Breaking
the Sequence Barrier"; vLLM architecture, memory and benchmarks deep dive,
"Hardware-level optimizations"):

1. the scheduler (C++, ``Scheduler``) plans the iteration on the host;
2. swapped-out blocks come back from the pinned host pool (``pa_swap_in``),
   then a preempted sequence's blocks go out to it (``pa_swap_out``);
3. for every layer: the iteration's new K/V rows - prompt rows of the
   prefill chunks and one token per decoding sequence - are written through
   the slot mapping (``pa_reshape_and_cache``), the chunks attend to their
   prefix (``pa_prefill_chunk``) and the decode batch attends to its context
   (``pa_decode``).

The model itself (projections, sampling) is out of scope: queries and new K/V
rows are inputs the caller provides for each iteration. In graph mode the
decode-only iterations replay one captured graph of the L layers' scatter and
decode (record once, replay in one launch: "Hardware-level optimizations"),
sized for ``max_batch`` sequences: slots, tables and lengths are refreshed in
static device buffers before each replay; unused batch rows have context 0
(zero output) and slot -1 (nothing written).
"""

import ctypes

import numpy as np
import torch

from . import _lib as L


class Engine:
    def __init__(self, requests, *, num_layers, num_q_heads, num_kv_heads, head_dim, block_size,
                 num_blocks, num_host_blocks, max_blocks_per_seq, max_batch, chunk_tokens,
                 device="cuda", dtype=torch.bfloat16, use_graph=False):
        self.dev = torch.device(device)
        self.dtype = dtype
        self.L, self.hq, self.hkv, self.d = num_layers, num_q_heads, num_kv_heads, head_dim
        self.bs = block_size
        self.max_blocks = max_blocks_per_seq
        self.max_batch = max_batch
        self.scale = 1.0 / float(np.sqrt(head_dim))
        self.sched = L.Scheduler(requests, num_blocks=num_blocks, num_host_blocks=num_host_blocks,
                                 block_size=block_size, max_blocks_per_seq=max_blocks_per_seq,
                                 max_batch=max_batch, chunk_tokens=chunk_tokens)
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        hshape = (max(num_host_blocks, 1), num_kv_heads, block_size, head_dim)
        self.key_caches = [torch.zeros(shape, dtype=dtype, device=self.dev) for _ in range(self.L)]
        self.value_caches = [torch.zeros(shape, dtype=dtype, device=self.dev)
                             for _ in range(self.L)]
        self.host_keys = [torch.zeros(hshape, dtype=dtype).pin_memory() for _ in range(self.L)]
        self.host_values = [torch.zeros(hshape, dtype=dtype).pin_memory() for _ in range(self.L)]
        self.max_ctx = max_blocks_per_seq * block_size
        self.graph_ws = None       # decode workspace captured in the graph
        self.eager_ws = None       # grown on demand for eager decode calls
        self.use_graph = use_graph
        self.graph = None
        if use_graph:
            self._static_buffers()
        self.decode_tokens = 0
        self.iterations = 0

    # ---------------------------------------------------------------- helpers
    def _i64(self, a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).to(self.dev,
                                                                         non_blocking=True)

    def _i32(self, a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(self.dev,
                                                                         non_blocking=True)

    def done(self):
        return self.sched.done()

    def _workspace(self, num_seqs, max_ctx):
        need = L.pa_decode_workspace_size(num_seqs, self.hq, self.hkv, self.d, self.bs, max_ctx)
        if self.eager_ws is None or self.eager_ws.numel() < need:
            self.eager_ws = L.decode_workspace(num_seqs, self.hq, self.hkv, self.d, self.bs,
                                               max_ctx, self.dev)
        return self.eager_ws

    # ------------------------------------------------------------------ graph
    def _static_buffers(self):
        B = self.max_batch
        self.g_slots = torch.full((B,), -1, dtype=torch.int64, device=self.dev)
        # tables and lengths share one buffer so that one copy refreshes both
        self.g_meta = torch.zeros((B * (self.max_blocks + 1),), dtype=torch.int32, device=self.dev)
        self.g_tables = self.g_meta[:B * self.max_blocks].view(B, self.max_blocks)
        self.g_lens = self.g_meta[B * self.max_blocks:]
        # two pinned staging sets, each reused once its previous copy is done
        self.h_slots = [torch.full((B,), -1, dtype=torch.int64).pin_memory() for _ in range(2)]
        self.h_meta = [torch.zeros((B * (self.max_blocks + 1),), dtype=torch.int32).pin_memory()
                       for _ in range(2)]
        self.h_done = [None, None]
        self.h_next = 0
        self.g_q = [torch.zeros((B, self.hq, self.d), dtype=self.dtype, device=self.dev)
                    for _ in range(self.L)]
        self.g_k = [torch.zeros((B, self.hkv, self.d), dtype=self.dtype, device=self.dev)
                    for _ in range(self.L)]
        self.g_v = [torch.zeros((B, self.hkv, self.d), dtype=self.dtype, device=self.dev)
                    for _ in range(self.L)]
        self.g_out = [torch.zeros((B, self.hq, self.d), dtype=torch.float32, device=self.dev)
                      for _ in range(self.L)]

    def _graph_body(self):
        for layer in range(self.L):
            L.pa_reshape_and_cache(self.g_k[layer], self.g_v[layer], self.key_caches[layer],
                                   self.value_caches[layer], self.g_slots)
            L.pa_decode(self.g_q[layer], self.key_caches[layer], self.value_caches[layer],
                        self.g_tables, self.g_lens, self.scale, self.max_ctx,
                        out=self.g_out[layer], workspace=self.graph_ws)

    def static_decode_inputs(self):
        """The graph's input buffers (lists per layer of [max_batch, ...]):
        decode inputs that a caller writes here in place are used without a
        copy."""
        return {"q_dec": self.g_q, "k_dec": self.g_k, "v_dec": self.g_v}

    def _capture(self):
        self.graph_ws = L.decode_workspace(self.max_batch, self.hq, self.hkv, self.d, self.bs,
                                           self.max_ctx, self.dev)
        # the body runs once outside capture (one-time library set-up), on
        # buffers that write nothing (every slot -1, every context 0)
        side = torch.cuda.Stream(self.dev)
        side.wait_stream(torch.cuda.current_stream(self.dev))
        with torch.cuda.stream(side):
            self._graph_body()
        torch.cuda.current_stream(self.dev).wait_stream(side)
        torch.cuda.synchronize(self.dev)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self._graph_body()
        torch.cuda.synchronize(self.dev)

    # ------------------------------------------------------------------- step
    def step(self, inputs_fn):
        """Run one iteration. ``inputs_fn(plan)`` returns the iteration's
        per-layer inputs: a dict with lists (one tensor per layer) ``q_dec``
        [n_dec, Hq, d], ``k_dec`` / ``v_dec`` [n_dec, Hkv, d], ``q_pre``
        [rows, Hq, d], ``k_pre`` / ``v_pre`` [rows, Hkv, d]. Returns
        (plan, decode outputs per layer, prefill outputs per layer); in graph
        mode the decode outputs are views of the graph's output buffers, valid
        until the next step."""
        plan = self.sched.step()
        n_dec = len(plan["decode_seqs"])
        n_rows = int(plan["prefill_cu"][-1])
        inputs = inputs_fn(plan)
        self.iterations += 1
        self.decode_tokens += n_dec

        if len(plan["swap_in"]):
            pairs = self._i64(plan["swap_in"])
            for layer in range(self.L):
                L.pa_swap_in(self.key_caches[layer], self.value_caches[layer],
                             self.host_keys[layer], self.host_values[layer], pairs)
        if len(plan["swap_out"]):
            pairs = self._i64(plan["swap_out"])
            for layer in range(self.L):
                L.pa_swap_out(self.key_caches[layer], self.value_caches[layer],
                              self.host_keys[layer], self.host_values[layer], pairs)

        dec_tables = dec_lens = None
        if n_dec:
            dec_tables, dec_lens = self.sched.tables(plan["decode_seqs"])
        graph_ok = self.use_graph and n_rows == 0 and n_dec <= self.max_batch
        if graph_ok and n_dec:
            if self.graph is None:
                self._capture()
            B, mb = self.max_batch, self.max_blocks
            k = self.h_next
            self.h_next ^= 1
            if self.h_done[k] is not None:
                self.h_done[k].synchronize()      # this set's previous copy has run
            hs = self.h_slots[k].numpy()
            hs[:] = -1
            hs[:n_dec] = plan["decode_slots"]
            hm = self.h_meta[k].numpy()
            tab = hm[:B * mb].reshape(B, mb)
            tab[:] = -1
            tab[:n_dec] = dec_tables
            hm[B * mb:] = 0
            hm[B * mb:B * mb + n_dec] = dec_lens
            stream = torch.cuda.current_stream(self.dev)
            self.g_slots.copy_(self.h_slots[k], non_blocking=True)
            self.g_meta.copy_(self.h_meta[k], non_blocking=True)
            self.h_done[k] = torch.cuda.Event()
            self.h_done[k].record(stream)
            for layer in range(self.L):
                for name, buf in (("q_dec", self.g_q), ("k_dec", self.g_k), ("v_dec", self.g_v)):
                    src = inputs[name][layer]
                    if src.data_ptr() != buf[layer].data_ptr():   # not already in place
                        buf[layer][:n_dec].copy_(src)
            self.graph.replay()
            return plan, [o[:n_dec] for o in self.g_out], []

        slots = np.concatenate([plan["prefill_slots"], plan["decode_slots"]]).astype(np.int64)
        slots_d = self._i64(slots) if slots.size else None
        if n_rows:
            npf = len(plan["prefill_seqs"])
            pre_tables, _ = self.sched.tables(plan["prefill_seqs"])
            cu = plan["prefill_cu"]
            pre_ctx = plan["prefill_start"] + (cu[1:] - cu[:-1])
            pt, pc, pcu = self._i32(pre_tables), self._i32(pre_ctx), self._i32(cu)
            max_q = int((cu[1:] - cu[:-1]).max())
            max_pre_ctx = int(pre_ctx.max())
        if n_dec:
            dt, dl = self._i32(dec_tables), self._i32(dec_lens)
            max_dec_ctx = int(dec_lens.max())
            ws = self._workspace(n_dec, max_dec_ctx)
        dec_out, pre_out = [], []
        for layer in range(self.L):
            kc, vc = self.key_caches[layer], self.value_caches[layer]
            if slots_d is not None:
                if n_rows and n_dec:
                    k_new = torch.cat([inputs["k_pre"][layer], inputs["k_dec"][layer]])
                    v_new = torch.cat([inputs["v_pre"][layer], inputs["v_dec"][layer]])
                elif n_rows:
                    k_new, v_new = inputs["k_pre"][layer], inputs["v_pre"][layer]
                else:
                    k_new, v_new = inputs["k_dec"][layer], inputs["v_dec"][layer]
                L.pa_reshape_and_cache(k_new, v_new, kc, vc, slots_d)
            if n_rows:
                pre_out.append(L.pa_prefill_chunk(inputs["q_pre"][layer], kc, vc, pt, pc, pcu,
                                                  max_q, self.scale, max_pre_ctx))
            if n_dec:
                dec_out.append(L.pa_decode(inputs["q_dec"][layer], kc, vc, dt, dl, self.scale,
                                           max_dec_ctx, workspace=ws))
        return plan, dec_out, pre_out

    def close(self):
        self.sched.close()


class _EngineConfig(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("scale", ctypes.c_float), ("use_graph", ctypes.c_int32),
                ("sched", L._SchedConfig)]


_BUFFER_FIELDS = ("key_caches", "value_caches", "host_keys", "host_values", "q_dec", "k_dec",
                  "v_dec", "q_pre", "k_pre", "v_pre", "out_dec", "out_pre")


class _EngineBuffers(ctypes.Structure):
    _fields_ = [(n, ctypes.POINTER(ctypes.c_void_p)) for n in _BUFFER_FIELDS]


class NativeEngine:
    """The same driver as ``Engine`` with the per-iteration work in C++
    (include/pa_engine.h): ``plan()`` schedules, the caller writes the
    iteration's inputs into ``inputs`` (per layer, rows in plan order), and
    ``execute()`` enqueues the device work on the engine's own stream (graph
    launches need a stream other than the legacy default one), ordered after
    the caller's stream; results are visible to the caller's stream after
    ``execute()`` returns. A caller that works on ``stream`` itself (``with
    torch.cuda.stream(engine.stream)``) saves the two cross-stream waits per
    iteration."""

    def __init__(self, requests, *, num_layers, num_q_heads, num_kv_heads, head_dim, block_size,
                 num_blocks, num_host_blocks, max_blocks_per_seq, max_batch, chunk_tokens,
                 device="cuda", use_graph=False):
        self.dev = torch.device(device)
        self.L, self.hq, self.hkv, self.d = num_layers, num_q_heads, num_kv_heads, head_dim
        self.max_batch, self.chunk = max_batch, chunk_tokens
        bf = torch.bfloat16
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        hshape = (max(num_host_blocks, 1), num_kv_heads, block_size, head_dim)
        Lr = range(num_layers)
        self.key_caches = [torch.zeros(shape, dtype=bf, device=self.dev) for _ in Lr]
        self.value_caches = [torch.zeros(shape, dtype=bf, device=self.dev) for _ in Lr]
        self.host_keys = [torch.zeros(hshape, dtype=bf).pin_memory() for _ in Lr]
        self.host_values = [torch.zeros(hshape, dtype=bf).pin_memory() for _ in Lr]

        def dev(rows, heads, dtype=bf):
            return [torch.zeros((rows, heads, head_dim), dtype=dtype, device=self.dev) for _ in Lr]
        self.inputs = {"q_dec": dev(max_batch, num_q_heads), "k_dec": dev(max_batch, num_kv_heads),
                       "v_dec": dev(max_batch, num_kv_heads), "q_pre": dev(chunk_tokens, num_q_heads),
                       "k_pre": dev(chunk_tokens, num_kv_heads),
                       "v_pre": dev(chunk_tokens, num_kv_heads)}
        self.out_dec = dev(max_batch, num_q_heads, torch.float32)
        self.out_pre = dev(chunk_tokens, num_q_heads, torch.float32)

        def ptrs(ts):
            a = (ctypes.c_void_p * num_layers)(*[t.data_ptr() for t in ts])
            self._keep.append(a)
            return ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p))
        self._keep = []
        bufs = _EngineBuffers(ptrs(self.key_caches), ptrs(self.value_caches), ptrs(self.host_keys),
                              ptrs(self.host_values), ptrs(self.inputs["q_dec"]),
                              ptrs(self.inputs["k_dec"]), ptrs(self.inputs["v_dec"]),
                              ptrs(self.inputs["q_pre"]), ptrs(self.inputs["k_pre"]),
                              ptrs(self.inputs["v_pre"]), ptrs(self.out_dec), ptrs(self.out_pre))
        cfg = _EngineConfig(num_layers, num_q_heads, num_kv_heads, head_dim,
                            1.0 / float(np.sqrt(head_dim)), int(bool(use_graph)),
                            L._SchedConfig(num_blocks, num_host_blocks, block_size,
                                           max_blocks_per_seq, max_batch, chunk_tokens))
        prompts = np.ascontiguousarray([int(p) for p, _ in requests], dtype=np.int32)
        outputs = np.ascontiguousarray([int(o) for _, o in requests], dtype=np.int32)
        self.stream = torch.cuda.Stream(self.dev)
        torch.cuda.synchronize(self.dev)        # the zero-filled buffers above are in place
        self._lib = L.lib()
        h = ctypes.c_void_p()
        L._check("pa_engine_create", self._lib.pa_engine_create(
            ctypes.byref(cfg), ctypes.byref(bufs), prompts.ctypes.data_as(ctypes.c_void_p),
            outputs.ctypes.data_as(ctypes.c_void_p), len(requests),
            ctypes.c_void_p(self.stream.cuda_stream), ctypes.byref(h)))
        self._h = h
        self.decode_tokens = 0

    def done(self):
        return bool(self._lib.pa_engine_done(self._h))

    @property
    def iterations(self):
        return int(self._lib.pa_engine_iterations(self._h))

    @property
    def graph_launches(self):
        return int(self._lib.pa_engine_graph_launches(self._h))

    def plan(self):
        p = L._StepPlan()
        L._check("pa_engine_plan", self._lib.pa_engine_plan(self._h, ctypes.byref(p)))
        plan = L._plan_dict(p)
        self.decode_tokens += len(plan["decode_seqs"])
        return plan

    def execute(self):
        caller = torch.cuda.current_stream(self.dev)
        same = caller.cuda_stream == self.stream.cuda_stream
        if not same:
            self.stream.wait_stream(caller)
        L._check("pa_engine_execute", self._lib.pa_engine_execute(self._h))
        if not same:
            caller.wait_stream(self.stream)

    def step(self, inputs_fn=None):
        """plan(), inputs written (from ``inputs_fn(plan)`` if given), execute();
        returns (plan, decode outputs per layer, prefill outputs per layer) as
        views valid until the next step."""
        plan = self.plan()
        n_dec = len(plan["decode_seqs"])
        rows = int(plan["prefill_cu"][-1])
        if inputs_fn is not None:
            given = inputs_fn(plan)
            for name, bufs in self.inputs.items():
                n = rows if name.endswith("pre") else n_dec
                for layer in range(self.L):
                    src = given[name][layer]
                    if n and src.data_ptr() != bufs[layer].data_ptr():
                        bufs[layer][:n].copy_(src[:n])
        self.execute()
        return plan, [o[:n_dec] for o in self.out_dec] if n_dec else [], \
            [o[:rows] for o in self.out_pre] if rows else []

    def close(self):
        if getattr(self, "_h", None):
            self._lib.pa_engine_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()
