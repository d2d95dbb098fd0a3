"""Continuous-batching step driver: the C++ driver of include/pa_engine.h
(in libpa.so), which runs the native scheduler's plans on the GPU through the
library's own entry points.

Each iteration (How vLLM gets real throughput on H100s, "Continuous batching
removes straggler bubbles"; Dissecting vLLM, "Continuous Batching: Breaking
the Sequence Barrier"; vLLM architecture, memory and benchmarks deep dive,
"Hardware-level optimizations"):

1. the scheduler (C++) plans the iteration on the host;
2. swapped-out blocks come back from the pinned host pool (``pa_swap_in``),
   then a preempted sequence's blocks go out to it (``pa_swap_out``);
3. for every layer: the iteration's new K/V rows - prompt rows of the
   prefill chunks and one token per decoding sequence - are written through
   the slot mapping (``pa_reshape_and_cache``, or its FP8 form), the chunks
   attend to their prefix (``pa_prefill_chunk``) and the decode batch attends
   to its context (``pa_decode``).

The model itself (projections, sampling) is out of scope: queries and new K/V
rows are inputs the caller writes into the engine's buffers for each
iteration. With ``use_graph`` the decode-only iterations replay one captured
HIP graph of the L layers' scatter and decode (record once, replay in one
launch: "Hardware-level optimizations"), sized for ``max_batch`` sequences;
unused batch rows have context 0 (zero output) and slot -1 (nothing written).
This module only marshals: every step runs in the C++ driver.
"""

import ctypes

import numpy as np
import torch

from . import _lib as L


class _EngineConfig(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("scale", ctypes.c_float), ("use_graph", ctypes.c_int32),
                ("sched", L._SchedConfig), ("kv_fp8", ctypes.c_int32)]


_BUFFER_FIELDS = ("key_caches", "value_caches", "host_keys", "host_values", "q_dec", "k_dec",
                  "v_dec", "q_pre", "k_pre", "v_pre", "out_dec", "out_pre", "k_scales",
                  "v_scales")


class _EngineBuffers(ctypes.Structure):
    _fields_ = [(n, ctypes.POINTER(ctypes.c_void_p)) for n in _BUFFER_FIELDS]


class Engine:
    """The C++ step driver: ``plan()`` schedules, the caller writes the
    iteration's inputs into ``inputs`` (per layer, rows in plan order), and
    ``execute()`` enqueues the device work on the engine's own stream (graph
    launches need a stream other than the legacy default one), ordered after
    the caller's stream; results are visible to the caller's stream after
    ``execute()`` returns. A caller that works on ``stream`` itself (``with
    torch.cuda.stream(engine.stream)``) saves the two cross-stream waits per
    iteration. ``kv_fp8``: the caches (and host pools) hold E4M3 codes with
    the per-layer, per-head float32 scales ``k_scales`` / ``v_scales`` (given,
    or 1/64 by default); inputs stay BF16."""

    def __init__(self, requests, *, num_layers, num_q_heads, num_kv_heads, head_dim, block_size,
                 num_blocks, num_host_blocks, max_blocks_per_seq, max_batch, chunk_tokens,
                 device="cuda", use_graph=False, kv_fp8=False, k_scales=None, v_scales=None):
        self.dev = torch.device(device)
        self.L, self.hq, self.hkv, self.d = num_layers, num_q_heads, num_kv_heads, head_dim
        self.max_batch, self.chunk = max_batch, chunk_tokens
        self.kv_fp8 = bool(kv_fp8)
        bf = torch.bfloat16
        cache_t = torch.uint8 if self.kv_fp8 else bf
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        hshape = (max(num_host_blocks, 1), num_kv_heads, block_size, head_dim)
        Lr = range(num_layers)
        self.key_caches = [torch.zeros(shape, dtype=cache_t, device=self.dev) for _ in Lr]
        self.value_caches = [torch.zeros(shape, dtype=cache_t, device=self.dev) for _ in Lr]
        self.host_keys = [torch.zeros(hshape, dtype=cache_t).pin_memory() for _ in Lr]
        self.host_values = [torch.zeros(hshape, dtype=cache_t).pin_memory() for _ in Lr]

        def scales(given):
            if given is None:
                return [torch.full((num_kv_heads,), 1 / 64, dtype=torch.float32,
                                   device=self.dev) for _ in Lr]
            return [torch.as_tensor(x, dtype=torch.float32).to(self.dev).contiguous()
                    for x in given]
        self.k_scales = scales(k_scales) if self.kv_fp8 else []
        self.v_scales = scales(v_scales) if self.kv_fp8 else []

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
        null = ctypes.POINTER(ctypes.c_void_p)()
        bufs = _EngineBuffers(ptrs(self.key_caches), ptrs(self.value_caches), ptrs(self.host_keys),
                              ptrs(self.host_values), ptrs(self.inputs["q_dec"]),
                              ptrs(self.inputs["k_dec"]), ptrs(self.inputs["v_dec"]),
                              ptrs(self.inputs["q_pre"]), ptrs(self.inputs["k_pre"]),
                              ptrs(self.inputs["v_pre"]), ptrs(self.out_dec), ptrs(self.out_pre),
                              ptrs(self.k_scales) if self.kv_fp8 else null,
                              ptrs(self.v_scales) if self.kv_fp8 else null)
        cfg = _EngineConfig(num_layers, num_q_heads, num_kv_heads, head_dim,
                            1.0 / float(np.sqrt(head_dim)), int(bool(use_graph)),
                            L._SchedConfig(num_blocks, num_host_blocks, block_size,
                                           max_blocks_per_seq, max_batch, chunk_tokens),
                            int(self.kv_fp8))
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
