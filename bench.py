"""Benchmark: paged-attention decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--profile]

A step is one pass of the hot path over one batch: for the full decode step
(the default workload, 64 sequences at context 8192, 16 layers, 4 KV / 16
query heads, head dim 256, block size 32, BF16) every layer runs
pa_reshape_and_cache for the new token and then pa_decode over the whole
paged context. Inputs are synthetic (seeded N(0,1), BF16) and resident in HBM
before the timed region. Prints ONE JSON line.

Roofline: the dominant call is pa_decode (its partition kernel plus the small
merge kernel). Its algorithmic bytes per call are the K/V rows of every
attended token, the query, the float32 output and the block-table entries in
use; the live duration comes from HIP events recorded on the launch stream
around every pa_decode call of the timed steps.

cpu_baseline: the fp64 CPU oracle, as it stands, on a bounded sample of the
same workload (one layer's sequences), in worker processes on the host cores.
"""

import argparse
import gc
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense BF16 matrix-core peak, TFLOP/s
DECODE_SOURCES = ["paged_kv_cache_215_amd/csrc/pa_decode.hip",
                  "paged_kv_cache_215_amd/csrc/pa_device.hpp"]
# the grouped decode's prefix pass is the chunk kernel in prefix mode
SHARED_SOURCES = DECODE_SOURCES + ["paged_kv_cache_215_amd/csrc/pa_prefill.hip"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def decode_kernel_name(fp8, group, head_dim, f32=False):
    """The partition kernel pa_decode launches for a shape: groups of 8 query
    heads over BF16 caches, and groups of 8 (and of 4 at d >= 128) over E4M3
    caches, run on the matrix cores; every other shape on the VALU kernel."""
    if not f32 and (group == 8 or (fp8 and group == 4 and head_dim >= 128)):
        return "decode_mfma_kernel"
    return "decode_partition_kernel"


def decode_bytes(layout, num_decode, num_q_heads, num_kv_heads, head_dim, elem_bytes,
                 unique_blocks=False, kv_bytes=None):
    """Algorithmic bytes of one pa_decode call: K+V rows of every attended
    token (each distinct physical block once when unique_blocks), q, float32
    out and the block-table entries in use. kv_bytes is the cache's element
    size when it differs from the query's (FP8: 1 byte per element, plus the
    two per-head float32 scale arrays)."""
    lens = layout.context_lens[:num_decode].astype(np.int64)
    bs = layout.block_size
    nblk = -(-lens // bs)
    if unique_blocks:
        seen = {}
        for b in range(num_decode):
            n = int(lens[b])
            for j in range(int(nblk[b])):
                blk = int(layout.block_tables[b, j])
                rows = min(bs, n - j * bs)
                seen[blk] = max(seen.get(blk, 0), rows)
        kv_tokens = sum(seen.values())
    else:
        kv_tokens = int(lens.sum())
    kv = 2 * kv_tokens * num_kv_heads * head_dim * (elem_bytes if kv_bytes is None else kv_bytes)
    scales = 0 if kv_bytes is None else 2 * num_kv_heads * 4
    q = num_decode * num_q_heads * head_dim * elem_bytes
    out = num_decode * num_q_heads * head_dim * 4
    bt = int(nblk.sum()) * 4
    return kv + scales + q + out + bt


def source_hash(paths):
    """Hash of the sources' code: comments and blank space are dropped, so a
    comment edit keeps the counters that were taken on the same kernel."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


# HBM counter summaries under profiles/: (workload, FP8 cache) -> file stem.
COUNTER_SETS = {
    ("c3_full_step", False): "decode_c3_hbm_counters",
    ("c3_full_step", True): "decode_fp8_c3_hbm_counters",
    ("c4_grpo_cow", False): "decode_c4_hbm_counters",
    ("c2_layer_decode", False): "decode_c2_hbm_counters",
    ("c2_layer_decode", True): "decode_fp8_c2_hbm_counters",
    ("c5_mixed_step", False): "decode_c5_hbm_counters",
    ("c5_mixed_step", True): "decode_fp8_c5_hbm_counters",
    ("c4_grpo_cow", True): "decode_fp8_c4_hbm_counters",
}


def _sources_for(workload):
    return SHARED_SOURCES if workload == "c4_grpo_cow" else DECODE_SOURCES


def load_traffic(workload="c3_full_step", fp8=False):
    """HBM traffic per decode call from the committed rocprofv3 counter
    summary of this workload, only if it was taken on the current kernel
    source."""
    stem = COUNTER_SETS.get((workload, fp8))
    if stem is None:
        return None
    try:
        with open(os.path.join(ROOT, "profiles", stem + ".json")) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("source_hash") != source_hash(_sources_for(workload)):
        return None
    return c.get("hbm_bytes_per_call")


# ---------------------------------------------------------------- CPU leg ---

_ARR = {}


def _cpu_worker_init(folder):
    _ARR["folder"] = folder


def _cpu_arr(name):
    if name not in _ARR:
        _ARR[name] = np.load(os.path.join(_ARR["folder"], name + ".npy"), mmap_mode="r")
    return _ARR[name]


def _cpu_worker(args):
    layer, b, scale, fp8 = args
    import oracle  # the oracle is used here only, to time it
    q = _cpu_arr(f"q{layer}")
    kc = _cpu_arr(f"kc{layer}")
    vc = _cpu_arr(f"vc{layer}")
    bt = _cpu_arr("bt")
    lens = _cpu_arr("lens")
    if fp8:
        return oracle.fp8.decode_fp8_ref(q[b:b + 1], kc, vc, _cpu_arr(f"ks{layer}"),
                                         _cpu_arr(f"vs{layer}"), bt[b:b + 1], lens[b:b + 1], scale)
    return oracle.decode_ref(q[b:b + 1], kc, vc, bt[b:b + 1], lens[b:b + 1], scale)


# Worker processes of the CPU baseline at most: a one-GPU job's CPU share on
# the GPU hosts (the oracle runs one single-threaded process per core).
CPU_SHARE_CORES = 16


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or the platform's name."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def cpu_baseline(case, layers, seq_layers_per_step):
    """Time the oracle on every sequence of the given layers; scale to the
    seconds of a full step (seq_layers_per_step sequence-layers)."""
    import shutil
    import tempfile
    from multiprocessing import get_context
    from workloads import to_numpy_bits

    S = case.num_decode_seqs
    folder = tempfile.mkdtemp(prefix="pa_cpu_baseline_")
    try:
        np.save(os.path.join(folder, "bt.npy"), case.layout.block_tables[:S])
        np.save(os.path.join(folder, "lens.npy"), case.layout.context_lens[:S].astype(np.int64))
        for layer in layers:
            np.save(os.path.join(folder, f"q{layer}.npy"), to_numpy_bits(case.queries[layer]))
            np.save(os.path.join(folder, f"kc{layer}.npy"), to_numpy_bits(case.key_caches[layer]))
            np.save(os.path.join(folder, f"vc{layer}.npy"), to_numpy_bits(case.value_caches[layer]))
            if case.kv_fp8:
                np.save(os.path.join(folder, f"ks{layer}.npy"), case.k_scales[layer].cpu().numpy())
                np.save(os.path.join(folder, f"vs{layer}.npy"), case.v_scales[layer].cpu().numpy())
        try:
            host_cores = len(os.sched_getaffinity(0))
        except AttributeError:
            host_cores = os.cpu_count() or 1
        # one worker per core this process may run on, capped at the 16-core
        # CPU share a one-GPU job gets on these hosts (the affinity mask can
        # list every core of the machine)
        workers = max(1, min(CPU_SHARE_CORES, host_cores))
        saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                                "MKL_NUM_THREADS")}
        for k in saved:
            os.environ[k] = "1"
        try:
            ctx = get_context("spawn")
            with ctx.Pool(workers, initializer=_cpu_worker_init, initargs=(folder,)) as pool:
                # warm every worker (imports, page cache) outside the timed region
                pool.map(_cpu_worker, [(layers[0], b % S, case.scale, case.kv_fp8)
                                       for b in range(workers)], chunksize=1)
                tasks = [(layer, b, case.scale, case.kv_fp8) for layer in layers for b in range(S)]
                t0 = time.perf_counter()
                pool.map(_cpu_worker, tasks, chunksize=1)
                wall = time.perf_counter() - t0
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
    finally:
        shutil.rmtree(folder, ignore_errors=True)
    n_tasks = len(layers) * S
    return {"wall_s": wall, "workers": workers, "host_cores": host_cores, "tasks": n_tasks,
            "step_seconds": wall * seq_layers_per_step / n_tasks}


# ---------------------------------------------------------------- GPU leg ---

def run(args):
    import torch
    import paged_kv_cache_215_amd as pa
    from workloads import make_config_case

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU (MI355X); none is visible")
    pa.lib()                                   # fail loudly if the library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fp8 = args.kv == "fp8"
    log(f"[bench] generating {args.workload} (kv {args.kv}) ...")
    case = make_config_case(args.workload, device=dev, kv_fp8=fp8)
    torch.cuda.synchronize()
    L = case.num_layers
    S = case.num_decode_seqs
    elem = 2 if case.dtype == torch.bfloat16 else 4
    outs = [torch.empty((S, case.num_q_heads, case.head_dim), dtype=torch.float32, device=dev)
            for _ in range(L)]
    workspace = pa.decode_workspace(S, case.num_q_heads, case.num_kv_heads, case.head_dim,
                                    case.block_size, case.max_context_len, dev)
    stream = torch.cuda.current_stream(dev)

    pf = case.prefill
    if pf is not None:
        pf_ctx = int(max(int(x) for x in pf.context_lens.cpu()))
        pf_out = torch.empty((pf.query.shape[0], case.num_q_heads, case.head_dim),
                             dtype=torch.float32, device=dev)
        pf_ws = torch.empty(max(16, pa.pa_prefill_chunk_workspace_size(
            len(pf.q_lens), pf.query.shape[0], pf.max_q_len, case.num_q_heads, case.num_kv_heads,
            case.head_dim, case.block_size, pf_ctx)), dtype=torch.uint8, device=dev)

    # Event pairs for the timed calls are created before the timed region, so
    # that no allocation (and no garbage collection it might start) falls
    # inside it.
    spare_events = []

    def timed(events, fn):
        if events is None:
            fn()
            return
        e0, e1 = (spare_events.pop() if spare_events else
                  (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
        e0.record(stream)
        fn()
        e1.record(stream)
        events.append((e0, e1))

    def write(layer):
        if fp8:
            pa.pa_reshape_and_cache_fp8(case.new_keys[layer], case.new_values[layer],
                                        case.key_caches[layer], case.value_caches[layer],
                                        case.slot_mapping, case.k_scales[layer],
                                        case.v_scales[layer])
        else:
            pa.pa_reshape_and_cache(case.new_keys[layer], case.new_values[layer],
                                    case.key_caches[layer], case.value_caches[layer],
                                    case.slot_mapping)

    # Copy-on-write groups (the shared prompts of forked rollouts), found from
    # the block tables on the host before timing: such a batch is decoded
    # with pa_decode_shared, which reads each group's shared blocks once.
    groups = None
    if not args.no_shared_prefix:
        cu, pl, mg, mp = pa.find_shared_prefixes(case.layout.block_tables[:S],
                                                 case.layout.context_lens[:S], case.block_size)
        if len(pl):
            groups = (torch.as_tensor(cu, device=dev), torch.as_tensor(pl, device=dev), mg, mp)
            workspace = pa.decode_shared_workspace(S, case.num_q_heads, case.num_kv_heads,
                                                   case.head_dim, case.block_size,
                                                   case.max_context_len, len(pl), mg, mp, dev)
            log(f"[bench] {len(pl)} copy-on-write groups (largest {mg}, prefix {mp}): "
                f"pa_decode_shared")

    def attend(layer):
        if groups is not None:
            kw = dict(k_scale=case.k_scales[layer], v_scale=case.v_scales[layer]) if fp8 else {}
            pa.pa_decode_shared(case.queries[layer], case.key_caches[layer],
                                case.value_caches[layer], case.block_tables, case.context_lens,
                                groups[0], groups[1], groups[2], groups[3], case.scale,
                                case.max_context_len, out=outs[layer], workspace=workspace, **kw)
            return
        if fp8:
            pa.pa_decode_fp8(case.queries[layer], case.key_caches[layer], case.value_caches[layer],
                             case.k_scales[layer], case.v_scales[layer], case.block_tables,
                             case.context_lens, case.scale, case.max_context_len,
                             out=outs[layer], workspace=workspace)
        else:
            pa.pa_decode(case.queries[layer], case.key_caches[layer], case.value_caches[layer],
                         case.block_tables, case.context_lens, case.scale, case.max_context_len,
                         out=outs[layer], workspace=workspace)

    def prefill(layer):
        if fp8:
            pa.pa_prefill_chunk_fp8(pf.query, case.key_caches[layer], case.value_caches[layer],
                                    case.k_scales[layer], case.v_scales[layer], pf.block_tables,
                                    pf.context_lens, pf.cu_q_lens, pf.max_q_len, case.scale,
                                    pf_ctx, out=pf_out, workspace=pf_ws)
        else:
            pa.pa_prefill_chunk(pf.query, case.key_caches[layer], case.value_caches[layer],
                                pf.block_tables, pf.context_lens, pf.cu_q_lens, pf.max_q_len,
                                case.scale, pf_ctx, out=pf_out, workspace=pf_ws)

    def step(dec_events=None, pf_events=None):
        for layer in range(L):
            if case.slot_mapping is not None:
                write(layer)
            timed(dec_events, lambda: attend(layer))
            if pf is not None:
                timed(pf_events, lambda: prefill(layer))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    dec_events, pf_events = [], []
    calls = args.steps * L * (2 if pf is not None else 1)
    spare_events.extend((torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                        for _ in range(calls))
    gc.collect()
    gc.disable()  # (the interpreter's collector stays out of the timed region)
    try:
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step(dec_events, pf_events)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    finally:
        gc.enable()
    decode_ms = [a.elapsed_time(b) for a, b in dec_events]
    avg_decode_s = float(np.mean(decode_ms)) / 1e3

    # The same step replayed from one captured HIP graph (a second, labelled
    # line: the headline value stays the eager step). Every replay rewrites
    # the same new tokens and recomputes the same outputs, so the outputs of
    # the first and of the last replay must equal the eager step's bit for bit.
    graph_line = None
    if args.graph_steps > 0:
        eager_out = [o.clone() for o in outs]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        first_ok = all(torch.equal(a, b) for a, b in zip(outs, eager_out))
        g0 = time.perf_counter()
        for _ in range(args.graph_steps):
            graph.replay()
        torch.cuda.synchronize()
        g_elapsed = time.perf_counter() - g0
        last_ok = all(torch.equal(a, b) for a, b in zip(outs, eager_out))
        if not (first_ok and last_ok):
            raise SystemExit("graph replay differs from the eager step")
        graph_line = {"steps": args.graph_steps,
                      "ms_per_step": round(g_elapsed / args.graph_steps * 1e3, 4),
                      "tokens_per_s": round(S * args.graph_steps / g_elapsed, 2),
                      "outputs_equal_eager": True}
        log(f"[bench] graph replay: {graph_line}")
        del graph, eager_out

    # Cold-cache decode calls (one-layer workloads): a 1 GiB write, more than
    # the 256 MB last-level cache holds, goes between calls, outside the events,
    # so every call reads its K/V from HBM. The full 16-layer step needs none:
    # each layer's 2 GiB of K/V already exceeds that cache.
    cold_ms = []
    if L == 1 and args.cold_calls > 0:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        for i in range(args.cold_calls):
            flush.fill_(i & 0xFF)
            ev = []
            timed(ev, lambda: attend(0))
            torch.cuda.synchronize()
            cold_ms.append(ev[0][0].elapsed_time(ev[0][1]))
        del flush

    def pctl(ms):
        q = np.percentile(np.asarray(ms) * 1e3, [10, 50, 90])
        return {"p10": round(float(q[0]), 2), "p50": round(float(q[1]), 2), "p90": round(float(q[2]), 2)}

    unique = args.workload == "c4_grpo_cow"
    bytes_call = decode_bytes(case.layout, S, case.num_q_heads, case.num_kv_heads, case.head_dim,
                              elem, unique_blocks=unique, kv_bytes=1 if fp8 else None)
    achieved_gbs = bytes_call / avg_decode_s / 1e9
    ms_per_step = elapsed / args.steps * 1e3
    tokens_per_s = S * args.steps / elapsed
    log(f"[bench] {args.steps} steps in {elapsed * 1e3:.2f} ms: {ms_per_step:.3f} ms/step, "
        f"{tokens_per_s:.1f} tok/s; pa_decode avg {avg_decode_s * 1e6:.1f} us "
        f"(min {min(decode_ms) * 1e3:.1f}, max {max(decode_ms) * 1e3:.1f}), "
        f"{achieved_gbs:.1f} GB/s = {achieved_gbs / HBM_PEAK_GBS:.3f} of HBM peak")
    traffic = (load_traffic(args.workload, fp8)
               if groups is not None or args.workload != "c4_grpo_cow" else None)

    result = {
        "metric": "paged-attn decode tokens/s & achieved HBM GB/s (% of 8 TB/s), 1 MI355X",
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8_e4m3 kv, bf16 q" if fp8 else "bf16") if elem == 2 else "f32",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "num_seqs": S,
            "context_len": int(case.max_context_len),
            "layers": L,
            "num_q_heads": case.num_q_heads,
            "num_kv_heads": case.num_kv_heads,
            "head_dim": case.head_dim,
            "block_size": case.block_size,
            "kv_cache": "fp8_e4m3 (per-head scales)" if fp8 else "bf16",
            "step": ("per layer: " +
                     ("pa_reshape_and_cache_fp8(new tokens) + " if fp8 and case.slot_mapping is not None else
                      "pa_reshape_and_cache(new tokens) + " if case.slot_mapping is not None else "") +
                     ("pa_decode_shared" if groups is not None else
                      "pa_decode_fp8" if fp8 else "pa_decode")) +
                    ((" + pa_prefill_chunk_fp8" if fp8 else " + pa_prefill_chunk")
                     if pf is not None else ""),
        },
        "roofline": {
            "kernel": (("pa_decode_shared (prefill_kernel prefix pass + " if groups is not None else
                        ("pa_decode_fp8 (" if fp8 else "pa_decode (")) +
                       f"{decode_kernel_name(fp8, case.num_q_heads // case.num_kv_heads, case.head_dim, elem == 4)}"
                       " + decode_merge_kernel)"),
            "bound": "hbm",
            "achieved": round(achieved_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_call": bytes_call,
            "avg_call_us": round(avg_decode_s * 1e6, 2),
            "call_us": pctl(decode_ms),
        },
        "cpu_baseline": None,
    }
    if unique:
        # shared prompt blocks counted once per reader: the rate the call would
        # need without prefix sharing (may exceed the HBM peak)
        logical = decode_bytes(case.layout, S, case.num_q_heads, case.num_kv_heads, case.head_dim,
                               elem, unique_blocks=False, kv_bytes=1 if fp8 else None)
        result["roofline"]["logical_bytes_per_call"] = logical
        result["roofline"]["effective_logical_gbs"] = round(logical / avg_decode_s / 1e9, 1)
    if graph_line is not None:
        result["graph_replay"] = graph_line
    if cold_ms:
        cold_s = float(np.median(cold_ms)) / 1e3
        result["roofline"]["cold_cache"] = {
            "calls": len(cold_ms), "flush_bytes": 1 << 30, "call_us": pctl(cold_ms),
            "achieved_at_p50": round(bytes_call / cold_s / 1e9, 1),
            "frac_at_p50": round(bytes_call / cold_s / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"[bench] cold-cache pa_decode p50 {cold_s * 1e6:.1f} us, "
            f"{bytes_call / cold_s / 1e9:.1f} GB/s")
    if pf is not None:
        pf_s = float(np.mean([a.elapsed_time(b) for a, b in pf_events])) / 1e3
        flop = 0
        for pre, ql in zip(pf.prefix_lens, pf.q_lens):
            flop += 4 * case.num_q_heads * case.head_dim * sum(pre + i + 1 for i in range(ql))
        result["prefill"] = {
            "kernel": ("pa_prefill_chunk_fp8" if fp8 else "pa_prefill_chunk") +
                      " (prefill_kernel + prefill_merge_kernel)",
            "bound": "mfma",
            "avg_call_us": round(pf_s * 1e6, 2),
            "algorithmic_flop_per_call": flop,
            "achieved": round(flop / pf_s / 1e12, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(flop / pf_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        }
        log(f"[bench] pa_prefill_chunk avg {pf_s * 1e6:.1f} us, {flop / pf_s / 1e12:.1f} TFLOP/s")

    if not args.no_cpu_baseline:
        layers = list(range(min(L, args.cpu_sample_layers)))
        log(f"[bench] cpu baseline: oracle on {S} sequences x layers {layers} ...")
        cb = cpu_baseline(case, layers, S * L)
        result["cpu_baseline"] = {
            "value": round(S / cb["step_seconds"], 4),
            "unit": "tokens/s",
            "cores": cb["workers"],
            "workers": cb["workers"],
            "host_cores": cb["host_cores"],
            "cpu": cpu_model(),
            "effective_gbs": round(bytes_call * L / cb["step_seconds"] / 1e9, 3),
            "kind": "oracle",
            "sample": f"fp64 oracle {'decode_fp8_ref' if fp8 else 'decode_ref'} on all {S} "
                      f"sequences of {len(layers)} of the {L} "
                      f"layers ({cb['tasks']} of {S * L} sequence-layers per step; "
                      f"{cb['wall_s']:.2f} s wall on {cb['workers']} worker processes), "
                      f"scaled to a full step",
        }
        log(f"[bench] cpu baseline {cb['wall_s']:.2f} s for {cb['tasks']} seq-layers on "
            f"{cb['workers']} workers")
    print(json.dumps(result), flush=True)


def copy_calibration(nbytes=1 << 30, reps=5):
    """A plain device copy of known size (for scaling the HBM byte counters)."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": nbytes, "bytes_written": nbytes,
                                           "reps": reps}}), flush=True)


# ------------------------------------------------------- profile summaries ---

_KT = ("cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats --output-format csv "
       "-d <out>/{tag} -o kt -- python3 <repo>/bench.py {args} --no-cpu-baseline")
_PMC = ("rocprofv3 --pmc {counter} --output-format csv -d <out>/{tag} -o p -- "
        "python3 <repo>/bench.py {args} --no-cpu-baseline")

# Kernel traces: tag -> (bench arguments, title, summary file).
TRACES = {
    "kt_c3": ("--steps 5 --warmup 1",
              "pa kernels, 64 seqs x 8192 ctx x 16 layers (bs 32)", "decode_c3_kernel_trace.md"),
    "kt_c3_fp8": ("--kv fp8 --steps 5 --warmup 1",
                  "pa kernels, FP8 E4M3 cache, 64 seqs x 8192 ctx x 16 layers (bs 32)",
                  "decode_fp8_c3_kernel_trace.md"),
    "kt_c5": ("--workload c5_mixed_step --steps 5 --warmup 1 --cold-calls 0",
              "pa kernels, mixed step: 255 decode seqs + 512-row prefill chunk",
              "mixed_c5_kernel_trace.md"),
    "kt_c5_fp8": ("--workload c5_mixed_step --kv fp8 --steps 5 --warmup 1 --cold-calls 0",
                  "pa kernels, mixed step over an FP8 cache: 255 decode seqs + 512-row "
                  "prefill chunk", "mixed_fp8_c5_kernel_trace.md"),
    "kt_c2": ("--workload c2_layer_decode --steps 10 --warmup 2 --cold-calls 10",
              "pa kernels, one ragged layer: 32 seqs, contexts U[512, 8192], bs 16",
              "decode_c2_kernel_trace.md"),
    "kt_c2_fp8": ("--workload c2_layer_decode --kv fp8 --steps 10 --warmup 2 --cold-calls 10",
                  "pa kernels, one ragged layer over an FP8 cache: 32 seqs, contexts "
                  "U[512, 8192], bs 16", "decode_fp8_c2_kernel_trace.md"),
    "kt_c4": ("--workload c4_grpo_cow --steps 10 --warmup 2 --cold-calls 10",
              "pa kernels, copy-on-write batch (8 prompts x 16 rollouts, 4096-token shared "
              "prompt, tails U[0, 1024], bs 16) through pa_decode_shared",
              "decode_c4_kernel_trace.md"),
    "kt_c4_fp8": ("--workload c4_grpo_cow --kv fp8 --steps 10 --warmup 2 --cold-calls 10",
                  "pa kernels, the copy-on-write batch over an FP8 cache through "
                  "pa_decode_shared", "decode_fp8_c4_kernel_trace.md"),
}

# HBM counter passes: (workload, FP8 cache) -> (bench arguments, description,
# kernel-name filters of the decode call's kernels).
COUNTER_RUNS = {
    ("c3_full_step", False): ("--steps 2 --warmup 1",
                              "64 seqs x 8192 ctx, bs 32, 4 KV / 16 query heads, d 256, BF16",
                              ("decode_partition_kernel", "decode_mfma_kernel",
                               "decode_merge_kernel")),
    ("c3_full_step", True): ("--kv fp8 --steps 2 --warmup 1",
                             "64 seqs x 8192 ctx, bs 32, 4 KV / 16 query heads, d 256, FP8 E4M3",
                             ("decode_partition_kernel", "decode_mfma_kernel",
                              "decode_merge_kernel")),
    ("c4_grpo_cow", False): ("--workload c4_grpo_cow --steps 2 --warmup 1 --cold-calls 0",
                             "copy-on-write batch, 8 x 16 rollouts of a 4096-token prompt, "
                             "tails U[0, 1024], bs 16, BF16, pa_decode_shared",
                             ("prefill_kernel", "decode_partition_kernel", "decode_mfma_kernel",
                              "decode_merge_kernel")),
    ("c2_layer_decode", False): ("--workload c2_layer_decode --steps 2 --warmup 1 --cold-calls 0",
                                 "32 seqs, contexts U[512, 8192], bs 16, 4 KV / 16 query heads, "
                                 "d 256, BF16",
                                 ("decode_partition_kernel", "decode_mfma_kernel",
                                  "decode_merge_kernel")),
    ("c2_layer_decode", True): ("--workload c2_layer_decode --kv fp8 --steps 2 --warmup 1 "
                                "--cold-calls 0",
                                "32 seqs, contexts U[512, 8192], bs 16, 4 KV / 16 query heads, "
                                "d 256, FP8 E4M3",
                                ("decode_partition_kernel", "decode_mfma_kernel",
                                 "decode_merge_kernel")),
    ("c5_mixed_step", False): ("--workload c5_mixed_step --steps 2 --warmup 1 --cold-calls 0",
                               "the mixed step's decode of 255 seqs (prefill chunk not "
                               "counted), bs 16, BF16",
                               ("decode_partition_kernel", "decode_mfma_kernel",
                                "decode_merge_kernel")),
    ("c5_mixed_step", True): ("--workload c5_mixed_step --kv fp8 --steps 2 --warmup 1 "
                              "--cold-calls 0",
                              "the mixed step's decode of 255 seqs (prefill chunk not "
                              "counted), bs 16, FP8 E4M3",
                              ("decode_partition_kernel", "decode_mfma_kernel",
                               "decode_merge_kernel")),
    ("c4_grpo_cow", True): ("--workload c4_grpo_cow --kv fp8 --steps 2 --warmup 1 --cold-calls 0",
                            "copy-on-write batch, 8 x 16 rollouts of a 4096-token prompt, "
                            "tails U[0, 1024], bs 16, FP8 E4M3, pa_decode_shared",
                            ("prefill_kernel", "decode_partition_kernel", "decode_mfma_kernel",
                             "decode_merge_kernel")),
}

_COUNTER_STEMS = {"c2_layer_decode": "c2", "c3_full_step": "c3", "c4_grpo_cow": "c4",
                  "c5_mixed_step": "c5"}


def _counter_tags(key):
    stem = _COUNTER_STEMS[key[0]]
    return (f"pmc_fetch_{stem}{'_fp8' if key[1] else ''}",
            f"pmc_write_{stem}{'_fp8' if key[1] else ''}")


PROFILE_COMMANDS = {tag: _KT.format(tag=tag, args=a) for tag, (a, _, _) in TRACES.items()}
for _key, (_args, _, _) in COUNTER_RUNS.items():
    _f, _w = _counter_tags(_key)
    PROFILE_COMMANDS[_f] = _PMC.format(counter="FETCH_SIZE", tag=_f, args=_args)
    PROFILE_COMMANDS[_w] = _PMC.format(counter="WRITE_SIZE", tag=_w, args=_args)
PROFILE_COMMANDS.update({
    "pmc_prefill_c5": "rocprofv3 --pmc SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU "
                      "SQ_ACTIVE_INST_VALU SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_ACTIVE_INST_LDS "
                      "SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE --output-format csv -d <out>/pmc_prefill_c5 "
                      "-o p -- python3 <repo>/bench.py --workload c5_mixed_step --steps 2 --warmup 1 "
                      "--cold-calls 0 --no-cpu-baseline",
    "pmc_fetch_copy": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/pmc_fetch_copy -o p -- "
                      "python3 <repo>/bench.py --copy-calib",
    "pmc_write_copy": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/pmc_write_copy -o p -- "
                      "python3 <repo>/bench.py --copy-calib",
})



def _csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(folder, suffix):
    for dirpath, _, files in os.walk(folder):
        for name in files:
            if name.endswith(suffix):
                return os.path.join(dirpath, name)
    raise FileNotFoundError(f"no *{suffix} under {folder}")


def _short(name):
    name = name.replace("(pa::DecodeArgs)", "").replace("(pa::PrefillArgs)", "")
    name = name.replace("(pa::ScatterArgs)", "").replace("void ", "")
    return name if len(name) < 70 else name[:67] + "..."


def _counter_means(folder, counter):
    out = {}
    for r in _csv(_find(folder, "counter_collection.csv")):
        if r["Counter_Name"] != counter:
            continue
        out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: (len(v), sum(v) / len(v)) for k, v in out.items()}


SIMDS, XCDS = 256 * 4, 8   # MI355X: 256 CUs of 4 SIMDs in 8 XCDs


def _summarize_prefill_counters(folder, kt_folder, dst):
    """Matrix-unit and VALU activity of the prefill kernel in the mixed step.
    SQ_VALU_MFMA_BUSY_CYCLES sums the busy cycles of every SIMD's matrix
    unit; GRBM_GUI_ACTIVE sums the GPU's busy cycles over the XCDs, so one
    XCD's share is the kernel's length in cycles."""
    names = ["SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU",
             "SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_LDS", "SQ_LDS_BANK_CONFLICT",
             "GRBM_GUI_ACTIVE"]
    vals = {}
    for c in names:
        m = {k: v for k, v in _counter_means(folder, c).items() if "prefill_kernel" in k}
        if m:
            kname = next(iter(m))
            vals[c] = m[kname][1]
    if "GRBM_GUI_ACTIVE" not in vals or "SQ_VALU_MFMA_BUSY_CYCLES" not in vals:
        return
    cycles = vals["GRBM_GUI_ACTIVE"] / XCDS
    lines = [f"# Counters of the prefill kernel in the mixed step (`{_short(kname)}`)", "",
             "512-row causal chunk on a 3,584-token paged prefix, 16 query / 4 KV heads, d 256, "
             "BF16; per dispatch, averaged over the profiled steps.", "",
             "| counter | per dispatch |", "|---|---|"]
    lines += [f"| {c} | {vals[c]:,.0f} |" for c in names if c in vals]
    mfma_busy = vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * cycles)
    lines += ["", f"Kernel length: {cycles:,.0f} cycles (GRBM_GUI_ACTIVE / {XCDS} XCDs).", "",
              f"Matrix-unit busy: {mfma_busy * 100:.1f} % of the {SIMDS} SIMDs' cycles "
              f"(SQ_VALU_MFMA_BUSY_CYCLES / ({SIMDS} x kernel cycles)); "
              f"{vals['SQ_VALU_MFMA_BUSY_CYCLES'] / max(1.0, vals['SQ_INSTS_MFMA']):.1f} busy cycles "
              "per matrix instruction."]
    if "SQ_WAVE_CYCLES" in vals and "SQ_WAIT_ANY" in vals:
        lines.append(f"Waves waiting: {vals['SQ_WAIT_ANY'] / vals['SQ_WAVE_CYCLES'] * 100:.1f} % of "
                     f"their cycles; VALU issue: "
                     f"{vals.get('SQ_ACTIVE_INST_VALU', 0) / vals['SQ_WAVE_CYCLES'] * 100:.1f} %.")
    if os.path.isdir(kt_folder):
        for r in _csv(_find(kt_folder, "kernel_stats.csv")):
            if "prefill_kernel" in r["Name"]:
                us = float(r["AverageNs"]) / 1e3
                lines.append(f"Clock implied by the kernel trace's {us:.2f} us average: "
                             f"{cycles / us / 1e3:.2f} GHz.")
    lines += ["", "Command:", "", f"    {PROFILE_COMMANDS['pmc_prefill_c5']}"]
    with open(os.path.join(dst, "prefill_c5_counters.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    log("wrote prefill_c5_counters.md")


def _algorithmic_decode_bytes(workload, fp8):
    """Algorithmic bytes of one decode call of a workload (its structure only:
    no value tensors are drawn)."""
    from workloads import make_config_case
    case = make_config_case(workload, structure_only=True)
    S = case.num_decode_seqs
    return decode_bytes(case.layout, S, case.num_q_heads, case.num_kv_heads, case.head_dim, 2,
                        unique_blocks=workload == "c4_grpo_cow", kv_bytes=1 if fp8 else None)


def _summarize_traffic(src, dst, key, calib):
    """FETCH_SIZE / WRITE_SIZE per decode call of one workload, scaled by the
    plain-copy calibration, into profiles/<stem>.{json,md}."""
    f_tag, w_tag = _counter_tags(key)
    if not all(os.path.isdir(os.path.join(src, t)) for t in (f_tag, w_tag)):
        return
    args, desc, filters = COUNTER_RUNS[key]
    fetch = _counter_means(os.path.join(src, f_tag), "FETCH_SIZE")
    write = _counter_means(os.path.join(src, w_tag), "WRITE_SIZE")
    parts = [k for k in fetch if any(f in k for f in filters)]
    copy_name, f_factor, w_factor, cf, cw = calib
    per_call_read = sum(fetch[k][1] for k in parts) * 1024 * f_factor
    per_call_write = sum(write.get(k, (0, 0.0))[1] for k in parts) * 1024 * w_factor
    algo = _algorithmic_decode_bytes(*key)
    stem = COUNTER_SETS[key]
    need = [f_tag, w_tag, "pmc_fetch_copy", "pmc_write_copy"]
    summary = {
        "workload": f"{key[0]} ({desc})",
        "source_hash": source_hash(_sources_for(key[0])),
        "copy_calibration": {"kernel": copy_name, "bytes_each_way": 1 << 30,
                             "fetch_size_kib": cf, "write_size_kib": cw,
                             "fetch_scale": f_factor, "write_scale": w_factor},
        "per_kernel_kib_per_dispatch": {
            _short(k): {"FETCH_SIZE": fetch[k][1], "WRITE_SIZE": write.get(k, (0, 0.0))[1],
                        "dispatches": fetch[k][0]} for k in parts},
        "hbm_read_bytes_per_call": per_call_read,
        "hbm_write_bytes_per_call": per_call_write,
        "hbm_bytes_per_call": per_call_read + per_call_write,
        "algorithmic_bytes_per_call": algo,
        "commands": {t: PROFILE_COMMANDS[t] for t in need},
    }
    with open(os.path.join(dst, stem + ".json"), "w") as f:
        json.dump(summary, f, indent=1)
    lines = [f"# HBM traffic of one decode call: {key[0]} ({desc})", "",
             "Per dispatch, averaged over the profiled steps; FETCH_SIZE and WRITE_SIZE are "
             "in KiB. Each counter ran in a pass of its own.", "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB |", "|---|---|---|"]
    for k in parts:
        lines.append(f"| `{_short(k)}` | {fetch[k][1]:.1f} | {write.get(k, (0, 0.0))[1]:.1f} |")
    lines += ["", f"Calibration: a plain 1 GiB device copy (`{_short(copy_name)}`, "
                  f"`bench.py --copy-calib`) reads as FETCH_SIZE {cf:.1f} KiB and "
                  f"WRITE_SIZE {cw:.1f} KiB, so fetch counts are scaled by "
                  f"{f_factor:.4f} and write counts by {w_factor:.4f}.", "",
              f"Traffic per call: read {per_call_read / 1e9:.4f} GB, write "
              f"{per_call_write / 1e9:.4f} GB, total {(per_call_read + per_call_write) / 1e9:.4f} GB "
              f"(algorithmic bytes: {algo / 1e9:.4f} GB, ratio "
              f"{(per_call_read + per_call_write) / algo:.3f}).", "", "Commands:", ""]
    lines += [f"    {PROFILE_COMMANDS[t]}" for t in need]
    with open(os.path.join(dst, stem + ".md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    log(f"wrote {stem}.{{json,md}}")


def summarize_profiles(src, dst):
    """Turn rocprofv3 CSV output (folders named as in PROFILE_COMMANDS) into
    the short text summaries kept under profiles/."""
    os.makedirs(dst, exist_ok=True)
    for tag, (_, title, name) in TRACES.items():
        folder = os.path.join(src, tag)
        if not os.path.isdir(folder):
            continue
        rows = _csv(_find(folder, "kernel_stats.csv"))
        lines = [f"# rocprofv3 kernel trace: {title}", "",
                 "Command (run on one MI355X; `<repo>` is the repository root):", "",
                 f"    {PROFILE_COMMANDS[tag]}", "",
                 "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
        for r in rows:
            if "pa::" not in r["Name"]:
                continue
            lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
        lines.append("")
        lines.append("Kernels not listed are torch's input generation and the cache flushes "
                     "between cold calls (outside the timed calls).")
        with open(os.path.join(dst, name), "w") as f:
            f.write("\n".join(lines) + "\n")
        log(f"wrote {name}")

    if os.path.isdir(os.path.join(src, "pmc_prefill_c5")):
        _summarize_prefill_counters(os.path.join(src, "pmc_prefill_c5"),
                                    os.path.join(src, "kt_c5"), dst)

    if not all(os.path.isdir(os.path.join(src, t)) for t in ("pmc_fetch_copy", "pmc_write_copy")):
        return
    cf = _counter_means(os.path.join(src, "pmc_fetch_copy"), "FETCH_SIZE")
    cw = _counter_means(os.path.join(src, "pmc_write_copy"), "WRITE_SIZE")
    copy_name = [k for k in cf if "copyBuffer" in k][0]
    calib = 1 << 30                                   # bench.py --copy-calib moves 1 GiB each way
    cal = (copy_name, calib / (cf[copy_name][1] * 1024), calib / (cw[copy_name][1] * 1024),
           cf[copy_name][1], cw[copy_name][1])
    for key in COUNTER_RUNS:
        _summarize_traffic(src, dst, key, cal)


# ------------------------------------------------------------ components ---

def _event_ms(fn, reps, stream):
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def run_copy_swap(args):
    """Block moves: copy-on-write copies inside the device cache, and swaps
    between the device cache and a pinned host pool."""
    import torch
    import paged_kv_cache_215_amd as pa
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    hkv, bs, d, nb = 4, 32, 256, 16384          # the full step's block shape, one layer
    n = 4096                                    # blocks moved per call
    kc = torch.randn((nb, hkv, bs, d), device=dev).to(torch.bfloat16)
    vc = torch.randn((nb, hkv, bs, d), device=dev).to(torch.bfloat16)
    g = np.random.default_rng(0)
    perm = g.permutation(nb)
    pairs = torch.from_numpy(np.stack([perm[:n], perm[n:2 * n]], 1).astype(np.int64)).to(dev)
    block_bytes = hkv * bs * d * 2 * 2          # K and V
    copy_ms = _event_ms(lambda: pa.pa_copy_blocks(kc, vc, pairs), 20, stream)
    copy_gbs = 2 * n * block_bytes / (copy_ms / 1e3) / 1e9   # read + write
    hk = torch.empty((n, hkv, bs, d), dtype=torch.bfloat16).pin_memory()
    hv = torch.empty((n, hkv, bs, d), dtype=torch.bfloat16).pin_memory()
    out_pairs = torch.from_numpy(np.stack([perm[:n], np.arange(n)], 1).astype(np.int64)).to(dev)
    in_pairs = torch.from_numpy(np.stack([np.arange(n), perm[n:2 * n]], 1).astype(np.int64)).to(dev)
    out_ms = _event_ms(lambda: pa.pa_swap_out(kc, vc, hk, hv, out_pairs), 5, stream)
    in_ms = _event_ms(lambda: pa.pa_swap_in(kc, vc, hk, hv, in_pairs), 5, stream)
    # context for the copy roofline: the runtime's own contiguous
    # device-to-device copy of the same number of bytes (read + write)
    flat_src = torch.empty(n * block_bytes // 2, dtype=torch.bfloat16, device=dev)
    flat_dst = torch.empty_like(flat_src)
    rt_ms = _event_ms(lambda: flat_dst.copy_(flat_src), 20, stream)
    rt_gbs = 2 * flat_src.numel() * 2 / (rt_ms / 1e3) / 1e9
    del flat_src, flat_dst
    moved = n * block_bytes
    res = {
        "metric": "KV block moves: copy-on-write copies (HBM GB/s) and swaps to/from pinned host "
                  "memory (GB/s), 1 MI355X",
        "value": round(copy_gbs, 1), "unit": "GB/s", "n_gpus": 1, "higher_is_better": True,
        "data": "synthetic", "dtype": "bf16",
        "config": {"component": "copy_swap", "blocks_per_call": n, "block_bytes_kv": block_bytes,
                   "num_kv_heads": hkv, "block_size": bs, "head_dim": d},
        "copy_blocks": {"avg_call_us": round(copy_ms * 1e3, 2), "achieved": round(copy_gbs, 1),
                        "roofline": {"bound": "hbm", "achieved": round(copy_gbs, 1),
                                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "frac": round(copy_gbs / HBM_PEAK_GBS, 4), "traffic": None},
                        "runtime_contiguous_copy_gbs": round(rt_gbs, 1)},
        "swap_out": {"avg_call_us": round(out_ms * 1e3, 2),
                     "achieved_gbs": round(moved / (out_ms / 1e3) / 1e9, 2)},
        "swap_in": {"avg_call_us": round(in_ms * 1e3, 2),
                    "achieved_gbs": round(moved / (in_ms / 1e3) / 1e9, 2)},
    }
    print(json.dumps(res), flush=True)


def _engine_requests(scenario):
    if scenario == "stragglers":
        # the pages' four output lengths, short prompts: little work per
        # iteration, so launch and host costs show
        return [(16, o) for o in [50, 120, 240, 1024] * 8], dict(
            num_layers=16, max_batch=4, chunk_tokens=64, num_blocks=4096, num_host_blocks=256,
            max_blocks_per_seq=128)
    rng = np.random.default_rng(5)
    prompts = np.minimum(rng.geometric(1.0 / 1500.0, size=96), 6000)
    outs = rng.choice(np.array([50, 120, 240, 1024]), size=96)
    return list(zip(prompts.tolist(), outs.tolist())), dict(
        num_layers=16, max_batch=32, chunk_tokens=512, num_blocks=16384, num_host_blocks=256,
        max_blocks_per_seq=512)


def run_engine(args):
    """Continuous batching on the GPU: the C++ driver runs the native
    scheduler's plans eagerly and with decode-only iterations replayed from a
    captured graph, over a BF16 or (--kv fp8) an FP8 cache."""
    import torch
    from paged_kv_cache_215_amd.engine import Engine
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hq, hkv, d, bs = 16, 4, 256, 16
    fp8 = args.kv == "fp8"
    result = {"metric": "continuous-batching generated tokens/s (eager vs graph replay), "
                        "1 MI355X", "unit": "tokens/s", "n_gpus": 1, "higher_is_better": True,
              "data": "synthetic", "dtype": "fp8_e4m3 kv, bf16 q" if fp8 else "bf16",
              "scenarios": {}}
    for scenario in ("stragglers", "mixed"):
        reqs, cfg = _engine_requests(scenario)
        L = cfg["num_layers"]
        g = torch.Generator(device=dev)
        g.manual_seed(0)
        B, C = cfg["max_batch"], cfg["chunk_tokens"]
        bank = {"q_dec": [torch.randn((B, hq, d), generator=g, device=dev).to(torch.bfloat16)
                          for _ in range(L)],
                "k_dec": [torch.randn((B, hkv, d), generator=g, device=dev).to(torch.bfloat16)
                          for _ in range(L)],
                "q_pre": [torch.randn((C, hq, d), generator=g, device=dev).to(torch.bfloat16)
                          for _ in range(L)],
                "k_pre": [torch.randn((C, hkv, d), generator=g, device=dev).to(torch.bfloat16)
                          for _ in range(L)]}
        bank["v_dec"], bank["v_pre"] = bank["k_dec"], bank["k_pre"]

        out = {"requests": len(reqs), "layers": L, "max_batch": B, "chunk_tokens": C,
               "generated_tokens": int(sum(o for _, o in reqs))}
        for mode in ("eager", "graph"):
            graph = mode == "graph"
            eng = Engine(reqs, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
                         device=dev, use_graph=graph, kv_fp8=fp8, **cfg)
            # inputs produced in place in the engine's buffers (once: the
            # values do not matter for timing)
            for name in ("q_dec", "k_dec", "v_dec", "q_pre", "k_pre", "v_pre"):
                for layer in range(L):
                    eng.inputs[name][layer].copy_(bank[name][layer])
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            host = 0.0
            preempted = decode_only = 0
            with torch.cuda.stream(eng.stream):
                while not eng.done():
                    h0 = time.perf_counter()
                    plan, _, _ = eng.step()
                    host += time.perf_counter() - h0
                    preempted += len(plan["preempted"])
                    decode_only += int(len(plan["prefill_seqs"]) == 0)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
            out[mode] = {"tokens_per_s": round(eng.decode_tokens / wall, 1),
                         "wall_s": round(wall, 3), "iterations": eng.iterations,
                         "ms_per_iteration": round(wall / eng.iterations * 1e3, 4),
                         "host_ms_per_iteration": round(host / eng.iterations * 1e3, 4),
                         "decode_only_iterations": decode_only, "preemptions": preempted}
            log(f"[bench] engine {scenario} {mode}: {out[mode]}")
            eng.close()
            del eng
            torch.cuda.empty_cache()
        out["graph_speedup"] = round(out["graph"]["tokens_per_s"] / out["eager"]["tokens_per_s"], 3)
        result["scenarios"][scenario] = out
    result["value"] = result["scenarios"]["mixed"]["graph"]["tokens_per_s"]
    result["config"] = {"component": "engine", "num_q_heads": hq, "num_kv_heads": hkv,
                        "head_dim": d, "block_size": bs,
                        "kv_cache": "fp8_e4m3 (per-head scales)" if fp8 else "bf16"}
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cold-calls", type=int, default=20,
                    help="one-layer workloads: extra pa_decode calls timed after a 1 GiB cache "
                         "flush each (reported under roofline.cold_cache)")
    ap.add_argument("--workload", default="c3_full_step",
                    choices=["c2_layer_decode", "c3_full_step", "c4_grpo_cow", "c5_mixed_step"])
    ap.add_argument("--component", choices=["engine", "copy_swap"], default=None,
                    help="measure a component instead of the decode step: the continuous-"
                         "batching engine, or block copies and swaps")
    ap.add_argument("--kv", choices=["bf16", "fp8"], default="bf16",
                    help="KV cache element type (fp8: E4M3 codes with per-head scales)")
    ap.add_argument("--graph-steps", type=int, default=20,
                    help="also time this many steps replayed from one captured HIP graph "
                         "(reported beside the eager line; 0 = skip)")
    ap.add_argument("--no-shared-prefix", action="store_true",
                    help="decode copy-on-write batches with plain pa_decode (every member "
                         "reads the shared prompt) instead of pa_decode_shared")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-layers", type=int, default=4)
    ap.add_argument("--copy-calib", action="store_true",
                    help="run only a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--summarize-profile", metavar="DIR", default=None,
                    help="write profiles/ summaries from rocprofv3 CSV output under DIR")
    args = ap.parse_args()
    if args.summarize_profile:
        summarize_profiles(args.summarize_profile, os.path.join(ROOT, "profiles"))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    if "RANK" in os.environ and os.environ.get("WORLD_SIZE", "1") != "1":
        print("bench.py runs on one GPU only (WORLD_SIZE > 1 given)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calib:
        copy_calibration()
        return
    if args.component == "engine":
        run_engine(args)
        return
    if args.component == "copy_swap":
        run_copy_swap(args)
        return
    run(args)


if __name__ == "__main__":
    main()
