"""Shared plumbing for the GPU parity tests: run the HIP library on a generated
case and evaluate the oracle on the same inputs copied back to the host."""

import sys

import numpy as np
import torch

import oracle
import paged_kv_cache_215_amd as pa
from workloads import to_numpy_bits

ATOL = 1e-3          # max-abs error allowed on float32 attention outputs


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_decode(case, layer=0, **kw):
    return pa.pa_decode(case.queries[layer], case.key_caches[layer], case.value_caches[layer],
                        case.block_tables, case.context_lens, case.scale,
                        case.max_context_len, **kw)


def compact_inputs(case, layer, seqs):
    """Host copies of the blocks the given sequences use, with their tables
    renumbered into the compacted pool (the oracle is invariant under block
    renumbering, which its own tests pin)."""
    bt = case.layout.block_tables
    bs = case.block_size
    used = []
    for b in seqs:
        n = int(case.layout.context_lens[b])
        used.extend(int(x) for x in bt[b, : -(-n // bs)])
    uniq = sorted(set(used))
    remap = {blk: i for i, blk in enumerate(uniq)}
    idx = torch.as_tensor(uniq if uniq else [0], dtype=torch.int64,
                          device=case.key_caches[layer].device)
    kc = to_numpy_bits(case.key_caches[layer].index_select(0, idx))
    vc = to_numpy_bits(case.value_caches[layer].index_select(0, idx))
    tables = np.full((len(seqs), bt.shape[1]), -1, dtype=np.int32)
    for i, b in enumerate(seqs):
        n = int(case.layout.context_lens[b])
        for j in range(-(-n // bs)):
            tables[i, j] = remap[int(bt[b, j])]
    lens = np.array([case.layout.context_lens[b] for b in seqs], dtype=np.int64)
    q = to_numpy_bits(case.queries[layer])[list(seqs)]
    return q, kc, vc, tables, lens


def oracle_decode(case, layer=0, seqs=None):
    seqs = list(range(case.num_decode_seqs)) if seqs is None else list(seqs)
    q, kc, vc, tables, lens = compact_inputs(case, layer, seqs)
    return oracle.decode_ref(q, kc, vc, tables, lens, case.scale)


def max_abs_err(got, want):
    got = np.asarray(got, dtype=np.float64)
    return float(np.max(np.abs(got - want))) if got.size else 0.0


def gpu_prefill(case, **kw):
    p = case.prefill
    return pa.pa_prefill_chunk(p.query, case.key_caches[0], case.value_caches[0], p.block_tables,
                               p.context_lens, p.cu_q_lens, p.max_q_len, case.scale,
                               int(max(int(x) for x in p.context_lens.cpu())), **kw)


def oracle_prefill_rows(case, seq, rows):
    """Oracle rows of prefill sequence `seq` (index among the prefill
    sequences). Row i of a chunk of L rows at context n equals a one-row chunk
    at context n - L + i + 1 (the oracle's chunking invariance, pinned by its
    own tests), so sampled rows need only the blocks that row can see."""
    p = case.prefill
    b = case.num_decode_seqs + seq
    n = int(case.layout.context_lens[b])
    L = p.q_lens[seq]
    q0 = int(np.sum(p.q_lens[:seq]))
    bs = case.block_size
    qh = to_numpy_bits(p.query)
    out = []
    for i in rows:
        visible = n - L + i + 1
        blocks = [int(x) for x in case.layout.block_tables[b, : -(-visible // bs)]]
        idx = torch.as_tensor(blocks, dtype=torch.int64, device=case.key_caches[0].device)
        kc = to_numpy_bits(case.key_caches[0].index_select(0, idx))
        vc = to_numpy_bits(case.value_caches[0].index_select(0, idx))
        table = np.arange(len(blocks), dtype=np.int32)[None, :]
        out.append(oracle.prefill_chunk_ref(qh[q0 + i:q0 + i + 1], kc, vc, table,
                                            np.array([visible]), np.array([0, 1]), case.scale)[0])
    return np.stack(out)
