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


def gpu_decode_fp8(case, layer=0, **kw):
    return pa.pa_decode_fp8(case.queries[layer], case.key_caches[layer], case.value_caches[layer],
                            case.k_scales[layer], case.v_scales[layer], case.block_tables,
                            case.context_lens, case.scale, case.max_context_len, **kw)


def compact_inputs(case, layer, seqs, key_cache=None, value_cache=None):
    """Host copies of the blocks the given sequences use, with their tables
    renumbered into the compacted pool (the oracle is invariant under block
    renumbering, which its own tests pin). Also returns the renumbering."""
    kcache = case.key_caches[layer] if key_cache is None else key_cache
    vcache = case.value_caches[layer] if value_cache is None else value_cache
    bt = case.layout.block_tables
    bs = case.block_size
    used = []
    for b in seqs:
        n = int(case.layout.context_lens[b])
        used.extend(int(x) for x in bt[b, : -(-n // bs)])
    uniq = sorted(set(used))
    remap = {blk: i for i, blk in enumerate(uniq)}
    idx = torch.as_tensor(uniq if uniq else [0], dtype=torch.int64, device=kcache.device)
    kc = to_numpy_bits(kcache.index_select(0, idx))
    vc = to_numpy_bits(vcache.index_select(0, idx))
    tables = np.full((len(seqs), bt.shape[1]), -1, dtype=np.int32)
    for i, b in enumerate(seqs):
        n = int(case.layout.context_lens[b])
        for j in range(-(-n // bs)):
            tables[i, j] = remap[int(bt[b, j])]
    lens = np.array([case.layout.context_lens[b] for b in seqs], dtype=np.int64)
    q = to_numpy_bits(case.queries[layer])[list(seqs)]
    return q, kc, vc, tables, lens, remap


def _oracle_attend(case, layer, q, kc, vc, tables, lens):
    if case.kv_fp8:
        return oracle.fp8.decode_fp8_ref(q, kc, vc, case.k_scales[layer].cpu().numpy(),
                                         case.v_scales[layer].cpu().numpy(), tables, lens,
                                         case.scale)
    return oracle.decode_ref(q, kc, vc, tables, lens, case.scale)


def oracle_decode(case, layer=0, seqs=None):
    seqs = list(range(case.num_decode_seqs)) if seqs is None else list(seqs)
    q, kc, vc, tables, lens, _ = compact_inputs(case, layer, seqs)
    return _oracle_attend(case, layer, q, kc, vc, tables, lens)


def oracle_decode_after_write(case, key_before, value_before, layer=0, seqs=None):
    """Oracle of "write the new tokens, then attend": the blocks are taken
    from copies of the caches made before the device wrote the new tokens, and
    the oracle's own scatter writes them (so no oracle input comes from the
    device path)."""
    seqs = list(range(case.num_decode_seqs)) if seqs is None else list(seqs)
    q, kc, vc, tables, lens, remap = compact_inputs(case, layer, seqs, key_before, value_before)
    bs = case.block_size
    slots = case.slot_mapping.cpu().numpy()
    local = np.array([remap[int(s) // bs] * bs + int(s) % bs if int(s) // bs in remap else -1
                      for s in slots], dtype=np.int64)
    nk, nv = to_numpy_bits(case.new_keys[layer]), to_numpy_bits(case.new_values[layer])
    if case.kv_fp8:
        kc, vc = oracle.fp8.reshape_and_cache_fp8_ref(nk, nv, kc, vc, local,
                                                      case.k_scales[layer].cpu().numpy(),
                                                      case.v_scales[layer].cpu().numpy())
    else:
        kc, vc = oracle.reshape_and_cache_ref(nk, nv, kc, vc, local)
    return _oracle_attend(case, layer, q, kc, vc, tables, lens)


def max_abs_err(got, want):
    got = np.asarray(got, dtype=np.float64)
    return float(np.max(np.abs(got - want))) if got.size else 0.0


def gpu_prefill(case, **kw):
    p = case.prefill
    return pa.pa_prefill_chunk(p.query, case.key_caches[0], case.value_caches[0], p.block_tables,
                               p.context_lens, p.cu_q_lens, p.max_q_len, case.scale,
                               int(max(int(x) for x in p.context_lens.cpu())), **kw)


def _oracle_written_blocks(case, blocks, key_before, value_before):
    """Host copies of the given physical blocks taken before the device wrote
    the case's new tokens, with the oracle's own scatter of those tokens
    applied (tokens bound for other blocks are skipped)."""
    idx = torch.as_tensor(blocks, dtype=torch.int64, device=key_before.device)
    kc = to_numpy_bits(key_before.index_select(0, idx))
    vc = to_numpy_bits(value_before.index_select(0, idx))
    if case.slot_mapping is None:
        return kc, vc
    bs = case.block_size
    where = {blk: i for i, blk in enumerate(blocks)}
    local = np.array([where[int(s) // bs] * bs + int(s) % bs if int(s) // bs in where else -1
                      for s in case.slot_mapping.cpu().numpy()], dtype=np.int64)
    if case.kv_fp8:
        return oracle.fp8.reshape_and_cache_fp8_ref(
            to_numpy_bits(case.new_keys[0]), to_numpy_bits(case.new_values[0]), kc, vc, local,
            case.k_scales[0].cpu().numpy(), case.v_scales[0].cpu().numpy())
    return oracle.reshape_and_cache_ref(to_numpy_bits(case.new_keys[0]),
                                        to_numpy_bits(case.new_values[0]), kc, vc, local)


def oracle_prefill_rows(case, seq, rows, key_before, value_before):
    """Oracle rows of prefill sequence `seq` (index among the prefill
    sequences), on the caches as they were before the device wrote the step's
    tokens plus the oracle's own write. Row i of a chunk of L rows at context
    n equals a one-row chunk at context n - L + i + 1 (the oracle's chunking
    invariance, pinned by its own tests), so sampled rows need only the blocks
    that row can see."""
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
        kc, vc = _oracle_written_blocks(case, blocks, key_before, value_before)
        table = np.arange(len(blocks), dtype=np.int32)[None, :]
        out.append(oracle.prefill_chunk_ref(qh[q0 + i:q0 + i + 1], kc, vc, table,
                                            np.array([visible]), np.array([0, 1]), case.scale)[0])
    return np.stack(out)


def oracle_prefill_all_rows(case, seq, key_before, value_before):
    """Oracle of every row of prefill sequence `seq`'s chunk (one oracle call
    over the blocks of its whole context), on the caches as they were before
    the device wrote the step's tokens plus the oracle's own write."""
    p = case.prefill
    b = case.num_decode_seqs + seq
    n = int(case.layout.context_lens[b])
    L = p.q_lens[seq]
    q0 = int(np.sum(p.q_lens[:seq]))
    bs = case.block_size
    blocks = [int(x) for x in case.layout.block_tables[b, : -(-n // bs)]]
    kc, vc = _oracle_written_blocks(case, blocks, key_before, value_before)
    table = np.arange(len(blocks), dtype=np.int32)[None, :]
    qh = to_numpy_bits(p.query)[q0:q0 + L]
    if case.kv_fp8:
        return oracle.fp8.prefill_chunk_fp8_ref(qh, kc, vc, case.k_scales[0].cpu().numpy(),
                                                case.v_scales[0].cpu().numpy(), table,
                                                np.array([n]), np.array([0, L]), case.scale)
    return oracle.prefill_chunk_ref(qh, kc, vc, table, np.array([n]), np.array([0, L]),
                                    case.scale)


def gpu_prefill_fp8(case, **kw):
    p = case.prefill
    return pa.pa_prefill_chunk_fp8(p.query, case.key_caches[0], case.value_caches[0],
                                   case.k_scales[0], case.v_scales[0], p.block_tables,
                                   p.context_lens, p.cu_q_lens, p.max_q_len, case.scale,
                                   int(max(int(x) for x in p.context_lens.cpu())), **kw)
