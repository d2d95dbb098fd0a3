"""Test-side helpers: build paged pools from contiguous per-sequence K/V with
explicit loops, so oracle pins do not lean on the oracle's own table walk."""

import numpy as np


def bf16_bits(x):
    """float array -> BF16 bit patterns (uint16), round to nearest even."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def random_contiguous(rng, lens, num_kv_heads, head_dim, dtype):
    """Per-sequence contiguous K and V, N(0,1), stored as float32 or BF16 bits."""
    ks, vs = [], []
    for n in lens:
        k = rng.standard_normal((n, num_kv_heads, head_dim)).astype(np.float32)
        v = rng.standard_normal((n, num_kv_heads, head_dim)).astype(np.float32)
        if dtype == "bf16":
            k, v = bf16_bits(k), bf16_bits(v)
        ks.append(k)
        vs.append(v)
    return ks, vs


def lay_out(ks, vs, block_size, rng, extra_blocks=3, fill=None, shared=None):
    """Place contiguous per-sequence K/V into a shuffled physical pool.

    Returns (key_cache, value_cache, block_tables). Slots nobody owns hold
    ``fill`` (NaN by default). ``shared`` = list of (seq, source_seq, nblocks):
    seq reuses source_seq's first nblocks physical blocks (their contents must
    be equal, which the caller guarantees).
    """
    num_kv_heads, head_dim = ks[0].shape[1], ks[0].shape[2]
    dtype = ks[0].dtype
    shared = {s: (src, nb) for s, src, nb in (shared or [])}
    need = []
    for b, k in enumerate(ks):
        nb = -(-k.shape[0] // block_size)
        need.append(nb - (shared[b][1] if b in shared else 0))
    pool = sum(need) + extra_blocks
    order = list(rng.permutation(pool))
    if fill is None:
        fill = np.uint16(0x7FC0) if dtype == np.uint16 else np.float32(np.nan)
    kc = np.full((pool, num_kv_heads, block_size, head_dim), fill, dtype=dtype)
    vc = np.full_like(kc, fill)
    max_blocks = max(1, max(-(-k.shape[0] // block_size) for k in ks))
    tables = np.full((len(ks), max_blocks), -1, dtype=np.int32)
    for b, (k, v) in enumerate(zip(ks, vs)):
        n = k.shape[0]
        first_own = 0
        if b in shared:
            src, nb = shared[b]
            tables[b, :nb] = tables[src, :nb]
            first_own = nb
        for blk in range(first_own, -(-n // block_size)):
            tables[b, blk] = order.pop(0)
        for j in range(first_own * block_size, n):
            phys = tables[b, j // block_size]
            kc[phys, :, j % block_size, :] = k[j]
            vc[phys, :, j % block_size, :] = v[j]
    return kc, vc, tables
