"""Invariants of the seeded workload generators (structure only; CPU)."""

import numpy as np
import pytest
import torch

from workloads import make_config_case, make_case, to_numpy_bits


def _check_tables(case):
    lay = case.layout
    bs = lay.block_size
    owners = {}
    for b, n in enumerate(lay.context_lens):
        nb = -(-int(n) // bs)
        row = lay.block_tables[b]
        assert np.all(row[:nb] >= 0) and np.all(row[:nb] < lay.num_blocks)
        assert np.all(row[nb:] == -1)
        for j, blk in enumerate(row[:nb]):
            owners.setdefault(int(blk), set()).add((b, j))
    return owners


def test_c1_structure():
    c = make_config_case("c1_tiny")
    assert c.layout.num_blocks == 32
    assert list(c.layout.context_lens) == [100]
    owners = _check_tables(c)
    assert len(owners) == 7                      # ceil(100/16), all distinct
    perm = np.random.default_rng(1).permutation(32)
    assert list(c.layout.block_tables[0]) == list(perm[:7])
    assert c.dtype == torch.float32 and c.scale == 1 / 8
    kc = c.key_caches[0]
    assert torch.isnan(kc).sum().item() == (32 * 16 - 100) * 64
    last = int(c.layout.block_tables[0, 6])
    assert not torch.isnan(kc[last, :, :4]).any() and torch.isnan(kc[last, :, 4:]).all()


def test_c2_structure():
    c = make_config_case("c2_layer_decode", structure_only=True)
    lens = c.layout.context_lens
    assert len(lens) == 32 and lens.min() >= 512 and lens.max() <= 8192
    total = sum(-(-int(n) // 16) for n in lens)
    assert c.layout.num_blocks == int(np.ceil(1.1 * total))
    owners = _check_tables(c)
    assert all(len(v) == 1 for v in owners.values())     # drawn without replacement


def test_c3_structure():
    c = make_config_case("c3_full_step", structure_only=True)
    assert c.layout.num_blocks == 64 * 256
    assert np.all(c.layout.context_lens == 8192)
    owners = _check_tables(c)
    assert len(owners) == 16384
    slots = c.slot_mapping.numpy()
    assert len(slots) == 64
    for b in range(64):
        assert slots[b] == int(c.layout.block_tables[b, 255]) * 32 + 31


def test_c4_structure():
    c = make_config_case("c4_grpo_cow", structure_only=True)
    lens = c.layout.context_lens
    assert len(lens) == 128 and lens.min() >= 4096 and lens.max() <= 4096 + 1024
    owners = _check_tables(c)
    bt = c.layout.block_tables
    for p in range(8):
        rows = bt[p * 16:(p + 1) * 16, :256]
        assert np.all(rows == rows[0])
    shared = [blk for blk, o in owners.items() if len(o) > 1]
    assert len(shared) == 8 * 256
    assert all(len(owners[blk]) == 16 for blk in shared)


def test_c5_structure():
    c = make_config_case("c5_mixed_step", structure_only=True)
    lens = c.layout.context_lens
    assert len(lens) == 256
    dec = lens[:255]
    assert dec.min() >= 51 and dec.max() <= 6000 + 1024
    assert lens[255] == 4096
    _check_tables(c)
    assert len(c.slot_mapping) == 255 + 512


def test_generation_is_deterministic():
    a = make_case(name="x", seed=9, context_lens=[5, 40], num_q_heads=4, num_kv_heads=2,
                  head_dim=16, block_size=16)
    b = make_case(name="x", seed=9, context_lens=[5, 40], num_q_heads=4, num_kv_heads=2,
                  head_dim=16, block_size=16)
    for x, y in zip(a.key_caches + a.queries, b.key_caches + b.queries):
        assert np.array_equal(to_numpy_bits(x), to_numpy_bits(y))


def test_shared_prefix_requires_block_boundary():
    with pytest.raises(ValueError):
        make_case(name="x", seed=1, context_lens=[20, 20], num_q_heads=2, num_kv_heads=1,
                  head_dim=16, block_size=16, shared_prefix=(2, 10), structure_only=True)
