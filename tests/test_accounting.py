"""Pins of the footprint and slot accounting against the pages' printed numbers."""

import json
import os

import numpy as np

import oracle


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_kv_footprint_worked_example(golden_dir):
    g = _load(golden_dir, "kv_footprint.json")
    b = oracle.kv_bytes(g["num_layers"], g["num_kv_heads"], g["head_dim"], g["num_tokens"],
                        g["bytes_per_elem"])
    assert b == 536_870_912
    # the pages' two roundings of the same example
    assert round(b / 1e9, 2) == g["printed_rounded_value"]
    assert b / 2 ** 30 == g["printed_half_a_gigabyte_gib"]


def test_kv_footprint_per_layer_and_c3_totals():
    per_layer_token = oracle.kv_bytes(1, 4, 256, 1, 2)
    assert per_layer_token == 4096
    # 64 sequences of 8192 tokens, 16 layers: 32 GiB of cache
    assert 64 * oracle.kv_bytes(16, 4, 256, 8192, 2) == 32 * 2 ** 30


def test_figures_1_and_2_allocation(golden_dir):
    g = _load(golden_dir, "figs_1_2_allocation.json")
    lens, max_len, bs = g["request_lengths"], g["max_len"], g["block_size"]
    c = g["contiguous"]
    assert oracle.contiguous_slots(lens, max_len) == c["reserved"]
    assert sum(lens) == c["used"]
    assert oracle.contiguous_slots(lens, max_len) - sum(lens) == c["unused"]
    assert round(100 * c["unused"] / c["reserved"]) == c["wasted_percent_rounded"]
    p = g["paged"]
    assert [oracle.accounting.blocks_needed(n, bs) for n in lens] == p["blocks_per_request"]
    assert oracle.paged_slots(lens, bs) == p["reserved"]
    assert oracle.paged_slots(lens, bs) - sum(lens) == p["unused"]
    assert oracle.contiguous_slots(lens, max_len) - oracle.paged_slots(lens, bs) == p["freed_vs_contiguous"]


def test_only_last_block_is_partial_bound():
    # Waste per sequence is at most bs - 1 slots, so the unused fraction of
    # what paged allocation reserves stays below 4% once n > 24 (bs - 1).
    rng = np.random.default_rng(0)
    for bs in (16, 32):
        for n in rng.integers(24 * (bs - 1) + 1, 20000, size=200):
            assert oracle.internal_fragmentation([int(n)], bs) < 0.04
        worst = max(oracle.internal_fragmentation([n], bs) for n in range(24 * (bs - 1) + 1,
                                                                          24 * (bs - 1) + 2 * bs))
        assert worst < 0.04
    # ... and the bound is not universal: the 100-token tiny case wastes 12 of 112.
    assert abs(oracle.internal_fragmentation([100], 16) - 12 / 112) < 1e-15
