"""Sensitivity of the oracle pins: plant a plausible mistake in the oracle (on
the CPU, via monkeypatch) and check that at least one pin fails for it."""

import numpy as np
import pytest

import oracle
import oracle.paged_ref as pr
import test_oracle as pins
from oracle.numerics import to_f64


def _mut_decode(gqa="div", max_sub=True, use_scale=True, drop_last=False, swap_index=False,
                normalize=True):
    def decode(query, key_cache, value_cache, block_tables, context_lens, scale):
        q_all = to_f64(query)
        S, Hq, d = q_all.shape
        Hkv = key_cache.shape[1]
        G = Hq // Hkv
        bs = key_cache.shape[2]
        out = np.zeros((S, Hq, d))
        for b in range(S):
            n = int(context_lens[b]) - (1 if drop_last and context_lens[b] > 1 else 0)
            if n <= 0:
                continue
            pos = np.arange(n)
            if swap_index:
                phys = np.asarray(block_tables[b])[pos % bs]
                offs = pos // bs
            else:
                phys = np.asarray(block_tables[b])[pos // bs]
                offs = pos % bs
            for h in range(Hq):
                g = h // G if gqa == "div" else h % Hkv
                K = to_f64(key_cache[phys, g, offs])
                V = to_f64(value_cache[phys, g, offs])
                s = (scale if use_scale else 1.0) * (K @ q_all[b, h])
                m = s.max() if max_sub else 0.0
                with np.errstate(over="ignore", invalid="ignore"):
                    p = np.exp(s - m)
                    o = p @ V
                    out[b, h] = o / p.sum() if normalize else o
        return out
    return decode


DECODE_PINS = [
    pins.test_single_token_returns_its_value_exactly,
    pins.test_zero_query_gives_mean_of_values,
    pins.test_two_token_logistic_closed_form,
    pins.test_dominant_key_selects_its_value_without_overflow,
    pins.test_gqa_head_mapping_closed_form,
    pins.test_mqa_and_mha_reductions,
    pins.test_nan_in_unowned_slots_is_never_read,
    lambda: pins.test_decode_matches_dense_brute_force(4, 16, "bf16"),
]


def _some_pin_fails(fns):
    for fn in fns:
        try:
            fn()
        except (AssertionError, IndexError, ValueError, FloatingPointError):
            return True
    return False


@pytest.mark.parametrize("mutation", [
    dict(gqa="mod"), dict(max_sub=False), dict(use_scale=False), dict(drop_last=True),
    dict(swap_index=True), dict(normalize=False),
])
def test_decode_mutation_is_caught(monkeypatch, mutation):
    monkeypatch.setattr(oracle, "decode_ref", _mut_decode(**mutation))
    monkeypatch.setattr(pins.oracle, "decode_ref", _mut_decode(**mutation))
    assert _some_pin_fails(DECODE_PINS), mutation


def test_unmutated_decode_passes(monkeypatch):
    monkeypatch.setattr(pins.oracle, "decode_ref", _mut_decode())
    assert not _some_pin_fails(DECODE_PINS)


def _mut_prefill(shift):
    def prefill(query, key_cache, value_cache, block_tables, context_lens, cu_q_lens, scale):
        q_all = to_f64(query)
        total, Hq, d = q_all.shape
        Hkv = key_cache.shape[1]
        G = Hq // Hkv
        out = np.zeros((total, Hq, d))
        cu = np.asarray(cu_q_lens)
        for b in range(len(cu) - 1):
            n = int(context_lens[b])
            L = int(cu[b + 1] - cu[b])
            for g in range(Hkv):
                K = pr._gather_sequence(key_cache, block_tables[b], n, g)
                V = pr._gather_sequence(value_cache, block_tables[b], n, g)
                for i in range(L):
                    vis = min(n, max(1, n - L + i + 1 + shift))
                    for h in range(g * G, (g + 1) * G):
                        s = scale * (K[:vis] @ q_all[cu[b] + i, h])
                        p = np.exp(s - s.max())
                        out[cu[b] + i, h] = (p @ V[:vis]) / p.sum()
        return out
    return prefill


PREFILL_PINS = [
    lambda: pins.test_prefill_matches_dense_causal(35, 17),
    pins.test_prefill_without_prefix_is_standard_causal_attention,
]


@pytest.mark.parametrize("shift", [-1, 1])
def test_prefill_causal_offset_mutation_is_caught(monkeypatch, shift):
    monkeypatch.setattr(pins.oracle, "prefill_chunk_ref", _mut_prefill(shift))
    assert _some_pin_fails(PREFILL_PINS)


def test_unmutated_prefill_passes(monkeypatch):
    monkeypatch.setattr(pins.oracle, "prefill_chunk_ref", _mut_prefill(0))
    assert not _some_pin_fails(PREFILL_PINS)


def test_scatter_swapped_block_offset_is_caught(monkeypatch):
    def bad(key, value, key_cache, value_cache, slot_mapping):
        kc = np.array(key_cache, copy=True)
        vc = np.array(value_cache, copy=True)
        bs = kc.shape[2]
        for t, s in enumerate(np.asarray(slot_mapping)):
            if s < 0:
                continue
            off, blk = divmod(int(s), bs)
            if blk < kc.shape[0] and off < bs:
                kc[blk, :, off] = key[t]
                vc[blk, :, off] = value[t]
        return kc, vc
    monkeypatch.setattr(pins.oracle, "reshape_and_cache_ref", bad)
    assert _some_pin_fails([lambda: pins.test_scatter_round_trip_and_untouched_slots("bf16")])
