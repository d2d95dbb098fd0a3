"""GPU parity of pa_prefill_chunk (MFMA path, through the C ABI) against the
fp64 CPU oracle: max-abs error <= 1e-3 on float32 outputs."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_215_amd as pa
from gpu_helpers import (ATOL, gpu_prefill, max_abs_err, oracle_prefill_all_rows,
                         oracle_prefill_rows, say)
from workloads import make_case, make_config_case, to_numpy_bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _write_chunk(case):
    """Device write of the step's tokens; returns copies of the caches taken
    before it, from which the oracle makes its own write."""
    before = (case.key_caches[0].clone(), case.value_caches[0].clone())
    pa.pa_reshape_and_cache(case.new_keys[0], case.new_values[0], case.key_caches[0],
                            case.value_caches[0], case.slot_mapping)
    return before


def _full_check(case, tag=""):
    """Oracle over every row of every chunk (small cases)."""
    say(f"[prefill] {case.name} {tag}")
    kb, vb = _write_chunk(case)
    out = gpu_prefill(case)
    torch.cuda.synchronize()
    p = case.prefill
    nd = case.num_decode_seqs
    lay = case.layout
    kc, vc = oracle.reshape_and_cache_ref(
        to_numpy_bits(case.new_keys[0]), to_numpy_bits(case.new_values[0]), to_numpy_bits(kb),
        to_numpy_bits(vb), case.slot_mapping.cpu().numpy())
    want = oracle.prefill_chunk_ref(
        to_numpy_bits(p.query), kc, vc, lay.block_tables[nd:], lay.context_lens[nd:],
        p.cu_q_lens.cpu().numpy(), case.scale)
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    err = max_abs_err(got, want)
    say(f"    max-abs err {err:.3e}")
    assert err <= ATOL
    return out


@pytest.mark.parametrize("head_dim", [64, 128, 256])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("block_size", [16, 32])
def test_shapes(head_dim, group, block_size):
    # unaligned prefix and chunk lengths, several row tiles and key tiles
    case = make_case(name=f"pf_d{head_dim}_g{group}_bs{block_size}", seed=head_dim * group,
                     context_lens=[], num_q_heads=2 * group, num_kv_heads=2, head_dim=head_dim,
                     block_size=block_size, device=DEV, prefill_chunks=[(45, 37)])
    _full_check(case)


@pytest.mark.parametrize("prefix,q_len", [(0, 1), (0, 16), (0, 70), (1, 1), (31, 33),
                                          (100, 64), (300, 5), (700, 130)])
def test_edges(prefix, q_len):
    case = make_case(name=f"pf_edge_{prefix}_{q_len}", seed=prefix + q_len, context_lens=[],
                     num_q_heads=16, num_kv_heads=4, head_dim=256, block_size=16, device=DEV,
                     prefill_chunks=[(prefix, q_len)])
    _full_check(case)


def test_several_sequences_in_one_call():
    case = make_case(name="pf_multi", seed=77, context_lens=[], num_q_heads=16, num_kv_heads=4,
                     head_dim=256, block_size=16, device=DEV,
                     prefill_chunks=[(50, 20), (0, 48), (400, 100), (17, 1)])
    _full_check(case)


def test_single_row_matches_decode():
    case = make_case(name="pf_vs_decode", seed=78, context_lens=[], num_q_heads=16,
                     num_kv_heads=4, head_dim=256, block_size=16, device=DEV,
                     prefill_chunks=[(500, 1)])
    out = _full_check(case)
    p = case.prefill
    dec = pa.pa_decode(p.query, case.key_caches[0], case.value_caches[0], p.block_tables,
                       p.context_lens, case.scale, 501)
    torch.cuda.synchronize()
    assert float((dec - out).abs().max()) < 2e-3   # BF16-rounded weights vs fp32 weights


@pytest.mark.parametrize("prefix", [3584, 3590])
def test_c5_chunk_all_rows(prefix):
    # the mixed step's 512-row chunk on its 3584-token prefix (and an unaligned
    # prefix), after the step's 767-token scatter; every row against the oracle
    if prefix == 3584:
        case = make_config_case("c5_mixed_step", device=DEV)
    else:
        case = make_case(name="c5_unaligned", seed=55, context_lens=[100, 2000], num_q_heads=16,
                         num_kv_heads=4, head_dim=256, block_size=16, device=DEV,
                         write_new_token=True, prefill_chunks=[(prefix, 512)])
    kb, vb = _write_chunk(case)
    out = gpu_prefill(case)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    want = oracle_prefill_all_rows(case, 0, kb, vb)
    assert want.shape == got.shape
    err = max_abs_err(got, want)
    say(f"[prefill] c5 prefix {prefix}: all {got.shape[0]} rows, max-abs err {err:.3e}")
    assert err <= ATOL


def test_run_to_run_bit_identical():
    case = make_config_case("c5_mixed_step", device=DEV)
    _write_chunk(case)
    a = gpu_prefill(case)
    b = gpu_prefill(case)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_workspace_query():
    assert pa.pa_prefill_chunk_workspace_size(1, 512, 512, 16, 4, 256, 16, 4096) > 0
    assert pa.pa_prefill_chunk_workspace_size(1, 37, 37, 4, 2, 64, 16, 82) == 0


def test_long_prefix_spans_several_splits():
    # a 30000-token prefix (1875 blocks of 16, more than one split stages):
    # sampled rows of a 300-row chunk against the oracle
    case = make_case(name="pf_long_prefix", seed=91, context_lens=[], num_q_heads=16,
                     num_kv_heads=4, head_dim=256, block_size=16, device=DEV,
                     prefill_chunks=[(30000, 300)])
    kb, vb = _write_chunk(case)
    out = gpu_prefill(case)
    torch.cuda.synchronize()
    rows = [0, 1, 150, 298, 299]
    err = max_abs_err(out.cpu().numpy()[rows], oracle_prefill_rows(case, 0, rows, kb, vb))
    say(f"[prefill] 30000-token prefix: sampled max-abs err {err:.3e}")
    assert np.all(np.isfinite(out.cpu().numpy())) and err <= ATOL


@pytest.mark.parametrize("scale", [-0.0625, 0.0, 0.3])
@pytest.mark.parametrize("group,head_dim", [(4, 256), (2, 128)])
def test_scale_sign_and_zero(scale, group, head_dim):
    # the kernel scales scores inside the exponent by |scale| and flips the
    # query's sign for a negative scale; a zero scale gives uniform weights
    case = make_case(name=f"pf_scale_{scale}_g{group}_d{head_dim}", seed=61, context_lens=[],
                     num_q_heads=4 * group, num_kv_heads=4, head_dim=head_dim, block_size=16,
                     device=DEV, prefill_chunks=[(90, 70)])
    case.scale = scale
    _full_check(case, tag=f"scale {scale}")


@pytest.mark.parametrize("seed", range(6))
def test_random_shapes_sweep(seed):
    # seeded draws of group, head size, block size and one to four chunks with
    # prefixes in [0, 600] and lengths in [1, 200] (prefix 0 and length 1
    # included), block tables a random permutation of the pool; every row of
    # every chunk against the oracle
    rng = np.random.default_rng(1000 + seed)
    group = int(rng.choice([1, 2, 4, 8]))
    head_dim = int(rng.choice([64, 128, 256]))
    block_size = int(rng.choice([16, 32]))
    n = int(rng.integers(1, 5))
    chunks = [(int(rng.choice([0, rng.integers(1, 601)])), int(rng.choice([1, rng.integers(2, 201)])))
              for _ in range(n)]
    hkv = int(rng.choice([1, 2, 4]))
    case = make_case(name=f"pf_sweep{seed}", seed=2000 + seed, context_lens=[],
                     num_q_heads=group * hkv, num_kv_heads=hkv, head_dim=head_dim,
                     block_size=block_size, device=DEV, prefill_chunks=chunks)
    _full_check(case, tag=f"G {group} Hkv {hkv} d {head_dim} bs {block_size} chunks {chunks}")
