"""Pins of the CPU oracle against things other than itself: dense brute force
on contiguous K/V, closed forms, invariants the pages' method implies, and
exact BF16 widening. CPU only."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle_helpers import bf16_bits, lay_out, random_contiguous


def _decode_vs_dense(rng, lens, num_kv_heads, group, head_dim, block_size, dtype, scale):
    ks, vs = random_contiguous(rng, lens, num_kv_heads, head_dim, dtype)
    num_q_heads = num_kv_heads * group
    q = rng.standard_normal((len(lens), num_q_heads, head_dim)).astype(np.float32)
    if dtype == "bf16":
        q = bf16_bits(q)
    kc, vc, bt = lay_out(ks, vs, block_size, rng)
    got = oracle.decode_ref(q, kc, vc, bt, np.array(lens), scale)
    for b, n in enumerate(lens):
        want = oracle.dense_attention_ref(q[b:b + 1], ks[b], vs[b], scale)[0]
        np.testing.assert_allclose(got[b], want, rtol=1e-12, atol=1e-13)
    return got


@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("block_size", [4, 16, 32])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_matches_dense_brute_force(group, block_size, dtype):
    rng = np.random.default_rng(100 + group * 10 + block_size)
    lens = [1, block_size - 1, block_size, block_size + 1, 3 * block_size + 5]
    _decode_vs_dense(rng, lens, 2, group, 32, block_size, dtype, 1 / math.sqrt(32))


def test_single_token_returns_its_value_exactly():
    rng = np.random.default_rng(1)
    ks, vs = random_contiguous(rng, [1], 1, 16, "f32")
    kc, vc, bt = lay_out(ks, vs, 16, rng)
    q = rng.standard_normal((1, 3, 16)).astype(np.float32)
    out = oracle.decode_ref(q, kc, vc, bt, np.array([1]), 0.25)
    for h in range(3):
        assert np.array_equal(out[0, h], vs[0][0, 0].astype(np.float64))


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(2)
    n = 37
    ks, vs = random_contiguous(rng, [n], 1, 8, "f32")
    kc, vc, bt = lay_out(ks, vs, 16, rng)
    q = np.zeros((1, 2, 8), dtype=np.float32)
    out = oracle.decode_ref(q, kc, vc, bt, np.array([n]), 0.125)
    mean = vs[0][:, 0, :].astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(out[0, 0], mean, rtol=0, atol=1e-15)
    np.testing.assert_allclose(out[0, 1], mean, rtol=0, atol=1e-15)


def test_two_token_logistic_closed_form():
    # q = e0, k0 = 0, k1 = 4 e0, scale 1/2: scores 0 and 2, so the weight of
    # token 1 is e^2 / (1 + e^2).
    d = 8
    k = np.zeros((2, 1, d), dtype=np.float32)
    k[1, 0, 0] = 4.0
    v = np.zeros((2, 1, d), dtype=np.float32)
    v[0, 0, :] = 1.0
    v[1, 0, :] = -3.0
    rng = np.random.default_rng(3)
    kc, vc, bt = lay_out([k], [v], 16, rng)
    q = np.zeros((1, 1, d), dtype=np.float32)
    q[0, 0, 0] = 1.0
    out = oracle.decode_ref(q, kc, vc, bt, np.array([2]), 0.5)
    w1 = math.exp(2.0) / (1.0 + math.exp(2.0))
    want = (1.0 - w1) * 1.0 + w1 * (-3.0)
    np.testing.assert_allclose(out[0, 0], np.full(d, want), rtol=1e-15, atol=1e-15)


def test_dominant_key_selects_its_value_without_overflow():
    # One key parallel to q with a huge score: scores ~1e3 overflow exp() unless
    # the maximum is subtracted; the output must be that token's value.
    rng = np.random.default_rng(4)
    n, d = 50, 16
    ks, vs = random_contiguous(rng, [n], 1, d, "f32")
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    ks[0][17, 0, :] = q[0, 0] * np.float32(1000.0 / float(np.dot(q[0, 0], q[0, 0])))
    kc, vc, bt = lay_out(ks, vs, 16, rng)
    out = oracle.decode_ref(q, kc, vc, bt, np.array([n]), 1.0)
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out[0, 0], vs[0][17, 0].astype(np.float64), rtol=0, atol=1e-12)


def test_gqa_head_mapping_closed_form():
    # KV head 0 holds values 1.0, KV head 1 values 2.0: query heads 0,1 (group 0)
    # must give 1.0 and heads 2,3 must give 2.0, whatever the keys.
    rng = np.random.default_rng(5)
    n, d = 40, 16
    k = rng.standard_normal((n, 2, d)).astype(np.float32)
    v = np.empty((n, 2, d), dtype=np.float32)
    v[:, 0, :] = 1.0
    v[:, 1, :] = 2.0
    kc, vc, bt = lay_out([k], [v], 16, rng)
    q = rng.standard_normal((1, 4, d)).astype(np.float32)
    out = oracle.decode_ref(q, kc, vc, bt, np.array([n]), 0.25)
    np.testing.assert_allclose(out[0, :2], 1.0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(out[0, 2:], 2.0, rtol=0, atol=1e-14)


def test_mqa_and_mha_reductions():
    rng = np.random.default_rng(6)
    # MQA: one KV head for all 8 query heads; MHA: group 1.
    _decode_vs_dense(rng, [9, 33], 1, 8, 16, 16, "f32", 0.25)
    _decode_vs_dense(rng, [9, 33], 4, 1, 16, 16, "f32", 0.25)


def test_context_zero_gives_zero_row():
    rng = np.random.default_rng(7)
    ks, vs = random_contiguous(rng, [5], 1, 8, "f32")
    kc, vc, bt = lay_out(ks, vs, 16, rng)
    q = rng.standard_normal((1, 1, 8)).astype(np.float32)
    out = oracle.decode_ref(q, kc, vc, bt, np.array([0]), 1.0)
    assert np.array_equal(out, np.zeros_like(out))


def test_block_permutation_invariance_bit_identical():
    rng = np.random.default_rng(8)
    lens = [70, 5, 33]
    ks, vs = random_contiguous(rng, lens, 2, 16, "bf16")
    q = bf16_bits(rng.standard_normal((3, 4, 16)))
    kc, vc, bt = lay_out(ks, vs, 16, rng)
    base = oracle.decode_ref(q, kc, vc, bt, np.array(lens), 0.25)
    perm = rng.permutation(kc.shape[0])          # new id of old block i = perm[i]
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    moved = oracle.decode_ref(q, kc2, vc2, bt2, np.array(lens), 0.25)
    assert np.array_equal(base, moved)


def test_copy_on_write_sharing_bit_identical():
    # Sequence 1 shares sequence 0's first 2 blocks (same prompt) vs. holding a
    # private copy of them: identical results.
    rng = np.random.default_rng(9)
    prompt_k = rng.standard_normal((32, 1, 16)).astype(np.float32)
    prompt_v = rng.standard_normal((32, 1, 16)).astype(np.float32)
    tails = [rng.standard_normal((t, 1, 16)).astype(np.float32) for t in (7, 20)]
    vtails = [rng.standard_normal((t, 1, 16)).astype(np.float32) for t in (7, 20)]
    ks = [np.concatenate([prompt_k, t]) for t in tails]
    vs = [np.concatenate([prompt_v, t]) for t in vtails]
    lens = np.array([k.shape[0] for k in ks])
    q = rng.standard_normal((2, 2, 16)).astype(np.float32)
    kc_s, vc_s, bt_s = lay_out(ks, vs, 16, rng, shared=[(1, 0, 2)])
    assert np.array_equal(bt_s[0, :2], bt_s[1, :2])
    kc_p, vc_p, bt_p = lay_out(ks, vs, 16, rng)
    assert not np.array_equal(bt_p[0, :2], bt_p[1, :2])
    shared = oracle.decode_ref(q, kc_s, vc_s, bt_s, lens, 0.25)
    private = oracle.decode_ref(q, kc_p, vc_p, bt_p, lens, 0.25)
    assert np.array_equal(shared, private)


def test_nan_in_unowned_slots_is_never_read():
    rng = np.random.default_rng(10)
    lens = [19, 1, 47]
    ks, vs = random_contiguous(rng, lens, 2, 16, "bf16")
    q = bf16_bits(rng.standard_normal((3, 4, 16)))
    kc_nan, vc_nan, bt = lay_out(ks, vs, 16, np.random.default_rng(11))
    kc_zero, vc_zero, bt2 = lay_out(ks, vs, 16, np.random.default_rng(11), fill=np.uint16(0))
    assert np.array_equal(bt, bt2)
    a = oracle.decode_ref(q, kc_nan, vc_nan, bt, np.array(lens), 0.25)
    b = oracle.decode_ref(q, kc_zero, vc_zero, bt, np.array(lens), 0.25)
    assert np.all(np.isfinite(a))
    assert np.array_equal(a, b)


def test_block_size_invariance():
    rng = np.random.default_rng(12)
    lens = [100, 64, 3]
    ks, vs = random_contiguous(rng, lens, 1, 32, "bf16")
    q = bf16_bits(rng.standard_normal((3, 4, 32)))
    kc16, vc16, bt16 = lay_out(ks, vs, 16, rng)
    kc32, vc32, bt32 = lay_out(ks, vs, 32, rng)
    a = oracle.decode_ref(q, kc16, vc16, bt16, np.array(lens), 0.2)
    b = oracle.decode_ref(q, kc32, vc32, bt32, np.array(lens), 0.2)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- prefill ---

def _prefill_setup(rng, prefix, q_len, num_kv_heads=2, group=2, d=16, bs=16, dtype="f32"):
    n = prefix + q_len
    ks, vs = random_contiguous(rng, [n], num_kv_heads, d, dtype)
    kc, vc, bt = lay_out(ks, vs, bs, rng)
    q = rng.standard_normal((q_len, num_kv_heads * group, d)).astype(np.float32)
    if dtype == "bf16":
        q = bf16_bits(q)
    return ks[0], vs[0], kc, vc, bt, q, n


@pytest.mark.parametrize("prefix,q_len", [(0, 20), (35, 17), (48, 16), (3, 1)])
def test_prefill_matches_dense_causal(prefix, q_len):
    rng = np.random.default_rng(20 + prefix)
    k, v, kc, vc, bt, q, n = _prefill_setup(rng, prefix, q_len, dtype="bf16")
    got = oracle.prefill_chunk_ref(q, kc, vc, bt, np.array([n]), np.array([0, q_len]), 0.25)
    want = oracle.dense_attention_ref(q, k, v, 0.25, causal=True)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_prefill_without_prefix_is_standard_causal_attention():
    # Row i of a chunk with no prefix sees keys 0..i: the lower-triangular mask.
    rng = np.random.default_rng(30)
    k, v, kc, vc, bt, q, n = _prefill_setup(rng, 0, 12, num_kv_heads=1, group=1)
    got = oracle.prefill_chunk_ref(q, kc, vc, bt, np.array([n]), np.array([0, 12]), 0.3)
    for i in range(12):
        s = 0.3 * (k[: i + 1, 0, :].astype(np.float64) @ q[i, 0].astype(np.float64))
        w = np.exp(s - s.max())
        w /= w.sum()
        np.testing.assert_allclose(got[i, 0], w @ v[: i + 1, 0, :].astype(np.float64),
                                   rtol=1e-12, atol=1e-13)


def test_prefill_single_row_equals_decode():
    rng = np.random.default_rng(31)
    k, v, kc, vc, bt, q, n = _prefill_setup(rng, 40, 1)
    a = oracle.prefill_chunk_ref(q, kc, vc, bt, np.array([n]), np.array([0, 1]), 0.25)
    b = oracle.decode_ref(q, kc, vc, bt, np.array([n]), 0.25)
    assert np.array_equal(a, b)


def test_prefill_chunking_invariance():
    # One 24-row chunk vs the same rows as two 12-row chunks (the first at
    # context n - 12): row results are bit-identical.
    rng = np.random.default_rng(32)
    k, v, kc, vc, bt, q, n = _prefill_setup(rng, 30, 24)
    whole = oracle.prefill_chunk_ref(q, kc, vc, bt, np.array([n]), np.array([0, 24]), 0.25)
    first = oracle.prefill_chunk_ref(q[:12], kc, vc, bt, np.array([n - 12]), np.array([0, 12]), 0.25)
    second = oracle.prefill_chunk_ref(q[12:], kc, vc, bt, np.array([n]), np.array([0, 12]), 0.25)
    assert np.array_equal(whole[:12], first)
    assert np.array_equal(whole[12:], second)


def test_prefill_two_sequences_in_one_call():
    rng = np.random.default_rng(33)
    lens_pre, lens_q = [20, 5], [7, 9]
    ns = [p + q for p, q in zip(lens_pre, lens_q)]
    ks, vs = random_contiguous(rng, ns, 1, 16, "f32")
    kc, vc, bt = lay_out(ks, vs, 16, rng)
    q = rng.standard_normal((sum(lens_q), 2, 16)).astype(np.float32)
    cu = np.array([0, 7, 16])
    got = oracle.prefill_chunk_ref(q, kc, vc, bt, np.array(ns), cu, 0.25)
    for b in range(2):
        want = oracle.dense_attention_ref(q[cu[b]:cu[b + 1]], ks[b], vs[b], 0.25, causal=True)
        np.testing.assert_allclose(got[cu[b]:cu[b + 1]], want, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- scatter ---

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scatter_round_trip_and_untouched_slots(dtype):
    rng = np.random.default_rng(40)
    nb, hkv, bs, d, t = 6, 2, 16, 8, 20
    sentinel = np.uint16(0x1234) if dtype == "bf16" else np.float32(-7.25)
    kc = np.full((nb, hkv, bs, d), sentinel)
    vc = np.full_like(kc, sentinel)
    k = rng.standard_normal((t, hkv, d)).astype(np.float32)
    v = rng.standard_normal((t, hkv, d)).astype(np.float32)
    if dtype == "bf16":
        k, v = bf16_bits(k), bf16_bits(v)
    slots = rng.choice(nb * bs, size=t, replace=False).astype(np.int64)
    slots[3] = -1                                        # skipped token
    kc2, vc2 = oracle.reshape_and_cache_ref(k, v, kc, vc, slots)
    written = np.zeros((nb, bs), dtype=bool)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = s // bs, s % bs
        written[blk, off] = True
        assert np.array_equal(kc2[blk, :, off, :].view(np.uint8), k[i].view(np.uint8))
        assert np.array_equal(vc2[blk, :, off, :].view(np.uint8), v[i].view(np.uint8))
    for blk in range(nb):
        for off in range(bs):
            if not written[blk, off]:
                assert np.array_equal(kc2[blk, :, off, :], kc[blk, :, off, :])
                assert np.array_equal(vc2[blk, :, off, :], vc[blk, :, off, :])
    # The inputs are not modified.
    assert np.all(kc == sentinel)


def test_scatter_preserves_nan_payload_bits():
    kc = np.zeros((1, 1, 16, 4), dtype=np.float32)
    vc = np.zeros_like(kc)
    payload = np.array([0x7FC01234, 0xFFC00001, 0x7F800001, 0x00000001], dtype=np.uint32)
    k = payload.view(np.float32).reshape(1, 1, 4)
    kc2, _ = oracle.reshape_and_cache_ref(k, k, kc, vc, np.array([5]))
    assert np.array_equal(kc2[0, 0, 5].view(np.uint32), payload)


# ------------------------------------------------------------- numerics ---

def test_bf16_widening_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0x0001, 0x4049], dtype=np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 0.0
    assert math.copysign(1.0, got[3]) == -1.0
    assert got[4] == math.inf
    assert got[5] == 2.0 ** -133                      # smallest BF16 subnormal
    assert got[6] == 3.140625
    assert np.isnan(oracle.bf16_bits_to_f64(np.array([0x7FC0], dtype=np.uint16)))[0]


def test_bf16_widening_agrees_with_torch():
    x = torch.randn(4096, generator=torch.Generator().manual_seed(0)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.bf16_bits_to_f64(bits), x.double().numpy())
    # and the test-side rounding helper agrees with torch's round-to-nearest-even
    f = torch.randn(4096, generator=torch.Generator().manual_seed(1))
    np.testing.assert_array_equal(bf16_bits(f.numpy()),
                                  f.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
