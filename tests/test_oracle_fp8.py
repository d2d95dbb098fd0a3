"""Pins of the FP8 (E4M3) oracle against what the format definition and the
mathematics fix: closed-form code values, exact round trips, tie and
saturation rules, torch's own E4M3 cast where its rules coincide (in range),
the rounding error bound, per-head scales, and decode on exactly representable
caches reducing to the BF16 oracle."""

import numpy as np
import pytest
import torch

from oracle import fp8
from oracle.dense_ref import dense_attention_ref
from oracle.paged_ref import decode_ref, prefill_chunk_ref
from oracle_helpers import lay_out


def _f32(x):
    return np.float32(x)


# ---- the code table ------------------------------------------------------------------------

def test_code_values_closed_forms():
    v = fp8.e4m3_value
    assert v(0x00) == 0.0 and not np.signbit(v(0x00))
    assert v(0x80) == 0.0 and np.signbit(v(0x80))
    assert v(0x01) == 2.0 ** -9            # smallest subnormal
    assert v(0x07) == 7 * 2.0 ** -9        # largest subnormal
    assert v(0x08) == 2.0 ** -6            # smallest normal
    assert v(0x38) == 1.0                  # exponent field 7 = bias
    assert v(0x3C) == 1.5
    assert v(0x7E) == 448.0                # largest finite
    assert v(0x77) == 240.0                # 1.875 * 2^7
    assert np.isnan(v(0x7F)) and np.isnan(v(0xFF))
    assert v(0xFE) == -448.0
    assert v(0x78) == 256.0                # exponent field 15 is finite apart from m = 7


def test_code_table_order_and_symmetry():
    codes = np.arange(0x7F)
    vals = fp8.e4m3_value(codes)
    assert np.all(np.diff(vals) > 0)
    assert np.array_equal(fp8.e4m3_value(codes | 0x80), -vals)
    finite = np.isfinite(fp8.e4m3_value(np.arange(256)))
    assert finite.sum() == 254


def test_code_table_matches_torch_float8_e4m3fn():
    ours = fp8.e4m3_value(np.arange(256))
    theirs = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(theirs))
    ok = ~np.isnan(ours)
    assert np.array_equal(ours[ok], theirs[ok])


# ---- the quantizer ---------------------------------------------------------------------

def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    y = fp8.e4m3_value(codes).astype(np.float32)
    assert np.array_equal(fp8.quantize_e4m3(y), codes.astype(np.uint8))


def test_ties_go_to_the_even_code_and_off_ties_to_the_nearer():
    codes = np.arange(0x7E)
    lo = fp8.e4m3_value(codes)
    hi = fp8.e4m3_value(codes + 1)
    mid = ((lo + hi) / 2).astype(np.float32)   # exact in float32 (5 significant bits)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)
    q = fp8.quantize_e4m3(mid).astype(np.int64)
    even = np.where(codes % 2 == 0, codes, codes + 1)
    assert np.array_equal(q, even)
    up = np.nextafter(mid, np.float32(np.inf))
    down = np.nextafter(mid, np.float32(0))
    assert np.array_equal(fp8.quantize_e4m3(up).astype(np.int64), codes + 1)
    assert np.array_equal(fp8.quantize_e4m3(down).astype(np.int64), codes)
    assert np.array_equal(fp8.quantize_e4m3(-mid).astype(np.int64), even | 0x80)


def test_subnormal_rounding():
    q = fp8.quantize_e4m3
    assert q(_f32(2.0 ** -10)) == 0x00                 # tie between 0 and 2^-9: even is 0
    assert q(_f32(3 * 2.0 ** -10)) == 0x02             # tie between 1 and 2 (x 2^-9): 2
    assert q(_f32(2.0 ** -11)) == 0x00
    assert q(_f32(1e-30)) == 0x00 and q(_f32(-1e-30)) == 0x80
    assert q(_f32(15 * 2.0 ** -10)) == 0x08            # tie 7/8 x 2^-6 .. 2^-6: code 8 is even


def test_saturation_nan_and_signed_zero():
    q = fp8.quantize_e4m3
    for big in (448.0, 448.5, 463.9, 464.0, 480.0, 1e4, 3.0e38, np.inf):
        assert q(_f32(big)) == 0x7E
        assert q(_f32(-big)) == 0xFE
    assert q(_f32(np.nan)) == 0x7F
    assert q(-np.abs(np.float32(np.nan))) == 0xFF
    assert q(_f32(0.0)) == 0x00 and q(_f32(-0.0)) == 0x80


def test_in_range_quantization_matches_torch_cast():
    rng = np.random.default_rng(7)
    mag = np.exp2(rng.uniform(-12, np.log2(448.0), 300_000))
    y = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    y = np.concatenate([y, rng.standard_normal(100_000).astype(np.float32)])
    theirs = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.quantize_e4m3(y), theirs)


def test_rounding_error_bound():
    # normal range: |E4M3(y) - y| <= 2^-4 |y| (half an ulp at 3 mantissa bits);
    # subnormal range: <= 2^-10 absolute
    rng = np.random.default_rng(3)
    y = (rng.standard_normal(200_000) * 40).astype(np.float32)
    y = y[np.abs(y) <= 448]
    back = fp8.e4m3_value(fp8.quantize_e4m3(y))
    err = np.abs(back - y.astype(np.float64))
    normal = np.abs(y) >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(y[normal]))
    assert np.all(err[~normal] <= 2.0 ** -10)


# ---- scatter with per-head scales --------------------------------------------------------

def test_quantize_rows_uses_each_heads_scale():
    # x = s_h * value(c) with power-of-two scales: the code is recovered exactly
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 0x7E, size=(5, 3, 16))
    scales = np.array([0.25, 2.0, 8.0], dtype=np.float32)
    x = (fp8.e4m3_value(codes) * scales[None, :, None]).astype(np.float32)
    assert np.array_equal(fp8.quantize_rows(x, scales), codes.astype(np.uint8))
    # swapping two heads' scales changes the codes
    assert not np.array_equal(fp8.quantize_rows(x, scales[[1, 0, 2]]), codes.astype(np.uint8))


def test_quantize_rows_inexact_quotient():
    # x / s = 1/3 lies between 0.3125 (0x2A) and 0.34375 (0x2B), nearer the latter
    x = np.ones((1, 1, 1), dtype=np.float32)
    assert fp8.quantize_rows(x, np.array([3.0], dtype=np.float32))[0, 0, 0] == 0x2B


def test_bf16_sources_widen_exactly():
    bits = np.array([[[0x3F80, 0xC0A0, 0x4380]]], dtype=np.uint16)  # 1.0, -5.0, 256.0
    codes = fp8.quantize_rows(bits, np.array([1.0], dtype=np.float32))
    assert list(fp8.e4m3_value(codes).ravel()) == [1.0, -5.0, 256.0]


def test_scatter_writes_only_mapped_slots():
    rng = np.random.default_rng(5)
    nb, hkv, bs, d = 4, 2, 16, 8
    kc = rng.integers(0, 256, size=(nb, hkv, bs, d), dtype=np.uint8)
    vc = rng.integers(0, 256, size=(nb, hkv, bs, d), dtype=np.uint8)
    key = rng.standard_normal((3, hkv, d)).astype(np.float32)
    val = rng.standard_normal((3, hkv, d)).astype(np.float32)
    ks = np.array([0.5, 1.0], dtype=np.float32)
    vs = np.array([1.0, 0.125], dtype=np.float32)
    slots = np.array([17, -1, 63])
    nk, nv = fp8.reshape_and_cache_fp8_ref(key, val, kc, vc, slots, ks, vs)
    changed = np.zeros((nb, bs), dtype=bool)
    changed[1, 1] = changed[3, 15] = True
    for blk in range(nb):
        for off in range(bs):
            if not changed[blk, off]:
                assert np.array_equal(nk[blk, :, off], kc[blk, :, off])
                assert np.array_equal(nv[blk, :, off], vc[blk, :, off])
    for t, (blk, off) in ((0, (1, 1)), (2, (3, 15))):
        for h in range(hkv):
            want_k = [fp8.quantize_e4m3(np.float32(x) / ks[h]) for x in key[t, h]]
            want_v = [fp8.quantize_e4m3(np.float32(x) / vs[h]) for x in val[t, h]]
            assert list(nk[blk, h, off]) == want_k
            assert list(nv[blk, h, off]) == want_v


# ---- decode over the FP8 cache -----------------------------------------------------------

def test_decode_on_representable_cache_equals_plain_decode():
    # K/V drawn as s_h * value(code): dequantization is exact, so FP8 decode
    # must equal the plain oracle on the same values
    rng = np.random.default_rng(9)
    lens, hkv, d, bs = [1, 17, 40], 2, 16, 16
    ks_h = np.array([0.5, 0.03125], dtype=np.float32)
    vs_h = np.array([2.0, 0.25], dtype=np.float32)
    kcodes = [rng.integers(0, 0x7E, size=(n, hkv, d)) | (rng.integers(0, 2, (n, hkv, d)) << 7)
              for n in lens]
    vcodes = [rng.integers(0, 0x7E, size=(n, hkv, d)) | (rng.integers(0, 2, (n, hkv, d)) << 7)
              for n in lens]
    kvals = [(fp8.e4m3_value(c) * ks_h[None, :, None]).astype(np.float32) for c in kcodes]
    vvals = [(fp8.e4m3_value(c) * vs_h[None, :, None]).astype(np.float32) for c in vcodes]
    kc, vc, bt = lay_out(kvals, vvals, bs, np.random.default_rng(1), fill=0.0)
    # quantize_rows wants heads on the second-to-last axis: [NB, bs, H_kv, d]
    kq = fp8.quantize_rows(kc.transpose(0, 2, 1, 3), ks_h).transpose(0, 2, 1, 3)
    vq = fp8.quantize_rows(vc.transpose(0, 2, 1, 3), vs_h).transpose(0, 2, 1, 3)
    q = rng.standard_normal((len(lens), 4, d)).astype(np.float32)
    got = fp8.decode_fp8_ref(q, kq, vq, ks_h, vs_h, bt, np.array(lens), 0.25)
    want = decode_ref(q, kc, vc, bt, np.array(lens), 0.25)
    assert np.array_equal(got, want)


def _representable_case(rng, lens, hkv, d, bs, ks_h, vs_h):
    """Contiguous K/V drawn as s_h * value(code) (random finite codes), laid
    into a shuffled pool; returns code caches, value caches and tables."""
    kcodes = [rng.integers(0, 0x7E, size=(n, hkv, d)) | (rng.integers(0, 2, (n, hkv, d)) << 7)
              for n in lens]
    vcodes = [rng.integers(0, 0x7E, size=(n, hkv, d)) | (rng.integers(0, 2, (n, hkv, d)) << 7)
              for n in lens]
    kvals = [(fp8.e4m3_value(c) * ks_h[None, :, None]).astype(np.float32) for c in kcodes]
    vvals = [(fp8.e4m3_value(c) * vs_h[None, :, None]).astype(np.float32) for c in vcodes]
    kc, vc, bt = lay_out(kvals, vvals, bs, np.random.default_rng(1), fill=0.0)
    kq = fp8.quantize_rows(kc.transpose(0, 2, 1, 3), ks_h).transpose(0, 2, 1, 3)
    vq = fp8.quantize_rows(vc.transpose(0, 2, 1, 3), vs_h).transpose(0, 2, 1, 3)
    return kq, vq, kc, vc, bt, kvals, vvals


def test_prefill_on_representable_cache_equals_plain_prefill():
    # exact dequantization: the FP8 chunk must equal the plain chunk oracle on
    # the same values, for chunks with and without a cached prefix
    rng = np.random.default_rng(19)
    lens, q_lens, hkv, d, bs = [40, 23, 9], [7, 23, 1], 2, 16, 16
    ks_h = np.array([0.25, 0.0625], dtype=np.float32)
    vs_h = np.array([4.0, 0.125], dtype=np.float32)
    kq, vq, kc, vc, bt, _, _ = _representable_case(rng, lens, hkv, d, bs, ks_h, vs_h)
    cu = np.concatenate([[0], np.cumsum(q_lens)])
    q = rng.standard_normal((int(cu[-1]), 4, d)).astype(np.float32)
    got = fp8.prefill_chunk_fp8_ref(q, kq, vq, ks_h, vs_h, bt, np.array(lens), cu, 0.3)
    want = prefill_chunk_ref(q, kc, vc, bt, np.array(lens), cu, 0.3)
    assert np.array_equal(got, want)


def test_prefill_fp8_matches_dense_causal_attention():
    # brute force on the contiguous dequantized K/V (no table walk): the
    # bottom-right causal chunk of each sequence
    rng = np.random.default_rng(21)
    lens, q_lens, hkv, d, bs = [37, 16], [5, 16], 2, 8, 16
    ks_h = np.array([0.5, 0.125], dtype=np.float32)
    vs_h = np.array([0.25, 2.0], dtype=np.float32)
    kq, vq, _, _, bt, kvals, vvals = _representable_case(rng, lens, hkv, d, bs, ks_h, vs_h)
    cu = np.concatenate([[0], np.cumsum(q_lens)])
    q = rng.standard_normal((int(cu[-1]), 4, d)).astype(np.float32)
    got = fp8.prefill_chunk_fp8_ref(q, kq, vq, ks_h, vs_h, bt, np.array(lens), cu, 0.35)
    for b in range(len(lens)):
        want = dense_attention_ref(q[cu[b]:cu[b + 1]], kvals[b], vvals[b], 0.35, causal=True)
        assert np.max(np.abs(got[cu[b]:cu[b + 1]] - want)) < 1e-12


def test_prefill_fp8_single_row_equals_fp8_decode():
    # a one-row chunk at the end of its context is a decode query
    rng = np.random.default_rng(23)
    lens, hkv, d, bs = [50, 1, 16], 1, 8, 16
    ks_h = np.array([0.5], dtype=np.float32)
    vs_h = np.array([0.75], dtype=np.float32)
    kq, vq, _, _, bt, _, _ = _representable_case(rng, lens, hkv, d, bs, ks_h, vs_h)
    q = rng.standard_normal((len(lens), 2, d)).astype(np.float32)
    cu = np.arange(len(lens) + 1)
    got = fp8.prefill_chunk_fp8_ref(q, kq, vq, ks_h, vs_h, bt, np.array(lens), cu, 0.5)
    want = fp8.decode_fp8_ref(q, kq, vq, ks_h, vs_h, bt, np.array(lens), 0.5)
    assert np.array_equal(got, want)


def test_dequantize_closed_form():
    codes = np.array([0x38, 0x40, 0xB8, 0x01], dtype=np.uint8).reshape(1, 2, 1, 2)
    got = fp8.dequantize(codes, np.array([3.0, 0.5], dtype=np.float32))
    assert got.ravel().tolist() == [3.0, 6.0, -0.5, 2.0 ** -10]


# ---- sensitivity: plausible mistakes planted in the oracle must fail a pin ----------------

def _ties_away(y):
    y = np.asarray(y, dtype=np.float32)
    mag = np.minimum(np.abs(y.astype(np.float64)), fp8.E4M3_MAX)
    vals = fp8._VALUES
    below = np.searchsorted(vals, mag, side="right") - 1
    above = np.minimum(below + 1, len(vals) - 1)
    pick = (vals[above] - mag) <= (mag - vals[below])
    code = np.where(pick, above, below)
    code = np.where(np.isnan(y), 0x7F, code)
    return (code | (np.signbit(y).astype(np.int64) << 7)).astype(np.uint8)


def _no_saturation(y):
    y = np.asarray(y, dtype=np.float32)
    code = fp8.__dict__["_orig_quantize"](y)
    over = np.abs(y.astype(np.float64)) > 464.0
    return np.where(over, code | 0x7F, code).astype(np.uint8)


def _truncate(y):
    y = np.asarray(y, dtype=np.float32)
    mag = np.minimum(np.abs(np.nan_to_num(y.astype(np.float64))), fp8.E4M3_MAX)
    code = np.searchsorted(fp8._VALUES, mag, side="right") - 1
    code = np.where(np.isnan(y), 0x7F, code)
    return (code | (np.signbit(y).astype(np.int64) << 7)).astype(np.uint8)


def _value_bias8(code):
    c = np.asarray(code).astype(np.int64)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -7, (1 + m / 8.0) * np.exp2(e - 8.0))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


def _quantize_rows_multiply(x, scale):
    xf = fp8._to_f32(x)
    s = np.asarray(scale, dtype=np.float32)
    return fp8.quantize_e4m3((xf * s[:, None]).astype(np.float32))


def _quantize_rows_first_head(x, scale):
    xf = fp8._to_f32(x)
    s = np.asarray(scale, dtype=np.float32)
    return fp8.quantize_e4m3((xf / s[0]).astype(np.float32))


PINS = [
    test_code_values_closed_forms,
    test_code_table_order_and_symmetry,
    test_code_table_matches_torch_float8_e4m3fn,
    test_every_finite_code_round_trips,
    test_ties_go_to_the_even_code_and_off_ties_to_the_nearer,
    test_subnormal_rounding,
    test_saturation_nan_and_signed_zero,
    test_in_range_quantization_matches_torch_cast,
    test_rounding_error_bound,
    test_quantize_rows_uses_each_heads_scale,
    test_quantize_rows_inexact_quotient,
    test_bf16_sources_widen_exactly,
    test_scatter_writes_only_mapped_slots,
    test_decode_on_representable_cache_equals_plain_decode,
    test_prefill_on_representable_cache_equals_plain_prefill,
    test_prefill_fp8_matches_dense_causal_attention,
    test_prefill_fp8_single_row_equals_fp8_decode,
    test_dequantize_closed_form,
]


def _some_pin_fails():
    for fn in PINS:
        try:
            fn()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


def _prefill_v_with_k_scale(query, key_codes, value_codes, k_scale, v_scale, block_tables,
                            context_lens, cu_q_lens, scale):
    from oracle.paged_ref import prefill_chunk_ref as plain
    return plain(query, fp8._DequantizedView(key_codes, k_scale),
                 fp8._DequantizedView(value_codes, k_scale), block_tables, context_lens,
                 cu_q_lens, scale)


def _prefill_unscaled_k(query, key_codes, value_codes, k_scale, v_scale, block_tables,
                        context_lens, cu_q_lens, scale):
    from oracle.paged_ref import prefill_chunk_ref as plain
    ones = np.ones_like(np.asarray(k_scale, dtype=np.float32))
    return plain(query, fp8._DequantizedView(key_codes, ones),
                 fp8._DequantizedView(value_codes, v_scale), block_tables, context_lens,
                 cu_q_lens, scale)


@pytest.mark.parametrize("mutation", ["ties_away", "no_saturation", "truncate", "bias8",
                                      "scale_multiplies", "one_scale_for_all_heads",
                                      "prefill_v_with_k_scale", "prefill_unscaled_k"])
def test_planted_fp8_mistake_fails_a_pin(monkeypatch, mutation):
    monkeypatch.setitem(fp8.__dict__, "_orig_quantize", fp8.quantize_e4m3)
    if mutation == "ties_away":
        monkeypatch.setattr(fp8, "quantize_e4m3", _ties_away)
    elif mutation == "no_saturation":
        monkeypatch.setattr(fp8, "quantize_e4m3", _no_saturation)
    elif mutation == "truncate":
        monkeypatch.setattr(fp8, "quantize_e4m3", _truncate)
    elif mutation == "bias8":
        monkeypatch.setattr(fp8, "e4m3_value", _value_bias8)
        monkeypatch.setattr(fp8, "_VALUES", _value_bias8(fp8._CODES))
    elif mutation == "scale_multiplies":
        monkeypatch.setattr(fp8, "quantize_rows", _quantize_rows_multiply)
    elif mutation == "prefill_v_with_k_scale":
        monkeypatch.setattr(fp8, "prefill_chunk_fp8_ref", _prefill_v_with_k_scale)
    elif mutation == "prefill_unscaled_k":
        monkeypatch.setattr(fp8, "prefill_chunk_fp8_ref", _prefill_unscaled_k)
    else:
        monkeypatch.setattr(fp8, "quantize_rows", _quantize_rows_first_head)
    assert _some_pin_fails()
