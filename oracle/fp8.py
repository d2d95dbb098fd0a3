"""FP8 (E4M3) KV cache: code values, quantizer, scatter and dequantization.

TEST INFRASTRUCTURE ONLY - see ``oracle/__init__.py``.

The pages name FP8 as a throughput lever: quantizing to FP8 doubles the
effective memory bandwidth (vLLM architecture, memory and benchmarks deep
dive, "Hardware-level optimizations"; How vLLM gets real throughput on H100s,
its summary of the article's later sections). Decode reads every cached byte
once per step, so halving the bytes of K and V halves the step's traffic.
They give no format, scale or rounding; the readings taken here:

* format: E4M3 of the OCP 8-bit floating-point specification - 1 sign bit,
  4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
  subnormals m/8 * 2^-6; there are no infinities; S.1111.111 is NaN, so the
  largest finite magnitude is 1.75 * 2^8 = 448.
* scale: one float32 scale per KV head for K and one for V. A stored code is
  E4M3(x / s): x widened to float32 (exact for BF16) and divided by s in
  float32, the precision the device works in, then rounded to the nearest
  E4M3 value, ties to the even code (mantissa LSB 0). Magnitudes above 448
  (infinity included) saturate to +-448; NaN stays NaN (S.1111.111, sign
  kept); the sign of zero is kept.
* dequantized value = value(code) * s, exact in float64.

Decode and chunked prefill over an FP8 cache are the BF16 definitions applied
to the dequantized values.

The quantizer below rounds by searching the table of the 127 non-negative
finite code values for the nearest one; it shares nothing with the device's
bit-level rounding.
"""

import numpy as np

from .numerics import to_f64

E4M3_MAX = 448.0
E4M3_NAN = 0x7F  # positive NaN code; 0xFF is the negative one


def e4m3_value(code):
    """float64 value of E4M3 codes (any integer array, 0..255)."""
    c = np.asarray(code).astype(np.int64)
    if np.any((c < 0) | (c > 255)):
        raise ValueError("E4M3 codes are 8-bit")
    negative = (c & 0x80) != 0
    exponent = (c >> 3) & 0xF
    mantissa = (c & 0x7).astype(np.float64)
    magnitude = np.where(exponent == 0,
                         mantissa / 8.0 * 2.0 ** -6,
                         (1.0 + mantissa / 8.0) * np.exp2(exponent.astype(np.float64) - 7.0))
    magnitude = np.where((exponent == 15) & ((c & 0x7) == 7), np.nan, magnitude)
    return np.where(negative, -magnitude, magnitude)


# Non-negative finite codes 0x00..0x7E in code order, which is value order.
_CODES = np.arange(0x7F, dtype=np.int64)
_VALUES = e4m3_value(_CODES)


def quantize_e4m3(y):
    """E4M3 codes (uint8) of float32 values: nearest value, ties to the even
    code, saturation at 448, NaN to NaN, signed zero kept."""
    y = np.asarray(y, dtype=np.float32)
    mag = np.abs(y.astype(np.float64))
    nan = np.isnan(mag)
    mag = np.where(nan, 0.0, np.minimum(mag, E4M3_MAX))
    # below: largest table value <= mag; above: the next one (or the same at 448)
    below = np.searchsorted(_VALUES, mag, side="right") - 1
    above = np.minimum(below + 1, len(_VALUES) - 1)
    d_below = mag - _VALUES[below]
    d_above = _VALUES[above] - mag
    pick_above = (d_above < d_below) | ((d_above == d_below) & (_CODES[below] % 2 == 1))
    code = np.where(pick_above, _CODES[above], _CODES[below])
    code = np.where(nan, E4M3_NAN, code)
    sign = np.signbit(y).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def _to_f32(x):
    """Widen a stored tensor (uint16 BF16 bits or float32) to float32, exactly."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    if x.dtype == np.float32:
        return x
    raise TypeError(f"unsupported source element type {x.dtype}")


def quantize_rows(x, scale):
    """Codes of rows ``x [..., H_kv, d]`` with one float32 scale per head."""
    xf = _to_f32(x)
    s = np.asarray(scale, dtype=np.float32)
    if s.shape != (xf.shape[-2],):
        raise ValueError("one scale per KV head expected")
    y = (xf / s[:, None]).astype(np.float32)  # IEEE float32 division
    return quantize_e4m3(y)


def dequantize(codes, scale):
    """float64 values of a code cache ``[NB, H_kv, bs, d]`` with per-head scales."""
    s = np.asarray(scale, dtype=np.float32).astype(np.float64)
    return e4m3_value(codes) * s[None, :, None, None]


def reshape_and_cache_fp8_ref(key, value, key_cache, value_cache, slot_mapping,
                              k_scale, v_scale):
    """Return copies of the uint8 code caches with token ``t``'s quantized K/V
    written to slot ``slot_mapping[t]`` (slot = block * bs + offset, < 0
    skips); every other byte keeps its prior value."""
    kq = quantize_rows(key, k_scale)
    vq = quantize_rows(value, v_scale)
    kc = np.array(key_cache, dtype=np.uint8, copy=True)
    vc = np.array(value_cache, dtype=np.uint8, copy=True)
    block_size = kc.shape[2]
    slots = np.asarray(slot_mapping).astype(np.int64)
    for t in range(kq.shape[0]):
        slot = int(slots[t])
        if slot < 0:
            continue
        block, offset = divmod(slot, block_size)
        kc[block, :, offset, :] = kq[t]
        vc[block, :, offset, :] = vq[t]
    return kc, vc


class _DequantizedView:
    """The float64 values ``dequantize(codes, scale)`` of a code cache,
    computed only for the rows an index selects: ``view[blocks, head, rows,
    cols]`` with an integer head, as the sequence gather of the decode
    oracle indexes. Same values as dequantizing the whole cache first,
    without holding a float64 copy of it (eight times the code bytes)."""

    def __init__(self, codes, scale):
        self.codes = codes
        self.scale = np.asarray(scale, dtype=np.float32).astype(np.float64)
        self.shape = codes.shape

    def __getitem__(self, index):
        blocks, head, rows, cols = index
        return e4m3_value(self.codes[blocks, head, rows, cols]) * self.scale[head]


def decode_fp8_ref(query, key_codes, value_codes, k_scale, v_scale, block_tables,
                   context_lens, scale):
    """Decode attention over an FP8 cache: the attention of ``decode_ref`` on
    the dequantized K and V (float64 output)."""
    from .paged_ref import decode_ref

    return decode_ref(to_f64(query), _DequantizedView(key_codes, k_scale),
                      _DequantizedView(value_codes, v_scale), block_tables, context_lens, scale)


def prefill_chunk_fp8_ref(query, key_codes, value_codes, k_scale, v_scale, block_tables,
                          context_lens, cu_q_lens, scale):
    """Causal chunk attention over an FP8 cache: the attention of
    ``prefill_chunk_ref`` on the dequantized K and V (float64 output). The
    pages name FP8 caches and chunked prefill side by side as levers of the
    same serving step (vLLM architecture, memory and benchmarks deep dive,
    "Hardware-level optimizations"); quantizing changes the values K and V
    hold, not what the chunk attends to."""
    from .paged_ref import prefill_chunk_ref

    return prefill_chunk_ref(to_f64(query), _DequantizedView(key_codes, k_scale),
                             _DequantizedView(value_codes, v_scale), block_tables, context_lens,
                             cu_q_lens, scale)
