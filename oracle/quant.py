"""Quantised key/value caches of GroupQueryAttention.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

GroupQueryAttention page: Attributes table (``k_quant_type``,
``v_quant_type``: NONE, PER_TENSOR or PER_CHANNEL; ``kv_cache_bit_width``: 8
or 4) and Inputs table (``k_scale``/``v_scale``: float32; a single scale
with PER_TENSOR, ``kv_num_heads * head_size`` scales with PER_CHANNEL; int4 cache
elements are +8-biased nibbles, two per byte, the even head coordinate in the
low nibble).  The pages give no quantisation formula; the reading is the
symmetric one: a cache value is code * scale, and a new value x is stored as
code = clamp(round_half_even(x / scale), -2^(b-1), 2^(b-1) - 1).

The rounding decides an integer, so it is taken in the precision the page
fixes for the operands: x is a float32 key or value, x / scale is the float32
quotient (IEEE division, rounded to nearest), and that quotient is rounded
half to even.  Scales are expected positive and finite.
"""

import numpy as np

NONE, PER_TENSOR, PER_CHANNEL = 0, 1, 2


def channel_scales(scale, quant_type, kv_num_heads, head_size):
    """Scale of every (kv head, dim) as a (kv_num_heads, head_size) float64 array."""
    s = np.asarray(scale, dtype=np.float32).astype(np.float64).reshape(-1)
    if quant_type == PER_TENSOR:
        if s.size != 1:
            raise ValueError("PER_TENSOR takes one scale")
        return np.full((kv_num_heads, head_size), s[0])
    if quant_type == PER_CHANNEL:
        if s.size != kv_num_heads * head_size:
            raise ValueError("PER_CHANNEL takes kv_num_heads * head_size scales")
        return s.reshape(kv_num_heads, head_size)
    raise ValueError("quantised caches need PER_TENSOR or PER_CHANNEL")


def quotient(x, scale):
    """float32 quotient x / scale of x rounded to float32 (float64 array)."""
    x32 = np.asarray(x, np.float64).astype(np.float32)
    s32 = np.asarray(scale, np.float64).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        return (x32 / s32).astype(np.float64)


def quantize(x, scale, bits):
    """Codes of x for the given scale(s): float32 quotient, round half to even, clamp."""
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    t = quotient(x, scale)
    return np.clip(np.rint(t), lo, hi).astype(np.int64)


def rounding_margin(t):
    """Distance of each quotient from the nearest half-integer (a rounding
    boundary): how far a different computation of t may stray before its code
    can differ."""
    t = np.asarray(t, np.float64)
    return np.abs(t - np.floor(t) - 0.5)


def dequantize(codes, scale):
    return np.asarray(codes, np.float64) * scale


def pack_int4(codes):
    """(..., H) codes in [-8, 7] -> (..., H / 2) uint8, even coordinate low."""
    c = np.asarray(codes, np.int64) + 8
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed):
    """(..., H / 2) uint8 -> (..., H) codes."""
    b = np.asarray(packed, np.int64)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.int64)
    out[..., 0::2] = (b & 15) - 8
    out[..., 1::2] = (b >> 4) - 8
    return out


def store_codes(codes, bits):
    """Cache elements for the codes: int8 (8 bits) or packed uint8 (4 bits)."""
    return codes.astype(np.int8) if bits == 8 else pack_int4(codes)


def load_codes(cache_rows, bits):
    """Codes of cache rows (int8 or packed uint8)."""
    return np.asarray(cache_rows).astype(np.int64) if bits == 8 else unpack_int4(cache_rows)
