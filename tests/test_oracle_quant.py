"""Pins of the oracle's quantised key/value caches (GroupQueryAttention page,
Attributes table: k_quant_type, v_quant_type, kv_cache_bit_width; Inputs
table: k_scale, v_scale and the int4 nibble packing of past_key/present_key).

The packing is pinned by bytes worked out by hand from the page's wording
(+8 bias, even coordinate in the low nibble); the rounding by hand-chosen
ties and clamps; the attention by caches whose quantisation is lossless, where
the quantised path must give exactly what the plain float path gives on the
same values (that path has its own brute-force and SDPA pins).  CPU only."""

import numpy as np
import pytest

import oracle
from oracle import quant


# ---------------------------------------------------------------------------
# packing and rounding
# ---------------------------------------------------------------------------
def test_int4_bytes_by_hand():
    # (low, high) codes -> byte: (low + 8) | (high + 8) << 4
    codes = np.array([[-8, 7, 0, 0, 1, -1, 7, -8, -3, 5]])
    assert quant.pack_int4(codes).tolist() == [[0xF0, 0x88, 0x79, 0x0F, 0xD5]]


def test_int4_unpack_every_byte():
    b = np.arange(256, dtype=np.uint8)[:, None]
    c = quant.unpack_int4(b)
    assert c.shape == (256, 2)
    assert np.array_equal(c[:, 0], (np.arange(256) & 15) - 8)
    assert np.array_equal(c[:, 1], (np.arange(256) >> 4) - 8)
    assert np.array_equal(quant.pack_int4(c), b)


def test_round_half_even_and_clamp():
    s = np.float32(0.25)
    x = np.array([0.625, 0.875, -0.625, -0.875, 0.125, -0.125, 0.1, 40.0, -40.0, 31.8, -32.1])
    # quotients 2.5 3.5 -2.5 -3.5 0.5 -0.5 0.4 160 -160 127.2 -128.4
    assert quant.quantize(x, s, 8).tolist() == [2, 4, -2, -4, 0, 0, 0, 127, -128, 127, -128]
    # 4 bits clamp to [-8, 7]
    assert quant.quantize(x, s, 4).tolist() == [2, 4, -2, -4, 0, 0, 0, 7, -8, 7, -8]


def test_decision_in_float32():
    """The quotient is rounded to float32 before the half-even decision: find
    a float32 pair whose exact quotient lies just above a tie while the float32
    quotient is the tie itself; the code must follow the float32 quotient."""
    i = np.arange(1, 200000, dtype=np.float64)
    s = (1.0 + i * 2.0 ** -23).astype(np.float32)
    x = (2.5 * s.astype(np.float64)).astype(np.float32)
    x = np.nextafter(x, np.float32(np.inf))
    exact = x.astype(np.float64) / s.astype(np.float64)
    f32 = (x / s).astype(np.float64)
    hit = np.nonzero((f32 == 2.5) & (exact > 2.5))[0]
    assert hit.size > 0
    j = hit[0]
    assert quant.quantize(x[j], s[j], 8) == 2          # tie -> even
    assert np.rint(exact[j]) == 3                     # a float64 decision would differ


def test_round_trip_bound():
    rng = np.random.default_rng(0)
    for bits in (8, 4):
        top = (1 << (bits - 1)) - 1
        s = rng.uniform(0.01, 0.2, 64).astype(np.float32).astype(np.float64)
        x = rng.uniform(-top, top, (500, 64)) * s
        d = quant.dequantize(quant.quantize(x, s, bits), s)
        assert np.all(np.abs(d - x) <= s / 2 * (1 + 1e-6))


def test_channel_scales_layout():
    ks = np.arange(6, dtype=np.float32) + 1
    cs = quant.channel_scales(ks, quant.PER_CHANNEL, 2, 3)
    assert cs.tolist() == [[1, 2, 3], [4, 5, 6]]        # (kv head, dim), head-major
    assert quant.channel_scales([0.5], quant.PER_TENSOR, 2, 3).tolist() == [[0.5] * 3] * 2
    with pytest.raises(ValueError):
        quant.channel_scales(ks, quant.PER_TENSOR, 2, 3)
    with pytest.raises(ValueError):
        quant.channel_scales([1.0], quant.PER_CHANNEL, 2, 3)


def test_rounding_margin():
    assert np.allclose(quant.rounding_margin([2.5, 2.0, 2.75, -1.5, -1.2]), [0, 0.5, 0.25, 0, 0.3])


# ---------------------------------------------------------------------------
# attention over quantised caches
# ---------------------------------------------------------------------------
def _pow2_scales(rng, kvN, H, per_channel):
    if per_channel:
        return (2.0 ** rng.integers(-4, 0, kvN * H)).astype(np.float32)
    return np.array([2.0 ** -3], np.float32)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("per_channel", [False, True])
@pytest.mark.parametrize("causal,window", [(1, -1), (1, 3), (0, -1)])
def test_prompt_lossless_equals_float_path(bits, per_channel, causal, window):
    """Prompt: keys and values that are exact multiples of their scales within
    the code range quantise without loss, so the output equals the float
    path's and the cache holds exactly those codes."""
    rng = np.random.default_rng(bits * 10 + per_channel * 3 + window + 7)
    B, S, N, kvN, H = 2, 6, 4, 2, 8
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    ks = _pow2_scales(rng, kvN, H, per_channel)
    vs = _pow2_scales(rng, kvN, H, per_channel)
    ksc = quant.channel_scales(ks, 2 if per_channel else 1, kvN, H)
    vsc = quant.channel_scales(vs, 2 if per_channel else 1, kvN, H)
    kc = rng.integers(lo, hi + 1, (B, S, kvN, H))
    vc = rng.integers(lo, hi + 1, (B, S, kvN, H))
    k = (kc * ksc[None, None]).astype(np.float32).reshape(B, S, kvN * H)
    v = (vc * vsc[None, None]).astype(np.float32).reshape(B, S, kvN * H)
    q = rng.standard_normal((B, S, N * H)).astype(np.float32)
    hb = H if bits == 8 else H // 2
    cdt = np.int8 if bits == 8 else np.uint8
    common = dict(seqlens_k=np.full(B, S - 1, np.int32), total_sequence_length=S,
                  num_heads=N, kv_num_heads=kvN, causal=causal, local_window_size=window)
    ref, pk, pv = oracle.gqa(q, k, v, present_key=np.zeros((B, kvN, S, H), np.float32),
                             present_value=np.zeros((B, kvN, S, H), np.float32), **common)
    got, qk, qv = oracle.gqa(q, k, v, present_key=np.zeros((B, kvN, S, hb), cdt),
                             present_value=np.zeros((B, kvN, S, hb), cdt), k_scale=ks, v_scale=vs,
                             k_quant_type=2 if per_channel else 1, v_quant_type=2 if per_channel else 1,
                             kv_cache_bit_width=bits, **common)
    assert np.array_equal(got, ref)
    assert np.array_equal(quant.load_codes(qk, bits), kc.transpose(0, 2, 1, 3))
    assert np.array_equal(quant.load_codes(qv, bits), vc.transpose(0, 2, 1, 3))


@pytest.mark.parametrize("bits", [8, 4])
def test_decode_lossless_past_and_append(bits):
    """Decode onto a shared past (int8, or packed int4): the past codes are read
    through their scales and the new row is appended as codes (lossless
    values), so the output equals the float path over the dequantised cache."""
    rng = np.random.default_rng(11)
    B, N, kvN, H, C = 3, 8, 2, 16, 12
    lo, hi = -(1 << (bits - 1)), 1 << (bits - 1)
    ks = _pow2_scales(rng, kvN, H, True)
    vs = _pow2_scales(rng, kvN, H, False)
    ksc = quant.channel_scales(ks, 2, kvN, H)
    vsc = quant.channel_scales(vs, 1, kvN, H)
    lens = np.array([4, 11, 0], np.int32)          # seqlens_k: totals 5, 12, 1
    past_c = rng.integers(lo, hi, (B, kvN, C, H))
    past_v = rng.integers(lo, hi, (B, kvN, C, H))
    nk = rng.integers(lo, hi, (B, 1, kvN, H))
    nv = rng.integers(lo, hi, (B, 1, kvN, H))
    k = (nk * ksc).astype(np.float32).reshape(B, 1, kvN * H)
    v = (nv * vsc).astype(np.float32).reshape(B, 1, kvN * H)
    q = rng.standard_normal((B, 1, N * H)).astype(np.float32)
    common = dict(seqlens_k=lens, total_sequence_length=12, num_heads=N, kv_num_heads=kvN)
    fk = (past_c * ksc[None, :, None, :]).astype(np.float32)
    fv = (past_v * vsc[None, :, None, :]).astype(np.float32)
    ref, rk, rv = oracle.gqa(q, k, v, past_key=fk, past_value=fv, present_key=fk,
                             present_value=fv, **common)
    pk, pv = quant.store_codes(past_c, bits), quant.store_codes(past_v, bits)
    got, gk, gv = oracle.gqa(q, k, v, past_key=pk, past_value=pv, present_key=pk,
                             present_value=pv, k_scale=ks, v_scale=vs, k_quant_type=2,
                             v_quant_type=1, kv_cache_bit_width=bits, **common)
    gk, gv = quant.load_codes(gk, bits), quant.load_codes(gv, bits)
    assert np.array_equal(got, ref)
    assert np.array_equal(gk * ksc[None, :, None, :], rk)
    assert np.array_equal(gv * vsc[None, :, None, :], rv)
    for b in range(B):
        assert np.array_equal(gk[b, :, lens[b]], nk[b, 0])     # appended row, as codes
        other = np.ones(C, bool)
        other[lens[b]] = False
        assert np.array_equal(gk[b][:, other], past_c[b][:, other])


def test_lossy_append_is_rounded_float_row():
    """With rotary and norm the appended key is the float path's key quantised:
    within half a scale step of it, and clamped where it leaves the range."""
    rng = np.random.default_rng(5)
    B, N, kvN, H, C = 2, 4, 2, 16, 8
    ks = np.array([0.02], np.float32)
    vs = np.array([0.015], np.float32)
    inv = 10000.0 ** (-np.arange(0, H, 2) / H)
    ang = np.arange(C)[:, None] * inv[None, :]
    cos, sin = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    qn = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    kn = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    lens = np.array([3, 6], np.int32)
    q = rng.standard_normal((B, 1, N * H)).astype(np.float32)
    k = rng.standard_normal((B, 1, kvN * H)).astype(np.float32)
    v = (3 * rng.standard_normal((B, 1, kvN * H))).astype(np.float32)   # some clamp
    pk = rng.integers(-128, 128, (B, kvN, C, H)).astype(np.int8)
    pv = rng.integers(-128, 128, (B, kvN, C, H)).astype(np.int8)
    common = dict(seqlens_k=lens, total_sequence_length=7, num_heads=N, kv_num_heads=kvN,
                  do_rotary=1, cos_cache=cos, sin_cache=sin, q_norm_weight=qn, k_norm_weight=kn)
    fk = (pk * 0.02).astype(np.float64)
    fv = (pv * np.float64(np.float32(0.015))).astype(np.float64)
    _, rk, rv = oracle.gqa(q, k, v, past_key=fk, past_value=fv, present_key=fk.copy(),
                           present_value=fv.copy(), **common)
    info = {}
    _, gk, gv = oracle.gqa(q, k, v, past_key=pk, past_value=pv, present_key=pk, present_value=pv,
                           k_scale=ks, v_scale=vs, k_quant_type=1, v_quant_type=1,
                           kv_cache_bit_width=8, info=info, **common)
    for b in range(B):
        row = lens[b]
        fk_row, fv_row = rk[b, :, row], rv[b, :, row]
        sk, sv = np.float64(ks[0]), np.float64(vs[0])
        assert np.all(np.abs(gk[b, :, row] * sk - np.clip(fk_row, -128 * sk, 127 * sk)) <= sk / 2 + 1e-6)
        assert np.all(np.abs(gv[b, :, row] * sv - np.clip(fv_row, -128 * sv, 127 * sv)) <= sv / 2 + 1e-6)
        assert np.allclose(info["k_quotient"][b, :, 0], fk_row / sk, rtol=1e-6, atol=1e-5)
    assert np.any(np.abs(v) / vs[0] > 128)    # the clamp was exercised


@pytest.mark.parametrize("bits", [8, 4])
def test_stored_key_codes_read_as_given(bits):
    """stored_key_codes: attention over a present cache whose new key codes
    are given equals attention over the cache those codes come from through
    the input path (keys that are exact multiples of the scales, with the
    chosen codes), and passing the oracle's own codes changes nothing."""
    rng = np.random.default_rng(21 + bits)
    B, S, N, kvN, H = 2, 5, 4, 2, 8
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    ks = _pow2_scales(rng, kvN, H, True)
    vs = _pow2_scales(rng, kvN, H, False)
    ksc = quant.channel_scales(ks, 2, kvN, H)
    vsc = quant.channel_scales(vs, 1, kvN, H)
    kc = rng.integers(lo + 1, hi, (B, S, kvN, H))
    vc = rng.integers(lo, hi + 1, (B, S, kvN, H))
    q = rng.standard_normal((B, S, N * H)).astype(np.float32)
    v = (vc * vsc[None, None]).astype(np.float32).reshape(B, S, kvN * H)
    hb = H if bits == 8 else H // 2
    cdt = np.int8 if bits == 8 else np.uint8
    common = dict(seqlens_k=np.full(B, S - 1, np.int32), total_sequence_length=S, num_heads=N,
                  kv_num_heads=kvN, k_scale=ks, v_scale=vs, k_quant_type=2, v_quant_type=1,
                  kv_cache_bit_width=bits)

    def run(codes, stored=None):
        k = (codes * ksc[None, None]).astype(np.float32).reshape(B, S, kvN * H)
        return oracle.gqa(q, k, v, present_key=np.zeros((B, kvN, S, hb), cdt),
                          present_value=np.zeros((B, kvN, S, hb), cdt), stored_key_codes=stored,
                          **common)

    out, pk, _ = run(kc)
    again, _, _ = run(kc, stored=pk)
    assert np.array_equal(again, out)
    moved = kc.copy()
    moved[1, 3, 0, 5] += 1                          # one code one step up
    moved[0, 0, 1, 2] -= 1                          # and one down
    want, wk, _ = run(moved)
    got, gk, _ = run(kc, stored=wk)
    assert np.array_equal(gk, wk)
    assert np.array_equal(got, want)
    assert not np.array_equal(got, out)


def test_quant_argument_errors():
    B, S, N, kvN, H = 1, 2, 2, 1, 8
    q = np.zeros((B, S, N * H), np.float32)
    k = np.zeros((B, S, kvN * H), np.float32)
    base = dict(seqlens_k=np.array([S - 1], np.int32), total_sequence_length=S,
                num_heads=N, kv_num_heads=kvN)
    c8 = np.zeros((B, kvN, S, H), np.int8)
    with pytest.raises(ValueError):   # bit width outside {4, 8}
        oracle.gqa(q, k, k, present_key=c8, present_value=c8, k_scale=[1.0], v_scale=[1.0],
                   k_quant_type=1, v_quant_type=1, kv_cache_bit_width=3, **base)
    with pytest.raises(ValueError):   # quantisation type without a bit width
        oracle.gqa(q, k, k, present_key=c8, present_value=c8, k_quant_type=1, **base)
    with pytest.raises(ValueError):   # int4 cache must be packed uint8, H/2 wide
        oracle.gqa(q, k, k, present_key=c8, present_value=c8, k_scale=[1.0], v_scale=[1.0],
                   k_quant_type=1, v_quant_type=1, kv_cache_bit_width=4, **base)
    with pytest.raises(ValueError):   # PER_CHANNEL needs kvN * H scales
        oracle.gqa(q, k, k, present_key=c8, present_value=c8, k_scale=[1.0], v_scale=[1.0],
                   k_quant_type=2, v_quant_type=1, kv_cache_bit_width=8, **base)
