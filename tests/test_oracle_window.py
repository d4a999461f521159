"""Pins of the oracle's sliding-window cache (GroupQueryAttention page,
Attributes table: sliding_window_cache) against its plain shared-cache path,
which the brute-force and SDPA pins cover: a token stream fed chunk by chunk
through a window buffer must give the outputs of the same stream through a
cache large enough never to evict, and the window buffer must hold the most
recent rows of that cache.  CPU only."""

import numpy as np
import pytest

import oracle


def _cos_sin(n, H):
    inv = 10000.0 ** (-np.arange(0, H, 2, dtype=np.float64) / H)
    ang = np.arange(n, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def _stream(seed, chunks, *, C, W, B=2, N=4, kvN=2, H=16, dtype=np.float64, rotary=True,
            norm=True, softcap=0.0, sink=True):
    rng = np.random.default_rng(seed)
    T = sum(chunks)
    cos, sin = _cos_sin(T + 1, H)
    cos, sin = cos.astype(dtype), sin.astype(dtype)
    big = T + 3
    full_k = np.zeros((B, kvN, big, H), dtype)
    full_v = np.zeros((B, kvN, big, H), dtype)
    win_k = rng.standard_normal((B, kvN, C, H)).astype(dtype)   # stale contents
    win_v = rng.standard_normal((B, kvN, C, H)).astype(dtype)
    qn = (1 + 0.1 * rng.standard_normal(H)).astype(dtype) if norm else None
    kn = (1 + 0.1 * rng.standard_normal(H)).astype(dtype) if norm else None
    hs = rng.standard_normal(N).astype(dtype) if sink else None
    done = 0
    for S in chunks:
        q = rng.standard_normal((B, S, N * H)).astype(dtype)
        k = rng.standard_normal((B, S, kvN * H)).astype(dtype)
        v = rng.standard_normal((B, S, kvN * H)).astype(dtype)
        total = done + S
        common = dict(seqlens_k=np.full(B, total - 1, np.int32), total_sequence_length=total,
                      cos_cache=cos if rotary else None, sin_cache=sin if rotary else None,
                      head_sink=hs, q_norm_weight=qn, k_norm_weight=kn, num_heads=N,
                      kv_num_heads=kvN, do_rotary=int(rotary), local_window_size=W,
                      softcap_value=softcap)
        ref, full_k, full_v = oracle.gqa(q, k, v, past_key=full_k, past_value=full_v,
                                         present_key=full_k, present_value=full_v, **common)
        got, win_k, win_v = oracle.gqa(q, k, v, past_key=win_k, past_value=win_v,
                                       present_key=win_k, present_value=win_v,
                                       sliding_window_cache=1, **common)
        yield S, total, ref, got, full_k, full_v, win_k, win_v
        done = total


@pytest.mark.parametrize("seed,chunks,C,W", [
    (1, [3, 4, 1, 1, 2, 4, 1, 1, 1, 3], 9, 5),
    (2, [1] * 14, 6, 5),                    # decode steps: one row dropped per step once full
    (3, [4, 4, 4, 4, 4], 8, 4),             # chunks that fill the buffer exactly
    (4, [2, 7, 1, 5], 12, 3),
])
def test_window_cache_matches_full_history(seed, chunks, C, W):
    for S, total, ref, got, fk, fv, wk, wv in _stream(seed, chunks, C=C, W=W):
        np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)
        fill = min(total, C)
        np.testing.assert_array_equal(wk[:, :, :fill], fk[:, :, total - fill:total])
        np.testing.assert_array_equal(wv[:, :, :fill], fv[:, :, total - fill:total])


def test_window_cache_f16_softcap():
    for S, total, ref, got, fk, fv, wk, wv in _stream(5, [3, 2, 5, 1, 4], C=10, W=4,
                                                      dtype=np.float16, softcap=3.0):
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
        fill = min(total, 10)
        np.testing.assert_array_equal(wk[:, :, :fill], fk[:, :, total - fill:total])


def test_window_cache_without_eviction_is_the_shared_cache():
    rng = np.random.default_rng(7)
    B, S, N, kvN, H, C = 2, 3, 4, 2, 16, 20
    q = rng.standard_normal((B, S, N * H))
    k = rng.standard_normal((B, S, kvN * H))
    v = rng.standard_normal((B, S, kvN * H))
    pk = rng.standard_normal((B, kvN, C, H))
    pv = rng.standard_normal((B, kvN, C, H))
    seq = np.array([9, 14], np.int32)          # totals 10 and 15: no eviction
    common = dict(seqlens_k=seq, total_sequence_length=15, num_heads=N, kv_num_heads=kvN,
                  local_window_size=6, past_key=pk, past_value=pv, present_key=pk,
                  present_value=pv)
    a = oracle.gqa(q, k, v, **common)
    b = oracle.gqa(q, k, v, sliding_window_cache=1, **common)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_window_cache_separate_buffers_match_the_shared_ones():
    # a stream through separate past and present window buffers (each call's
    # present becomes the next call's past) gives the shared buffer's outputs
    # and rows; present rows from fill on keep what they held
    rng = np.random.default_rng(11)
    B, N, kvN, H, C, W = 2, 4, 2, 16, 9, 5
    shared_k = rng.standard_normal((B, kvN, C, H))
    shared_v = rng.standard_normal((B, kvN, C, H))
    past_k, past_v = shared_k.copy(), shared_v.copy()
    done = 0
    for S in [3, 4, 1, 1, 2, 4, 1]:
        q = rng.standard_normal((B, S, N * H))
        k = rng.standard_normal((B, S, kvN * H))
        v = rng.standard_normal((B, S, kvN * H))
        total = done + S
        common = dict(seqlens_k=np.full(B, total - 1, np.int32), total_sequence_length=total,
                      num_heads=N, kv_num_heads=kvN, local_window_size=W, sliding_window_cache=1)
        ref, shared_k, shared_v = oracle.gqa(q, k, v, past_key=shared_k, past_value=shared_v,
                                             present_key=shared_k, present_value=shared_v, **common)
        pres_k = np.full((B, kvN, C, H), np.nan)
        pres_v = np.full((B, kvN, C, H), np.nan)
        got, pres_k, pres_v = oracle.gqa(q, k, v, past_key=past_k, past_value=past_v,
                                         present_key=pres_k, present_value=pres_v, **common)
        fill = min(total, C)
        np.testing.assert_array_equal(got, ref)
        np.testing.assert_array_equal(pres_k[:, :, :fill], shared_k[:, :, :fill])
        np.testing.assert_array_equal(pres_v[:, :, :fill], shared_v[:, :, :fill])
        assert np.isnan(pres_k[:, :, fill:]).all() and np.isnan(pres_v[:, :, fill:]).all()
        past_k, past_v = pres_k, pres_v
        done = total


@pytest.mark.parametrize("bad", [
    dict(local_window_size=-1),
    dict(local_window_size=0),
    dict(local_window_size=8),                  # capacity 10 < W + S
    dict(causal=0, local_window_size=-1),
])
def test_window_cache_rejects(bad):
    rng = np.random.default_rng(0)
    B, S, N, kvN, H, C = 1, 3, 2, 1, 8, 10
    kw = dict(seqlens_k=np.array([11], np.int32), total_sequence_length=12, num_heads=N,
              kv_num_heads=kvN, past_key=np.zeros((B, kvN, C, H)),
              past_value=np.zeros((B, kvN, C, H)), present_key=np.zeros((B, kvN, C, H)),
              present_value=np.zeros((B, kvN, C, H)), sliding_window_cache=1,
              local_window_size=2)
    kw.update(bad)
    with pytest.raises(ValueError):
        oracle.gqa(rng.standard_normal((B, S, N * H)), rng.standard_normal((B, S, kvN * H)),
                   rng.standard_normal((B, S, kvN * H)), **kw)
