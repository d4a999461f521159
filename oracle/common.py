"""Building blocks of the oracle: per-head RMS normalisation, rotary embedding,
soft-capping, the default score scale, rounding to the storage type, and a
masked softmax-weighted sum.  All arithmetic is float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).
"""

import numpy as np


def round_to(x, dtype):
    """Round float64 values to the storage type ``dtype`` (float16 or float32).

    numpy converts float64 to float16/float32 with round-to-nearest-even,
    which is the reading taken for every materialised T tensor: the pages
    state no rounding mode.
    """
    return np.asarray(x, dtype=np.float64).astype(dtype)


def default_scale(scale, head_size):
    """Score multiplier.

    GroupQueryAttention page, Attributes table (``scale``); the
    DecoderMaskedMultiHeadAttention, SparseAttention and PackedAttention
    pages say the same: zero (or omission, passed here as ``None``) selects
    1/sqrt(head_size).  Any other value, negative ones included, is used as is.
    """
    if scale is None or scale == 0.0:
        return 1.0 / np.sqrt(float(head_size))
    return float(scale)


def rms_norm(x, weight, eps):
    """Per-head RMS normalisation over the last axis.

    GroupQueryAttention page, Inputs table (``q_norm_weight``,
    ``k_norm_weight``: shape ``(head_size)``, applied before rotary) and
    Attributes table (``qk_norm_epsilon``).  The pages give no formula; the
    reading is the usual root-mean-square norm with epsilon inside the root:
    ``y = x / sqrt(mean(x**2) + eps) * weight``.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def rotary(x, cos_rows, sin_rows, interleaved=False):
    """Rotary embedding of the leading ``2 * cos_rows.shape[-1]`` dims of x.

    ``x`` has shape ``(..., head_size)``; ``cos_rows``/``sin_rows`` have shape
    ``(..., r/2)`` and broadcast against ``x[..., :r/2]`` (the caller gathers
    the cache rows at each token's absolute position).  Dims at and beyond
    ``r`` pass through (partial rotary, SparseAttention page, Inputs table,
    ``cos_cache``).

    NeoX layout (SparseAttention page, Attributes table, ``rotary_interleaved``
    = 0; the only layout GroupQueryAttention implements, per its Description):
    pairs are (i, i + r/2) for i < r/2.  Interleaved layout pairs (2i, 2i+1).
    Each pair (a, b) becomes (a*cos - b*sin, b*cos + a*sin).
    """
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(cos_rows, dtype=np.float64)
    s = np.asarray(sin_rows, dtype=np.float64)
    half = c.shape[-1]
    r = 2 * half
    out = x.copy()
    if interleaved:
        a = x[..., 0:r:2]
        b = x[..., 1:r:2]
        out[..., 0:r:2] = a * c - b * s
        out[..., 1:r:2] = b * c + a * s
    else:
        a = x[..., :half]
        b = x[..., half:r]
        out[..., :half] = a * c - b * s
        out[..., half:r] = b * c + a * s
    return out


def softcap(x, cap):
    """Soft-capping of scores: ``cap * tanh(x / cap)`` for cap > 0, identity otherwise.

    GroupQueryAttention page, Attributes table (``softcap``: a positive value
    soft-caps the attention scores; 0 disables it).  The tanh form is the
    reading taken; the page names no formula.
    """
    x = np.asarray(x, dtype=np.float64)
    if cap is None or cap <= 0.0:
        return x
    return cap * np.tanh(x / cap)


def attend(scores, visible, values, sink=None):
    """Softmax-weighted sum of ``values`` over the visible keys of each row.

    ``scores``: (rows, keys) float64, already scaled, capped and biased.
    ``visible``: (rows, keys) bool; masked keys are excluded entirely.
    ``values``: (keys, head_size).
    ``sink``: None, or a float logit whose exponential joins each row's
    denominator only (GroupQueryAttention page, Inputs table ``head_sink`` and
    Attributes table ``smooth_softmax``; the reading is that the denominator
    gains exp(sink), taken with the same max shift as the scores).

    A row with no visible key produces 0 (with or without a sink).
    Returns (out, probs) where probs are the normalised weights (0 where masked).
    """
    scores = np.asarray(scores, dtype=np.float64)
    visible = np.asarray(visible, dtype=bool)
    v = np.asarray(values, dtype=np.float64)
    masked = np.where(visible, scores, -np.inf)
    m = np.max(masked, axis=-1, keepdims=True) if masked.shape[-1] else np.full(
        masked.shape[:-1] + (1,), -np.inf)
    if sink is not None:
        m = np.maximum(m, float(sink))
    any_vis = np.isfinite(m)
    m_safe = np.where(any_vis, m, 0.0)
    e = np.where(visible, np.exp(masked - m_safe), 0.0)
    den = np.sum(e, axis=-1, keepdims=True)
    if sink is not None:
        den = den + np.exp(float(sink) - m_safe)
    has_key = np.any(visible, axis=-1, keepdims=True)
    p = np.where(has_key, e / np.where(den > 0, den, 1.0), 0.0)
    return p @ v, p
