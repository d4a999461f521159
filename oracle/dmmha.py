"""Oracle for com.microsoft.DecoderMaskedMultiHeadAttention.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).
"""

import numpy as np

from .common import attend, default_scale, round_to


def dmmha(query, key, value, *, num_heads,
          mask_index=None, attention_bias=None,
          past_key=None, past_value=None, past_sequence_length=None,
          mask_filter_value=-10000.0, scale=0.0, output_qk=0):
    """Single-token decode attention, self or cross.

    Follows the DecoderMaskedMultiHeadAttention page: Description, Inputs,
    Outputs and Attributes tables.

    * head_size H = query hidden / num_heads; one key/value head per query head.
    * Self attention (``past_key`` given; past and present are one
      capacity-sized buffer): P = ``past_sequence_length[0]`` is the live
      length before this token, shared by the whole batch (the input is a
      single value).  The token's key and value rows (``key``/``value`` of
      shape (B, 1, N*H)) are written, rounded to T, at row P of every head;
      every other row keeps its past value.  Keys 0..P are attended.
    * Cross attention (no ``past_key``): ``key``/``value`` are the whole
      encoder tensors (B, N, kv_S, H); no cache.
    * score_j = scale * q . k_j, plus ``attention_bias[b|0, h|0, 0, j]`` (self
      attention only), plus ``mask_filter_value`` where ``mask_index[b, j]``
      is zero: the mask is additive and never removes a key.
    * Plain softmax over the attended keys, then the weighted sum of values.
    * ``qk`` (cross attention with ``output_qk`` = 1) is the score row once
      the mask term is added, not yet normalised, shape (B, N, 1, kv_S).

    Returns ``(output float64 (B, 1, N*H), present_key, present_value, qk)``;
    the present arrays are None for cross attention, qk is None unless asked.
    """
    q_in = np.asarray(query)
    dtype = q_in.dtype
    B, one, qh = q_in.shape
    if one != 1:
        raise ValueError("query must hold one token")
    N = int(num_heads)
    if qh % N:
        raise ValueError("query hidden size must be a multiple of num_heads")
    H = qh // N
    sc = default_scale(scale, H)
    q = q_in.astype(np.float64).reshape(B, N, H)

    present_k = present_v = None
    if past_key is not None:
        if attention_bias is not None and np.asarray(attention_bias).shape[2] != 1:
            raise ValueError("attention_bias must be (B|1, N|1, 1, total_S)")
        P = int(np.asarray(past_sequence_length).reshape(-1)[0])
        present_k = np.array(past_key, copy=True)
        present_v = np.array(past_value, copy=True)
        if P < 0 or P >= present_k.shape[2]:
            raise ValueError("past_sequence_length outside the cache capacity")
        present_k[:, :, P, :] = round_to(np.asarray(key, dtype=np.float64).reshape(B, N, H), dtype)
        present_v[:, :, P, :] = round_to(np.asarray(value, dtype=np.float64).reshape(B, N, H), dtype)
        keys = present_k[:, :, :P + 1, :].astype(np.float64)
        vals = present_v[:, :, :P + 1, :].astype(np.float64)
        n_keys = P + 1
    else:
        if attention_bias is not None:
            raise ValueError("attention_bias is for self attention only")
        keys = np.asarray(key, dtype=np.float64)
        vals = np.asarray(value, dtype=np.float64)
        if keys.shape[:2] != (B, N) or keys.shape[3] != H:
            raise ValueError("cross-attention key must be (B, N, kv_S, H)")
        n_keys = keys.shape[2]

    bias = None if attention_bias is None else np.asarray(attention_bias, dtype=np.float64)
    mask = None if mask_index is None else np.asarray(mask_index)
    out = np.zeros((B, N, H))
    qk = np.zeros((B, N, 1, n_keys)) if (output_qk and past_key is None) else None
    vis = np.ones((1, n_keys), dtype=bool)
    for b in range(B):
        for h in range(N):
            x = sc * (keys[b, h] @ q[b, h])                  # (n_keys,)
            if bias is not None:
                x = x + bias[b if bias.shape[0] > 1 else 0, h if bias.shape[1] > 1 else 0, 0, :n_keys]
            if mask is not None:
                x = x + np.where(mask[b, :n_keys] == 0, float(mask_filter_value), 0.0)
            if qk is not None:
                qk[b, h, 0, :] = x
            o, _ = attend(x[None, :], vis, vals[b, h])
            out[b, h] = o[0]
    return out.reshape(B, 1, N * H), present_k, present_v, qk
