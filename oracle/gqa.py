"""Oracle for com.microsoft.GroupQueryAttention (float caches only).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).
"""

import numpy as np

from .common import attend, default_scale, rms_norm, rotary, round_to, softcap
from . import quant


def gqa(query, key, value, *, seqlens_k, total_sequence_length,
        present_key, present_value,
        past_key=None, past_value=None,
        cos_cache=None, sin_cache=None, attention_bias=None, head_sink=None,
        q_norm_weight=None, k_norm_weight=None,
        num_heads, kv_num_heads, causal=1, do_rotary=0, local_window_size=-1,
        qk_norm_epsilon=1e-6, scale=0.0, smooth_softmax=-1, softcap_value=0.0,
        sliding_window_cache=0, k_scale=None, v_scale=None, k_quant_type=0, v_quant_type=0,
        kv_cache_bit_width=0, query_rows=None, info=None, stored_key_codes=None):
    """Grouped-query attention with a BNSH key/value cache.

    Follows the GroupQueryAttention page: Description, Inputs, Outputs and
    Attributes tables.  Arguments carry the page's input names; ``present_key``
    and ``present_value`` are the present buffers' contents before the call
    (for a shared past/present buffer pass the past arrays themselves; the
    oracle works on copies).  ``softcap_value`` is the ``softcap`` attribute.

    Steps, in the page's terms:

    1. head_size H = query hidden / num_heads; kv_num_heads divides num_heads,
       group g = num_heads / kv_num_heads, and query head h reads kv head
       h // g (Inputs table shapes; the head map is the usual grouped-query
       one).
    2. Each sample's total length is ``seqlens_k[b] + 1`` (Inputs table,
       ``seqlens_k``).  With a past cache the new rows are right-aligned:
       past_b = total_b - S, and query s sits at absolute position
       p = past_b + s (Implementation variants, the right-aligned causal bound
       of the chunked-prefill and shared-append routes).  Without a past
       cache past_b = 0.
    3. If both norm weights are given, each query and key head is RMS
       normalised (Inputs table, ``q_norm_weight``/``k_norm_weight``).
    4. If ``do_rotary``, queries and the new keys are rotated at p with the
       NeoX half-split (the page implements no interleaved rotary).
    5. Present cache: rows [0, past_b) come from the past cache, rows
       [past_b, past_b + S) are the new (normed, rotated) keys and the values,
       rounded to T; other rows keep the buffer's prior contents (Outputs
       table; Implementation variants on retaining unchanged cache rows).
       Without a past the float present cache may have its own type,
       float16 or float32 (Description: the cache a call over direct Q/K/V
       generates may be stored as either, whatever T is; a past cache has
       T's type).  Its new rows are then the same keys and values rounded
       to that type instead.
    6. Attention reads keys/values rounded to T: the present cache's rows
       (when the cache has T's type), else the new rows rounded to T.  With
       ``causal`` key j is visible iff j < total_b and j <= p, and, when
       ``local_window_size`` W >= 0, j >= p - W (W keys to the left of the
       query plus the query's own position).  With ``causal`` = 0 (allowed
       only without a past cache and with W = -1) every one of the S new keys
       is visible and ``seqlens_k`` is metadata only.
    7. score = scale * q . k; then softcap; then + attention_bias[b|0, h|0, s, j].
    8. Softmax over visible keys; ``head_sink[h]`` (or 0 when
       ``smooth_softmax`` = 1 and no sink is given) adds exp(sink) to the
       denominator only.  Output is the weighted sum of values, BSH layout.

    With ``sliding_window_cache`` = 1 (Attributes table: the past and present
    buffers have a fixed capacity and the oldest tokens leave at the front;
    the attribute requires ``local_window_size`` > 0 and a capacity that is
    large enough; Implementation variants: a shift step moves the rows that
    stay to the start of the buffer, the new chunk is written after them, and
    the attention applies the window's lower bound as well as the causal one)
    steps 2 and 5 read, for cache capacity C:

    2'. The buffer holds the most recent tokens, oldest first: before the call
        rows [0, F_b) with F_b = min(total_b - S, C).  Query s still sits at
        absolute position total_b - S + s.
    5'. D_b = max(0, F_b + S - C) oldest rows are dropped: rows [D_b, F_b)
        move to [0, F_b - D_b), the new rows follow, and the buffer then holds
        fill_b = F_b - D_b + S rows; row i holds absolute position
        a_b + i with a_b = total_b - fill_b.  Keys are visible by absolute
        position (step 6).  "Enough capacity" is read as C >= W + S, so every
        key in any new query's window is still in the buffer; the attention
        bias is not supported with this attribute.

    With ``kv_cache_bit_width`` b = 8 or 4 (``k_quant_type``/``v_quant_type``
    PER_TENSOR = 1 or PER_CHANNEL = 2, scales ``k_scale``/``v_scale``) the
    caches hold codes (``oracle.quant``): attention reads code * scale, and
    the new rows are stored as codes of the transformed keys and the values
    (T = float32; the quotient by the scale is taken in float32).  If ``info``
    is a dict it receives ``k_quotient`` and ``v_quotient``, the float32
    quotients of the new rows (B, kvN, S, H), from which a caller can tell how
    close each code is to a rounding boundary.

    ``stored_key_codes`` (quantised caches only; optional) is a present_key
    buffer whose new key rows replace the codes computed here before the
    attention reads the cache.  A test passes the codes a kernel stored where
    its float32 norm/rotary arithmetic put a quotient on the other side of a
    rounding tie, so that the attention definition is evaluated on the cache
    that kernel actually attended.

    ``query_rows`` (optional iterable of s indices) restricts the attention
    output to those query rows (the cache is always updated in full); the
    output then has shape (B, len(query_rows), num_heads * H).

    Returns ``(output float64, present_key, present_value)`` (the present
    buffers in their own types).
    """
    q_in = np.asarray(query)
    k_in = np.asarray(key)
    v_in = np.asarray(value)
    dtype = q_in.dtype
    B, S, qh = q_in.shape
    N, kvN = int(num_heads), int(kv_num_heads)
    if N <= 0 or kvN <= 0 or N % kvN:
        raise ValueError("kv_num_heads must divide num_heads")
    if qh % N:
        raise ValueError("query hidden size must be a multiple of num_heads")
    H = qh // N
    g = N // kvN
    if k_in.shape != (B, S, kvN * H) or v_in.shape != (B, S, kvN * H):
        raise ValueError("key/value must be (B, S, kv_num_heads * head_size)")
    if (q_norm_weight is None) != (k_norm_weight is None):
        raise ValueError("q_norm_weight and k_norm_weight must be given together")
    if not causal and local_window_size != -1:
        raise ValueError("causal = 0 requires local_window_size = -1")
    if not causal and past_key is not None:
        raise ValueError("bidirectional attention takes no past cache")

    pk_out = np.array(present_key, copy=True)
    pv_out = np.array(present_value, copy=True)
    cap = pk_out.shape[2]
    bits = int(kv_cache_bit_width)
    if bits not in (0, 4, 8):
        raise ValueError("kv_cache_bit_width must be 0, 4 or 8")
    if bits:
        want = (np.int8, H) if bits == 8 else (np.uint8, H // 2)
        for arr in (pk_out, pv_out) + ((np.asarray(past_key), np.asarray(past_value))
                                       if past_key is not None else ()):
            if arr.dtype != want[0] or arr.shape[3] != want[1]:
                raise ValueError("quantised caches hold int8 (8 bits) or packed uint8 (4 bits, H/2 bytes per row)")
        ks = quant.channel_scales(k_scale, int(k_quant_type), kvN, H)
        vs = quant.channel_scales(v_scale, int(v_quant_type), kvN, H)
        if info is not None:
            info["k_quotient"] = np.zeros((B, kvN, S, H))
            info["v_quotient"] = np.zeros((B, kvN, S, H))
    elif int(k_quant_type) or int(v_quant_type):
        raise ValueError("quantisation types need kv_cache_bit_width 8 or 4")
    cache_dt = pk_out.dtype if not bits else None
    # float64 caches are the oracle's exact mode for its own pins (any T, with
    # or without a past; the attention reads the unrounded cache rows)
    own_cache_type = not bits and cache_dt not in (dtype, np.float64)
    if not bits:
        if cache_dt not in (np.float16, np.float32, np.float64) or pv_out.dtype != cache_dt:
            raise ValueError("float caches are float16 or float32, keys and values alike")
        if own_cache_type and past_key is not None:
            raise ValueError("a past cache has the type of query, key and value")
    total_b = np.asarray(seqlens_k, dtype=np.int64) + 1
    win = bool(sliding_window_cache)
    if past_key is not None:
        past_b = total_b - S
    else:
        past_b = np.zeros(B, dtype=np.int64)
    if win:
        if not causal or local_window_size <= 0 or past_key is None:
            raise ValueError("sliding_window_cache needs causal, local_window_size > 0 and a past cache")
        if cap < local_window_size + S:
            raise ValueError("sliding_window_cache needs capacity >= local_window_size + S")
        if attention_bias is not None:
            raise ValueError("sliding_window_cache takes no attention_bias")
        if np.any(past_b < 0):
            raise ValueError("seqlens_k inconsistent with sequence length")
        fill_prev = np.minimum(past_b, cap)                   # F_b
        drop = np.maximum(0, fill_prev + S - cap)             # D_b
        fill = fill_prev - drop + S
        first_pos = total_b - fill                            # a_b
    elif np.any(past_b < 0) or np.any(past_b + S > cap):
        raise ValueError("seqlens_k inconsistent with sequence length or cache capacity")

    sc = default_scale(scale, H)
    # only the query rows asked for are transformed (each row on its own)
    rows = np.arange(S) if query_rows is None else np.asarray(list(query_rows), dtype=np.int64)
    q = q_in.astype(np.float64).reshape(B, S, N, H)[:, rows]
    k = k_in.astype(np.float64).reshape(B, S, kvN, H)
    v = v_in.astype(np.float64).reshape(B, S, kvN, H)

    if q_norm_weight is not None:
        q = rms_norm(q, q_norm_weight, qk_norm_epsilon)
        k = rms_norm(k, k_norm_weight, qk_norm_epsilon)

    pos = past_b[:, None] + np.arange(S)[None, :]          # (B, S) absolute positions
    if do_rotary:
        if cos_cache is None or sin_cache is None:
            raise ValueError("do_rotary needs cos_cache and sin_cache")
        cos = np.asarray(cos_cache, dtype=np.float64)
        sin = np.asarray(sin_cache, dtype=np.float64)
        if cos.shape[1] * 2 != H:
            raise ValueError("cos_cache width must be head_size / 2")
        if np.max(pos) >= cos.shape[0]:
            raise ValueError("rotary position beyond the cos/sin cache")
        c = cos[pos][:, :, None, :]                          # (B, S, 1, H/2)
        s_ = sin[pos][:, :, None, :]
        q = rotary(q, c[:, rows], s_[:, rows])
        k = rotary(k, c, s_)

    # present cache (materialised in T)
    for b in range(B):
        if win:
            f0, d = int(fill_prev[b]), int(drop[b])
            keep_k = np.asarray(past_key)[b, :, d:f0, :].copy()
            keep_v = np.asarray(past_value)[b, :, d:f0, :].copy()
            pk_out[b, :, :f0 - d, :] = keep_k
            pv_out[b, :, :f0 - d, :] = keep_v
            pb = f0 - d
        else:
            pb = int(past_b[b])
            if past_key is not None and pb > 0:
                pk_out[b, :, :pb, :] = np.asarray(past_key)[b, :, :pb, :]
                pv_out[b, :, :pb, :] = np.asarray(past_value)[b, :, :pb, :]
        if bits:
            kc = quant.quantize(k[b].transpose(1, 0, 2), ks[:, None, :], bits)
            vc = quant.quantize(v[b].transpose(1, 0, 2), vs[:, None, :], bits)
            if info is not None:
                info["k_quotient"][b] = quant.quotient(k[b].transpose(1, 0, 2), ks[:, None, :])
                info["v_quotient"][b] = quant.quotient(v[b].transpose(1, 0, 2), vs[:, None, :])
            pk_out[b, :, pb:pb + S, :] = quant.store_codes(kc, bits)
            if stored_key_codes is not None:
                pk_out[b, :, pb:pb + S, :] = np.asarray(stored_key_codes)[b, :, pb:pb + S, :]
            pv_out[b, :, pb:pb + S, :] = quant.store_codes(vc, bits)
        else:
            pk_out[b, :, pb:pb + S, :] = round_to(k[b].transpose(1, 0, 2), cache_dt)
            pv_out[b, :, pb:pb + S, :] = round_to(v[b].transpose(1, 0, 2), cache_dt)
    if own_cache_type:
        # no past: the attention's keys and values are the new rows in T
        att_k = round_to(k.transpose(0, 2, 1, 3), dtype)
        att_v = round_to(v.transpose(0, 2, 1, 3), dtype)
    else:
        att_k, att_v = pk_out, pv_out

    out = np.zeros((B, len(rows), N, H), dtype=np.float64)
    if head_sink is not None:
        sinks = np.asarray(head_sink, dtype=np.float64).reshape(N)
    elif smooth_softmax == 1:
        sinks = np.zeros(N)
    else:
        sinks = None
    bias = None if attention_bias is None else np.asarray(attention_bias, dtype=np.float64)
    W = int(local_window_size)

    for b in range(B):
        n_keys = S if not causal else int(total_b[b])
        p = pos[b, rows]                                      # (R,)
        j = np.arange(n_keys)                                 # absolute key positions
        if win:
            n_keys = int(fill[b])
            j = int(first_pos[b]) + np.arange(n_keys)
        if causal:
            vis = j[None, :] <= p[:, None]
            if W >= 0:
                vis &= j[None, :] >= (p[:, None] - W)
        else:
            vis = np.ones((len(rows), n_keys), dtype=bool)
        for h in range(N):
            kh = h // g
            if bits:
                keys = quant.dequantize(quant.load_codes(pk_out[b, kh, :n_keys, :], bits), ks[kh])
                vals = quant.dequantize(quant.load_codes(pv_out[b, kh, :n_keys, :], bits), vs[kh])
            else:
                keys = att_k[b, kh, :n_keys, :].astype(np.float64)
                vals = att_v[b, kh, :n_keys, :].astype(np.float64)
            x = sc * (q[b, :, h, :] @ keys.T)
            x = softcap(x, softcap_value)
            if bias is not None:
                bb = bias[b if bias.shape[0] > 1 else 0, h if bias.shape[1] > 1 else 0]
                x = x + bb[rows][:, :n_keys]
            o, _ = attend(x, vis, vals, None if sinks is None else sinks[h])
            out[b, :, h, :] = o
    return out.reshape(B, len(rows), N * H), pk_out, pv_out
