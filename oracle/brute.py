"""Pure-Python scalar brute force for tiny shapes.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

A second, independent formulation of the four operators, written with Python
floats and explicit loops over (batch, head, query, key, dim).  It uses none
of ``oracle.common`` so that a slip in the vectorised oracle (a wrong axis, a
dropped term, a transposed operand) shows up as a disagreement.  It is only
meant for shapes of a few elements per axis.  Cache rows are rounded to T
through numpy scalars, the only numpy use here.
"""

import math

import numpy as np


def _scale(scale, H):
    return 1.0 / math.sqrt(H) if (scale is None or scale == 0.0) else float(scale)


def _norm_head(vec, w, eps):
    ms = sum(x * x for x in vec) / len(vec)
    r = 1.0 / math.sqrt(ms + eps)
    return [vec[i] * r * float(w[i]) for i in range(len(vec))]


def _rot_head(vec, cos_row, sin_row, interleaved):
    half = len(cos_row)
    out = list(vec)
    for i in range(half):
        if interleaved:
            ia, ib = 2 * i, 2 * i + 1
        else:
            ia, ib = i, i + half
        a, b = vec[ia], vec[ib]
        c, s = float(cos_row[i]), float(sin_row[i])
        out[ia] = a * c - b * s
        out[ib] = b * c + a * s
    return out


def _softmax_sum(scores, vals, H, sink=None):
    """scores: list of (score, key index) for visible keys; vals(j) -> list."""
    if not scores and True:
        return [0.0] * H
    m = max(s for s, _ in scores)
    if sink is not None:
        m = max(m, sink)
    den = sum(math.exp(s - m) for s, _ in scores)
    if sink is not None:
        den += math.exp(sink - m)
    out = [0.0] * H
    for s, j in scores:
        p = math.exp(s - m) / den
        vj = vals(j)
        for d in range(H):
            out[d] += p * vj[d]
    return out


def _f(x):
    return float(x)


def brute_gqa(query, key, value, *, seqlens_k, present_key, present_value,
              past_key=None, past_value=None, cos_cache=None, sin_cache=None,
              attention_bias=None, head_sink=None, q_norm_weight=None,
              k_norm_weight=None, num_heads, kv_num_heads, causal=1, do_rotary=0,
              local_window_size=-1, qk_norm_epsilon=1e-6, scale=0.0,
              smooth_softmax=-1, softcap_value=0.0):
    dt = np.asarray(query).dtype
    B, S, qh = np.asarray(query).shape
    N, kvN = num_heads, kv_num_heads
    H = qh // N
    g = N // kvN
    sc = _scale(scale, H)
    pk = np.array(present_key, copy=True)
    pv = np.array(present_value, copy=True)
    out = np.zeros((B, S, N * H))
    for b in range(B):
        total = int(seqlens_k[b]) + 1
        past = total - S if past_key is not None else 0
        if past_key is not None:
            for kh in range(kvN):
                for j in range(past):
                    pk[b, kh, j] = past_key[b, kh, j]
                    pv[b, kh, j] = past_value[b, kh, j]
        # new keys / values into the cache
        for s in range(S):
            p = past + s
            for kh in range(kvN):
                kv = [_f(key[b, s, kh * H + d]) for d in range(H)]
                if q_norm_weight is not None:
                    kv = _norm_head(kv, k_norm_weight, qk_norm_epsilon)
                if do_rotary:
                    kv = _rot_head(kv, cos_cache[p], sin_cache[p], False)
                for d in range(H):
                    pk[b, kh, p, d] = dt.type(kv[d])
                    pv[b, kh, p, d] = value[b, s, kh * H + d]
        for s in range(S):
            p = past + s
            for h in range(N):
                qv = [_f(query[b, s, h * H + d]) for d in range(H)]
                if q_norm_weight is not None:
                    qv = _norm_head(qv, q_norm_weight, qk_norm_epsilon)
                if do_rotary:
                    qv = _rot_head(qv, cos_cache[p], sin_cache[p], False)
                kh = h // g
                scores = []
                n_keys = total if causal else S
                for j in range(n_keys):
                    if causal:
                        if j > p:
                            continue
                        if local_window_size >= 0 and j < p - local_window_size:
                            continue
                    x = sc * sum(qv[d] * _f(pk[b, kh, j, d]) for d in range(H))
                    if softcap_value and softcap_value > 0:
                        x = softcap_value * math.tanh(x / softcap_value)
                    if attention_bias is not None:
                        bb = 0 if attention_bias.shape[0] == 1 else b
                        hh = 0 if attention_bias.shape[1] == 1 else h
                        x += _f(attention_bias[bb, hh, s, j])
                    scores.append((x, j))
                sink = None
                if head_sink is not None:
                    sink = _f(head_sink[h])
                elif smooth_softmax == 1:
                    sink = 0.0
                o = _softmax_sum(scores, lambda j: [_f(pv[b, kh, j, d]) for d in range(H)], H, sink)
                for d in range(H):
                    out[b, s, h * H + d] = o[d]
    return out, pk, pv


def brute_dmmha(query, key, value, *, num_heads, mask_index=None, attention_bias=None,
                past_key=None, past_value=None, past_sequence_length=None,
                mask_filter_value=-10000.0, scale=0.0, output_qk=0):
    dt = np.asarray(query).dtype
    B, _, qh = np.asarray(query).shape
    N = num_heads
    H = qh // N
    sc = _scale(scale, H)
    out = np.zeros((B, 1, N * H))
    pk = pv = qk = None
    if past_key is not None:
        P = int(np.asarray(past_sequence_length).reshape(-1)[0])
        pk = np.array(past_key, copy=True)
        pv = np.array(past_value, copy=True)
        for b in range(B):
            for h in range(N):
                for d in range(H):
                    pk[b, h, P, d] = dt.type(_f(key[b, 0, h * H + d]))
                    pv[b, h, P, d] = dt.type(_f(value[b, 0, h * H + d]))
        n_keys = P + 1
        kget = lambda b, h, j, d: _f(pk[b, h, j, d])
        vget = lambda b, h, j, d: _f(pv[b, h, j, d])
    else:
        n_keys = np.asarray(key).shape[2]
        kget = lambda b, h, j, d: _f(key[b, h, j, d])
        vget = lambda b, h, j, d: _f(value[b, h, j, d])
        if output_qk:
            qk = np.zeros((B, N, 1, n_keys))
    for b in range(B):
        for h in range(N):
            scores = []
            for j in range(n_keys):
                x = sc * sum(_f(query[b, 0, h * H + d]) * kget(b, h, j, d) for d in range(H))
                if attention_bias is not None:
                    bb = 0 if attention_bias.shape[0] == 1 else b
                    hh = 0 if attention_bias.shape[1] == 1 else h
                    x += _f(attention_bias[bb, hh, 0, j])
                if mask_index is not None and int(mask_index[b, j]) == 0:
                    x += float(mask_filter_value)
                if qk is not None:
                    qk[b, h, 0, j] = x
                scores.append((x, j))
            o = _softmax_sum(scores, lambda j: [vget(b, h, j, d) for d in range(H)], H)
            for d in range(H):
                out[b, 0, h * H + d] = o[d]
    return out, pk, pv, qk


def brute_sparse(query, key, value, past_key, past_value, *, block_row_indices,
                 block_col_indices, total_sequence_length, key_total_sequence_lengths,
                 num_heads, kv_num_heads, sparse_block_size, cos_cache=None,
                 sin_cache=None, do_rotary=0, rotary_interleaved=0, scale=0.0):
    dt = np.asarray(query).dtype
    B, S, width = np.asarray(query).shape
    N, kvN = num_heads, kv_num_heads
    if key is None:
        H = width // (N + 2 * kvN)
        qget = lambda b, s, h, d: _f(query[b, s, h * H + d])
        kget = lambda b, s, h, d: _f(query[b, s, (N + h) * H + d])
        vget = lambda b, s, h, d: _f(query[b, s, (N + kvN + h) * H + d])
    else:
        H = width // N
        qget = lambda b, s, h, d: _f(query[b, s, h * H + d])
        kget = lambda b, s, h, d: _f(key[b, s, h * H + d])
        vget = lambda b, s, h, d: _f(value[b, s, h * H + d])
    g = N // kvN
    bs = sparse_block_size
    L = np.asarray(block_row_indices).shape[0]
    sc = _scale(scale, H)
    pk = np.array(past_key, copy=True)
    pv = np.array(past_value, copy=True)
    out = np.zeros((B, S, N * H))
    inter = rotary_interleaved == 1
    for b in range(B):
        ktot = int(key_total_sequence_lengths[b])
        past = 0 if int(total_sequence_length) == S else ktot - S
        for s in range(S):
            p = past + s
            for kh in range(kvN):
                kv = [kget(b, s, kh, d) for d in range(H)]
                if do_rotary == 1:
                    kv = _rot_head(kv, cos_cache[p], sin_cache[p], inter)
                for d in range(H):
                    pk[b, kh, p, d] = dt.type(kv[d])
                    pv[b, kh, p, d] = dt.type(vget(b, s, kh, d))
        for s in range(S):
            p = past + s
            r = p // bs
            for h in range(N):
                l = h % L
                lo = int(block_row_indices[l][r])
                hi = int(block_row_indices[l][r + 1])
                allowed = [int(c) for c in block_col_indices[l][lo:hi]]
                qv = [qget(b, s, h, d) for d in range(H)]
                if do_rotary == 1:
                    qv = _rot_head(qv, cos_cache[p], sin_cache[p], inter)
                kh = h // g
                scores = []
                for j in range(ktot):
                    if j > p or (j // bs) not in allowed:
                        continue
                    x = sc * sum(qv[d] * _f(pk[b, kh, j, d]) for d in range(H))
                    scores.append((x, j))
                o = _softmax_sum(scores, lambda j: [_f(pv[b, kh, j, d]) for d in range(H)], H)
                for d in range(H):
                    out[b, s, h * H + d] = o[d]
    return out, pk, pv


def brute_packed(input, weights, bias, token_offset, cumulative_sequence_length, *,
                 num_heads, attention_bias=None, qkv_hidden_sizes=None, scale=0.0):
    x = np.asarray(input)
    T, D = x.shape
    n_out = np.asarray(weights).shape[1]
    if qkv_hidden_sizes:
        qs, ks, vs = qkv_hidden_sizes
    else:
        qs = ks = vs = n_out // 3
    N = num_heads
    Hq, Hv = qs // N, vs // N
    sc = _scale(scale, Hq)
    S = np.asarray(token_offset).shape[1]
    flat = [int(a) for a in np.asarray(token_offset).reshape(-1)]
    qkv = [[sum(_f(x[t, i]) * _f(weights[i, c]) for i in range(D)) + _f(bias[c])
            for c in range(n_out)] for t in range(T)]
    out = np.zeros((T, N * Hv))
    cum = [int(c) for c in cumulative_sequence_length]
    for b in range(len(cum) - 1):
        for t in range(cum[b], cum[b + 1]):
            for h in range(N):
                scores = []
                for u in range(cum[b], cum[b + 1]):
                    s_ = sc * sum(qkv[t][h * Hq + d] * qkv[u][qs + h * Hq + d] for d in range(Hq))
                    if attention_bias is not None:
                        bb = 0 if attention_bias.shape[0] == 1 else b
                        hh = 0 if attention_bias.shape[1] == 1 else h
                        s_ += _f(attention_bias[bb, hh, flat[t] - b * S, flat[u] - b * S])
                    scores.append((s_, u))
                o = _softmax_sum(scores, lambda u: [qkv[u][qs + ks + h * Hv + d] for d in range(Hv)], Hv)
                for d in range(Hv):
                    out[t, h * Hv + d] = o[d]
    return out
