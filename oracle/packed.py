"""Oracle for com.microsoft.PackedAttention.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).
"""

import numpy as np

from .common import attend, default_scale


def packed_schedule(cumulative_sequence_length, token_count):
    """Per packed token: owning sequence and position inside it.

    PackedAttention page, Inputs table (``cumulative_sequence_length``: the
    packed tokens cum[i] .. cum[i + 1] - 1 belong to sequence i).  seq(t) is the b with
    cum[b] <= t < cum[b + 1]; pos(t) = t - cum[b].  Written as a plain scan.
    Returns two int32 arrays of length ``token_count``.
    """
    cum = np.asarray(cumulative_sequence_length, dtype=np.int64)
    seq = np.empty(token_count, dtype=np.int32)
    pos = np.empty(token_count, dtype=np.int32)
    for b in range(len(cum) - 1):
        for t in range(int(cum[b]), int(cum[b + 1])):
            seq[t] = b
            pos[t] = t - int(cum[b])
    return seq, pos


def packed(input, weights, bias, token_offset, cumulative_sequence_length, *,
           num_heads, attention_bias=None, qkv_hidden_sizes=None, scale=0.0,
           sequences=None):
    """Self-attention with a fused QKV projection over a padding-removed stream.

    Follows the PackedAttention page: Description, Inputs, Outputs and
    Attributes tables.

    1. qkv = input @ weights + bias in float64, no rounding; the columns
       hold Q for every head, then K for every head, then V.
    2. Sizes come from ``qkv_hidden_sizes`` or, when omitted, bias length / 3;
       q_hidden must equal k_hidden.  Hq = q_hidden / N, Hv = v_hidden / N.
    3. The packed tokens cum[b] .. cum[b + 1] - 1 form sequence b; a token attends
       every key of its own sequence and no other (there is no mask input).
    4. score = scale * q . k (+ attention_bias[b|0, h|0, pad(t), pad(t')]);
       the bias is indexed in padded coordinates, pad(t) = token_offset.flat[t]
       - b * S where S is the padded sequence length carried by token_offset.
    5. Softmax over the sequence's keys, weighted sum of values; the output is
       [token_count, v_hidden] in packed token order.

    ``sequences`` (optional iterable of b) computes only those sequences' rows;
    the other rows of the returned array are left at 0.
    """
    x = np.asarray(input, dtype=np.float64)
    Wt = np.asarray(weights, dtype=np.float64)
    bv = np.asarray(bias, dtype=np.float64)
    T = x.shape[0]
    N = int(num_heads)
    if qkv_hidden_sizes is None or len(qkv_hidden_sizes) == 0:
        if bv.shape[0] % 3:
            raise ValueError("bias length must split in three")
        qs = ks = vs = bv.shape[0] // 3
    else:
        qs, ks, vs = (int(a) for a in qkv_hidden_sizes)
    if qs != ks:
        raise ValueError("q_hidden must equal k_hidden")
    if qs % N or vs % N:
        raise ValueError("hidden sizes must be divisible by num_heads")
    Hq, Hv = qs // N, vs // N
    sc = default_scale(scale, Hq)
    tok = np.asarray(token_offset)
    Bp, S = tok.shape
    cum = np.asarray(cumulative_sequence_length, dtype=np.int64)
    flat = tok.reshape(-1).astype(np.int64)
    bias_a = None if attention_bias is None else np.asarray(attention_bias, dtype=np.float64)

    qkv = x @ Wt + bv
    q = qkv[:, :qs].reshape(T, N, Hq)
    k = qkv[:, qs:qs + ks].reshape(T, N, Hq)
    v = qkv[:, qs + ks:qs + ks + vs].reshape(T, N, Hv)
    out = np.zeros((T, N, Hv))
    seqs = range(len(cum) - 1) if sequences is None else sequences
    for b in seqs:
        t0, t1 = int(cum[b]), int(cum[b + 1])
        if t1 <= t0:
            continue
        pad = flat[t0:t1] - b * S
        vis = np.ones((t1 - t0, t1 - t0), dtype=bool)
        for h in range(N):
            s_ = sc * (q[t0:t1, h, :] @ k[t0:t1, h, :].T)
            if bias_a is not None:
                bb = bias_a[b if bias_a.shape[0] > 1 else 0, h if bias_a.shape[1] > 1 else 0]
                s_ = s_ + bb[np.ix_(pad, pad)]
            o, _ = attend(s_, vis, v[t0:t1, h, :])
            out[t0:t1, h, :] = o
    return out.reshape(T, N * Hv)
