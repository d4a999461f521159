"""Oracle for com.microsoft.SparseAttention.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).
"""

import numpy as np

from .common import attend, default_scale, rotary, round_to


def csr_visible_blocks(block_row_indices, block_col_indices, layout, row):
    """Set of key blocks that query block ``row`` of ``layout`` attends.

    SparseAttention page, Inputs table (``block_row_indices``: CSR row
    pointers per layout; ``block_col_indices``: column indices, right-padded
    past the layout's non-zero count).  The active entries of row r are
    ``cols[layout][rp[layout][r] : rp[layout][r + 1]]``; padding is ignored and
    the column order carries no meaning (set semantics).
    """
    rp = np.asarray(block_row_indices)
    cols = np.asarray(block_col_indices)
    lo, hi = int(rp[layout, row]), int(rp[layout, row + 1])
    return set(int(c) for c in cols[layout, lo:hi])


def sparse(query, key, value, past_key, past_value, *, block_row_indices,
           block_col_indices, total_sequence_length, key_total_sequence_lengths,
           num_heads, kv_num_heads, sparse_block_size,
           cos_cache=None, sin_cache=None, do_rotary=0, rotary_interleaved=0,
           scale=0.0, query_rows=None):
    """Block-sparse causal grouped-query attention with an in-place cache.

    Follows the SparseAttention page: Description, Inputs, Outputs and
    Attributes tables.

    1. ``key``/``value`` None means ``query`` is packed [Q|K|V] of width
       (N + 2 kvN) * H and is split in that order.
    2. The call is a prompt iff ``total_sequence_length`` == S; then past_b = 0.
       Otherwise past_b = key_total_sequence_lengths[b] - S (reading: the new
       rows end at the sample's total key length).
    3. With ``do_rotary`` = 1 the first r = 2 * cos_cache width dims of every
       query and new key head are rotated at position past_b + s, NeoX
       half-split unless ``rotary_interleaved`` = 1; other dims pass through.
    4. The new keys (rotated) and values are written in place, rounded to T,
       at rows [past_b, past_b + S) of the caches.
    5. Query head h uses layout l = h mod num_layout ("layouts cycle over query
       heads") and kv head h // (N / kvN).  Key j is visible to the query at
       position p iff j <= p, j < key_total_sequence_lengths[b], and block
       j // bs is in the CSR column set of query block p // bs.
    6. Plain softmax over visible keys and the weighted sum of values.

    ``query_rows`` restricts the output rows as in ``oracle.gqa``.
    Returns ``(output float64, present_key T, present_value T)``.
    """
    q_in = np.asarray(query)
    dtype = q_in.dtype
    B, S, width = q_in.shape
    N, kvN = int(num_heads), int(kv_num_heads)
    if N % kvN:
        raise ValueError("kv_num_heads must divide num_heads")
    if key is None:
        H = width // (N + 2 * kvN)
        qf = q_in.astype(np.float64)
        q = qf[:, :, :N * H]
        k = qf[:, :, N * H:(N + kvN) * H]
        v = qf[:, :, (N + kvN) * H:]
    else:
        H = width // N
        q = q_in.astype(np.float64)
        k = np.asarray(key, dtype=np.float64)
        v = np.asarray(value, dtype=np.float64)
    g = N // kvN
    bs = int(sparse_block_size)
    # only the query rows asked for are rotated (each row on its own)
    rows = np.arange(S) if query_rows is None else np.asarray(list(query_rows), dtype=np.int64)
    q = q.reshape(B, S, N, H)[:, rows]
    k = k.reshape(B, S, kvN, H)
    v = v.reshape(B, S, kvN, H)
    rp = np.asarray(block_row_indices)
    cols = np.asarray(block_col_indices)
    L = rp.shape[0]
    key_total = np.asarray(key_total_sequence_lengths, dtype=np.int64)
    if int(total_sequence_length) == S:
        past_b = np.zeros(B, dtype=np.int64)
    else:
        past_b = key_total - S
    pk = np.array(past_key, copy=True)
    pv = np.array(past_value, copy=True)
    pos = past_b[:, None] + np.arange(S)[None, :]
    if do_rotary == 1:
        cos = np.asarray(cos_cache, dtype=np.float64)
        sin = np.asarray(sin_cache, dtype=np.float64)
        c = cos[pos][:, :, None, :]
        s_ = sin[pos][:, :, None, :]
        q = rotary(q, c[:, rows], s_[:, rows], interleaved=(rotary_interleaved == 1))
        k = rotary(k, c, s_, interleaved=(rotary_interleaved == 1))
    for b in range(B):
        pb = int(past_b[b])
        pk[b, :, pb:pb + S, :] = round_to(k[b].transpose(1, 0, 2), dtype)
        pv[b, :, pb:pb + S, :] = round_to(v[b].transpose(1, 0, 2), dtype)

    sc = default_scale(scale, H)
    out = np.zeros((B, len(rows), N, H))
    for b in range(B):
        n_keys = int(key_total[b])
        j = np.arange(n_keys)
        p = pos[b, rows]
        base = (j[None, :] <= p[:, None])
        for l in range(L):
            heads = [h for h in range(N) if h % L == l]
            if not heads:
                continue
            vis = base.copy()
            for ri, pp in enumerate(p):
                allowed = csr_visible_blocks(rp, cols, l, int(pp) // bs)
                blk_ok = np.isin(j // bs, np.fromiter(allowed, dtype=np.int64, count=len(allowed)))
                vis[ri] &= blk_ok
            for h in heads:
                kh = h // g
                keys = pk[b, kh, :n_keys].astype(np.float64)
                vals = pv[b, kh, :n_keys].astype(np.float64)
                x = sc * (q[b, :, h, :] @ keys.T)
                o, _ = attend(x, vis, vals)
                out[b, :, h, :] = o
    return out.reshape(B, len(rows), N * H), pk, pv
