"""Seeded synthetic inputs for the attention operators.

This module only draws inputs: it holds none of the operators' arithmetic, so
the HIP path and the CPU oracle can both be fed from it without sharing any
attention code.  Every draw is made with ``numpy.random.default_rng(seed)``
in float64, in the order the fields are listed, then cast to the storage type
with round-to-nearest-even.  Integer fields (lengths, CSR layouts, packed
schedules) are built deterministically from the drawn lengths.

Named workloads (sizes and distributions):

* ``gqa_prompt_small``  GroupQueryAttention prompt, no past cache: B=1, S=128,
  N=8, kvN=2, H=64, fp32, causal, scale 1/8, seqlens_k=[127], Q/K/V ~ N(0,1).
* ``gqa_decode``        GroupQueryAttention decode of one new token: B=16, N=32,
  kvN=8, H=128, fp16, shared BNSH cache of capacity 4096, past lengths uniform
  in [1024, 4095], rotary (theta 10000), Q/K/V/cache ~ N(0,1).
* ``gqa_decode_int8``   the decode above over an int8 cache: float32 Q/K/V,
  uniform random int8 codes, per-channel key and value scales 3/127 times
  uniform [0.5, 1.5).
* ``gqa_decode_int4``   the same over a packed int4 cache (two codes per byte),
  uniform random bytes, scales drawn as for int8.
* ``gqa_long_prefill``  GroupQueryAttention prompt: B=4, S=4096, N=32, kvN=8,
  H=128, fp16, causal, local window 1024, softcap 50, head_sink ~ N(0,1),
  Q/K RMSNorm weights ~ 1+N(0,0.1), rotary theta 10000.
* ``sparse_prompt``     SparseAttention prompt: B=2, S=8192, N=32, kvN=8, H=128,
  fp16, block 64, four CSR layouts (8 local blocks plus every 8th vertical
  block, lower triangular), NeoX rotary over the full head.
* ``sparse_generation`` SparseAttention token generation: the sparse prompt's
  configuration continued by one token after a past of 8191 rows.
* ``packed_varlen``     PackedAttention: 64 sequences, lengths uniform in
  [32, 512] (padded length 512), hidden 768, weights [768, 2304] ~ N(0,0.02),
  bias ~ N(0,0.02), 12 heads of 64, fp16.
"""

import numpy as np

F16 = np.float16
F32 = np.float32


def _cast(a, dtype):
    return np.asarray(a, dtype=np.float64).astype(dtype)


def normal(rng, shape, dtype, std=1.0, mean=0.0):
    """float64 N(mean, std) draws cast to ``dtype`` (round to nearest even)."""
    return _cast(rng.standard_normal(shape) * std + mean, dtype)


def rope_cache(max_seq, rot_dim, dtype, theta=10000.0):
    """cos/sin caches of shape (max_seq, rot_dim/2) with angle p * theta^(-2i/rot_dim).

    These are operator inputs (the rotary tables), generated in float64 and
    cast to ``dtype``.
    """
    half = rot_dim // 2
    inv = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / rot_dim)
    ang = np.arange(max_seq, dtype=np.float64)[:, None] * inv[None, :]
    return _cast(np.cos(ang), dtype), _cast(np.sin(ang), dtype)


# --------------------------------------------------------------------------
# GroupQueryAttention
# --------------------------------------------------------------------------

def gqa_case(rng, *, B, S, N, kvN, H, dtype=F16, past=None, past_lens=None,
             cap=None, rotary=False, rope_rows=None, norm=False, bias=None,
             sink=False, smooth_softmax=-1, softcap=0.0, window=-1, causal=1,
             scale=0.0, total_lens=None, quant=None, cache_dtype=None):
    """A GroupQueryAttention call with random data.

    past: None (prompt), "shared" (present buffer is the past buffer, capacity
    ``cap``) or "concat" (separate present buffer of seq past_seq + S).
    past_lens: per-batch past length (int array); drawn when None.
    total_lens: prompt only: per-batch total length (<= S); default S.
    cache_dtype: prompt only: the present buffers' float type (default dtype).
    bias: None or one of "full", "b1" (batch dim 1), "h1" (head dim 1), "11".
    quant: None or dict(bits=8|4, k="tensor"|"channel", v=...): quantised
    caches (float32 dtype) holding uniform random codes, with scales drawn by
    ``quant_scales``; a separate present buffer starts as bytes 0x5A.
    Returns dict(inputs=..., attrs=..., shared=bool).
    """
    q = normal(rng, (B, S, N * H), dtype)
    k = normal(rng, (B, S, kvN * H), dtype)
    v = normal(rng, (B, S, kvN * H), dtype)
    inputs = dict(query=q, key=k, value=v)
    shared = False
    if quant is not None:
        return _gqa_quant_case(rng, inputs, B=B, S=S, N=N, kvN=kvN, H=H, past=past,
                               past_lens=past_lens, cap=cap, rotary=rotary, norm=norm,
                               bias=bias, sink=sink, smooth_softmax=smooth_softmax,
                               softcap=softcap, window=window, causal=causal, scale=scale,
                               total_lens=total_lens, quant=quant)
    if past is None:
        tl = np.full(B, S, dtype=np.int64) if total_lens is None else np.asarray(total_lens)
        seqlens_k = (tl - 1).astype(np.int32)
        present_seq = S if cap is None else cap
        # a prompt's present cache may have its own float type
        cdt = dtype if cache_dtype is None else cache_dtype
        pk = np.zeros((B, kvN, present_seq, H), cdt)
        pv = np.zeros((B, kvN, present_seq, H), cdt)
        inputs.update(present_key=pk, present_value=pv)
        max_pos = S
    else:
        if cap is None:
            cap = S + 16
        if past_lens is None:
            past_lens = rng.integers(0, cap - S + 1, B)
        past_lens = np.asarray(past_lens, dtype=np.int64)
        seqlens_k = (past_lens + S - 1).astype(np.int32)
        if past == "shared":
            pk = normal(rng, (B, kvN, cap, H), dtype)
            pv = normal(rng, (B, kvN, cap, H), dtype)
            inputs.update(past_key=pk, past_value=pv, present_key=pk, present_value=pv)
            shared = True
        else:
            past_seq = int(np.max(past_lens)) if cap is None else cap - S
            pk = normal(rng, (B, kvN, past_seq, H), dtype)
            pv = normal(rng, (B, kvN, past_seq, H), dtype)
            inputs.update(past_key=pk, past_value=pv,
                          present_key=np.full((B, kvN, past_seq + S, H), np.nan, dtype),
                          present_value=np.full((B, kvN, past_seq + S, H), np.nan, dtype))
        max_pos = int(np.max(past_lens)) + S
    inputs["seqlens_k"] = seqlens_k
    total = int(np.max(seqlens_k)) + 1
    if causal == 0:
        total = S
    if rotary:
        rows = max(max_pos, total) if rope_rows is None else rope_rows
        c, s_ = rope_cache(rows, H, dtype)
        inputs.update(cos_cache=c, sin_cache=s_)
    if bias is not None:
        bshape = {"full": (B, N), "b1": (1, N), "h1": (B, 1), "11": (1, 1)}[bias]
        inputs["attention_bias"] = normal(rng, bshape + (S, total), dtype)
    if sink:
        inputs["head_sink"] = normal(rng, (N,), dtype)
    if norm:
        inputs["q_norm_weight"] = normal(rng, (H,), dtype, std=0.1, mean=1.0)
        inputs["k_norm_weight"] = normal(rng, (H,), dtype, std=0.1, mean=1.0)
    attrs = dict(num_heads=N, kv_num_heads=kvN, causal=causal, do_rotary=int(rotary),
                 local_window_size=window, qk_norm_epsilon=1e-6, scale=scale,
                 smooth_softmax=smooth_softmax, softcap=softcap)
    return dict(op="gqa", inputs=inputs, attrs=attrs, total_sequence_length=total,
                shared=shared)


def quant_scales(rng, kind, kvN, H, bits):
    """float32 cache scales: one value ("tensor") or kvN*H values ("channel").
    The base step is 3/127 (8 bits) or 3/7 (4 bits), so that N(0,1) data
    spans about three standard deviations of the code range; per-channel
    scales are the base times uniform [0.5, 1.5)."""
    base = 3.0 / ((1 << (bits - 1)) - 1)
    if kind == "tensor":
        return np.array([base], np.float32)
    return (base * rng.uniform(0.5, 1.5, kvN * H)).astype(np.float32)


def random_codes(rng, shape, bits):
    """Uniform random cache elements: int8 codes, or packed uint8 bytes."""
    if bits == 8:
        return rng.integers(-128, 128, shape).astype(np.int8)
    return rng.integers(0, 256, shape).astype(np.uint8)


def _gqa_quant_case(rng, inputs, *, B, S, N, kvN, H, past, past_lens, cap, rotary, norm, bias,
                    sink, smooth_softmax, softcap, window, causal, scale, total_lens, quant):
    bits = int(quant["bits"])
    hc = H if bits == 8 else H // 2
    cdt = np.int8 if bits == 8 else np.uint8
    shared = False
    if past is None:
        tl = np.full(B, S, dtype=np.int64) if total_lens is None else np.asarray(total_lens)
        seqlens_k = (tl - 1).astype(np.int32)
        present_seq = S if cap is None else cap
        inputs.update(present_key=np.zeros((B, kvN, present_seq, hc), cdt),
                      present_value=np.zeros((B, kvN, present_seq, hc), cdt))
        max_pos = S
    else:
        if cap is None:
            cap = S + 16
        if past_lens is None:
            past_lens = rng.integers(0, cap - S + 1, B)
        past_lens = np.asarray(past_lens, dtype=np.int64)
        seqlens_k = (past_lens + S - 1).astype(np.int32)
        if past == "shared":
            pk = random_codes(rng, (B, kvN, cap, hc), bits)
            pv = random_codes(rng, (B, kvN, cap, hc), bits)
            inputs.update(past_key=pk, past_value=pv, present_key=pk, present_value=pv)
            shared = True
        else:
            past_seq = cap - S
            pk = random_codes(rng, (B, kvN, past_seq, hc), bits)
            pv = random_codes(rng, (B, kvN, past_seq, hc), bits)
            fill = np.full((B, kvN, past_seq + S, hc), 0x5A, np.uint8).view(cdt)
            inputs.update(past_key=pk, past_value=pv, present_key=fill, present_value=fill.copy())
        max_pos = int(np.max(past_lens)) + S
    inputs["seqlens_k"] = seqlens_k
    total = int(np.max(seqlens_k)) + 1
    if causal == 0:
        total = S
    dtype = F32
    if rotary:
        c, s_ = rope_cache(max(max_pos, total), H, dtype)
        inputs.update(cos_cache=c, sin_cache=s_)
    if bias is not None:
        bshape = {"full": (B, N), "b1": (1, N), "h1": (B, 1), "11": (1, 1)}[bias]
        inputs["attention_bias"] = normal(rng, bshape + (S, total), dtype)
    if sink:
        inputs["head_sink"] = normal(rng, (N,), dtype)
    if norm:
        inputs["q_norm_weight"] = normal(rng, (H,), dtype, std=0.1, mean=1.0)
        inputs["k_norm_weight"] = normal(rng, (H,), dtype, std=0.1, mean=1.0)
    kind = {"tensor": 1, "channel": 2}
    inputs["k_scale"] = quant_scales(rng, quant["k"], kvN, H, bits)
    inputs["v_scale"] = quant_scales(rng, quant["v"], kvN, H, bits)
    attrs = dict(num_heads=N, kv_num_heads=kvN, causal=causal, do_rotary=int(rotary),
                 local_window_size=window, qk_norm_epsilon=1e-6, scale=scale,
                 smooth_softmax=smooth_softmax, softcap=softcap,
                 k_quant_type=kind[quant["k"]], v_quant_type=kind[quant["v"]],
                 kv_cache_bit_width=bits)
    return dict(op="gqa", inputs=inputs, attrs=attrs, total_sequence_length=total,
                shared=shared)


def gqa_prompt_small(seed=1):
    """GroupQueryAttention prompt, no past: B=1 S=128 N=8 kvN=2 H=64 fp32 causal."""
    rng = np.random.default_rng(seed)
    B, S, N, kvN, H = 1, 128, 8, 2, 64
    q = normal(rng, (B, S, N * H), F32)
    k = normal(rng, (B, S, kvN * H), F32)
    v = normal(rng, (B, S, kvN * H), F32)
    inputs = dict(query=q, key=k, value=v,
                  seqlens_k=np.array([127], np.int32),
                  present_key=np.zeros((B, kvN, S, H), F32),
                  present_value=np.zeros((B, kvN, S, H), F32))
    attrs = dict(num_heads=N, kv_num_heads=kvN, causal=1, do_rotary=0,
                 local_window_size=-1, qk_norm_epsilon=1e-6, scale=0.125,
                 smooth_softmax=-1, softcap=0.0)
    return dict(op="gqa", name="gqa_prompt_small", inputs=inputs, attrs=attrs,
                total_sequence_length=128, shared=False)


def gqa_decode(seed=2, batch=16, cap=4096):
    """GroupQueryAttention decode: B=16 N=32 kvN=8 H=128 fp16, shared cache 4096."""
    rng = np.random.default_rng(seed)
    B, S, N, kvN, H = batch, 1, 32, 8, 128
    past = rng.integers(1024, cap, B)
    q = normal(rng, (B, S, N * H), F16)
    k = normal(rng, (B, S, kvN * H), F16)
    v = normal(rng, (B, S, kvN * H), F16)
    pk = normal(rng, (B, kvN, cap, H), F16)
    pv = normal(rng, (B, kvN, cap, H), F16)
    c, s_ = rope_cache(cap, H, F16)
    inputs = dict(query=q, key=k, value=v, past_key=pk, past_value=pv,
                  present_key=pk, present_value=pv,
                  seqlens_k=past.astype(np.int32), cos_cache=c, sin_cache=s_)
    attrs = dict(num_heads=N, kv_num_heads=kvN, causal=1, do_rotary=1,
                 local_window_size=-1, qk_norm_epsilon=1e-6, scale=0.0,
                 smooth_softmax=-1, softcap=0.0)
    return dict(op="gqa", name="gqa_decode", inputs=inputs, attrs=attrs,
                total_sequence_length=int(past.max()) + 1, shared=True)


def gqa_window_decode(seed=6, batch=16, cap=1024, window=1023, max_total=4096):
    """GroupQueryAttention decode on a sliding-window cache: B=16 N=32 kvN=8
    H=128 fp16, shared window buffers of capacity 1024, window 1023, tokens
    seen before the step uniform in [1024, 4095] (every step evicts one row),
    rotary at absolute positions."""
    rng = np.random.default_rng(seed)
    B, S, N, kvN, H = batch, 1, 32, 8, 128
    past = rng.integers(cap, max_total, B)
    q = normal(rng, (B, S, N * H), F16)
    k = normal(rng, (B, S, kvN * H), F16)
    v = normal(rng, (B, S, kvN * H), F16)
    pk = normal(rng, (B, kvN, cap, H), F16)
    pv = normal(rng, (B, kvN, cap, H), F16)
    c, s_ = rope_cache(max_total, H, F16)
    inputs = dict(query=q, key=k, value=v, past_key=pk, past_value=pv,
                  present_key=pk, present_value=pv,
                  seqlens_k=past.astype(np.int32), cos_cache=c, sin_cache=s_)
    attrs = dict(num_heads=N, kv_num_heads=kvN, causal=1, do_rotary=1,
                 local_window_size=window, qk_norm_epsilon=1e-6, scale=0.0,
                 smooth_softmax=-1, softcap=0.0, sliding_window_cache=1)
    return dict(op="gqa", name="gqa_window_decode", inputs=inputs, attrs=attrs,
                total_sequence_length=int(past.max()) + 1, shared=True)


def gqa_decode_int8(seed=8, batch=16, cap=4096):
    """GroupQueryAttention decode over an int8 cache: B=16 N=32 kvN=8 H=128,
    float32 Q/K/V, shared int8 BNSH cache of capacity 4096 with uniform random
    codes, per-channel key and value scales (3/127 times uniform [0.5, 1.5)),
    past lengths uniform in [1024, 4095], rotary theta 10000."""
    rng = np.random.default_rng(seed)
    past = rng.integers(1024, cap, batch)
    return gqa_case(rng, B=batch, S=1, N=32, kvN=8, H=128, dtype=F32, past="shared",
                    past_lens=past, cap=cap, rotary=True,
                    quant=dict(bits=8, k="channel", v="channel")) | dict(name="gqa_decode_int8")


def gqa_decode_int4(seed=9, batch=16, cap=4096):
    """GroupQueryAttention decode over a packed int4 cache: as gqa_decode_int8
    with two codes per byte (uniform random bytes)."""
    rng = np.random.default_rng(seed)
    past = rng.integers(1024, cap, batch)
    return gqa_case(rng, B=batch, S=1, N=32, kvN=8, H=128, dtype=F32, past="shared",
                    past_lens=past, cap=cap, rotary=True,
                    quant=dict(bits=4, k="channel", v="channel")) | dict(name="gqa_decode_int4")


def gqa_long_prefill(seed=3, batch=4, seq=4096):
    """GroupQueryAttention prompt: B=4 S=4096 N=32 kvN=8 H=128 fp16, window 1024,
    softcap 50, head sink, Q/K RMSNorm, rotary."""
    rng = np.random.default_rng(seed)
    B, S, N, kvN, H = batch, seq, 32, 8, 128
    q = normal(rng, (B, S, N * H), F16)
    k = normal(rng, (B, S, kvN * H), F16)
    v = normal(rng, (B, S, kvN * H), F16)
    sink = normal(rng, (N,), F16)
    qw = normal(rng, (H,), F16, std=0.1, mean=1.0)
    kw = normal(rng, (H,), F16, std=0.1, mean=1.0)
    c, s_ = rope_cache(S, H, F16)
    inputs = dict(query=q, key=k, value=v, seqlens_k=np.full(B, S - 1, np.int32),
                  present_key=np.zeros((B, kvN, S, H), F16),
                  present_value=np.zeros((B, kvN, S, H), F16),
                  head_sink=sink, q_norm_weight=qw, k_norm_weight=kw,
                  cos_cache=c, sin_cache=s_)
    attrs = dict(num_heads=N, kv_num_heads=kvN, causal=1, do_rotary=1,
                 local_window_size=1024, qk_norm_epsilon=1e-6, scale=0.0,
                 smooth_softmax=-1, softcap=50.0)
    return dict(op="gqa", name="gqa_long_prefill", inputs=inputs, attrs=attrs,
                total_sequence_length=S, shared=False)


# --------------------------------------------------------------------------
# DecoderMaskedMultiHeadAttention
# --------------------------------------------------------------------------

def dmmha_self_case(rng, *, B, N, H, cap, past_len, dtype=F16, mask=False,
                    bias=None, scale=0.0, mask_filter_value=-10000.0):
    q = normal(rng, (B, 1, N * H), dtype)
    k = normal(rng, (B, 1, N * H), dtype)
    v = normal(rng, (B, 1, N * H), dtype)
    pk = normal(rng, (B, N, cap, H), dtype)
    pv = normal(rng, (B, N, cap, H), dtype)
    total = past_len + 1
    inputs = dict(query=q, key=k, value=v, past_key=pk, past_value=pv,
                  past_sequence_length=np.array([past_len], np.int32))
    if mask:
        m = (rng.random((B, total)) > 0.3).astype(np.int32)
        inputs["mask_index"] = m
    if bias is not None:
        bshape = {"full": (B, N), "b1": (1, N), "h1": (B, 1), "11": (1, 1)}[bias]
        inputs["attention_bias"] = normal(rng, bshape + (1, total), dtype)
    attrs = dict(num_heads=N, mask_filter_value=mask_filter_value, scale=scale,
                 output_qk=0, past_present_share_buffer=1)
    return dict(op="dmmha", inputs=inputs, attrs=attrs)


def dmmha_cross_case(rng, *, B, N, H, kv_len, dtype=F16, mask=False, scale=0.0,
                     output_qk=0, mask_filter_value=-10000.0):
    q = normal(rng, (B, 1, N * H), dtype)
    k = normal(rng, (B, N, kv_len, H), dtype)
    v = normal(rng, (B, N, kv_len, H), dtype)
    inputs = dict(query=q, key=k, value=v)
    if mask:
        inputs["mask_index"] = (rng.random((B, kv_len)) > 0.3).astype(np.int32)
    attrs = dict(num_heads=N, mask_filter_value=mask_filter_value, scale=scale,
                 output_qk=output_qk, past_present_share_buffer=0)
    return dict(op="dmmha", inputs=inputs, attrs=attrs)


# --------------------------------------------------------------------------
# SparseAttention
# --------------------------------------------------------------------------

def local_vertical_layouts(num_layout, n_blocks, local=8, stride=8):
    """CSR layouts: row r of layout l holds the ``local`` blocks ending at r and
    every ``stride``-th block c <= r with c mod stride == stride-1-l.

    Returns (row_ptr int32 (L, n_blocks+1), cols int32 (L, max_nnz)), columns
    sorted per row and padded with 0 past each layout's count.
    """
    rows_all = []
    for l in range(num_layout):
        rows = []
        for r in range(n_blocks):
            s = set(range(max(0, r - local + 1), r + 1))
            s |= {c for c in range(r + 1) if c % stride == (stride - 1 - l) % stride}
            rows.append(sorted(s))
        rows_all.append(rows)
    nnz = [sum(len(r) for r in rows) for rows in rows_all]
    max_nnz = max(nnz)
    rp = np.zeros((num_layout, n_blocks + 1), np.int32)
    cols = np.zeros((num_layout, max_nnz), np.int32)
    for l, rows in enumerate(rows_all):
        off = 0
        for r, cs in enumerate(rows):
            rp[l, r] = off
            cols[l, off:off + len(cs)] = cs
            off += len(cs)
        rp[l, n_blocks] = off
    return rp, cols


def sparse_case(rng, *, B, S, N, kvN, H, bs, dtype=F16, layouts=None, cap=None,
                past_lens=None, key_total=None, rotary=False, rot_dim=None,
                interleaved=0, packed_qkv=False, scale=0.0):
    """A SparseAttention call with random data.

    Prompt when past_lens is None (total_sequence_length = S); otherwise the new
    rows follow ``past_lens`` and total_sequence_length = max(past + S).
    ``layouts``: (row_ptr, cols) or None for a 4-layout local+vertical set.
    """
    cap = S if cap is None else cap
    if packed_qkv:
        q = normal(rng, (B, S, (N + 2 * kvN) * H), dtype)
        k = v = None
    else:
        q = normal(rng, (B, S, N * H), dtype)
        k = normal(rng, (B, S, kvN * H), dtype)
        v = normal(rng, (B, S, kvN * H), dtype)
    pk = np.zeros((B, kvN, cap, H), dtype)
    pv = np.zeros((B, kvN, cap, H), dtype)
    if past_lens is None:
        total = S
        kt = np.full(B, S, np.int32) if key_total is None else np.asarray(key_total, np.int32)
    else:
        past_lens = np.asarray(past_lens, np.int64)
        pk = normal(rng, (B, kvN, cap, H), dtype)
        pv = normal(rng, (B, kvN, cap, H), dtype)
        kt = (past_lens + S).astype(np.int32)
        total = int(kt.max())
        if total == S:
            raise ValueError("non-prompt case needs total > S")
    n_blocks = (cap + bs - 1) // bs
    if layouts is None:
        layouts = local_vertical_layouts(4, n_blocks, local=2, stride=3)
    rp, cols = layouts
    inputs = dict(query=q, key=k, value=v, past_key=pk, past_value=pv,
                  block_row_indices=rp, block_col_indices=cols,
                  key_total_sequence_lengths=kt)
    if rotary:
        rd = H if rot_dim is None else rot_dim
        c, s_ = rope_cache(cap, rd, dtype)
        inputs.update(cos_cache=c, sin_cache=s_)
    attrs = dict(num_heads=N, kv_num_heads=kvN, sparse_block_size=bs,
                 do_rotary=int(rotary), rotary_interleaved=interleaved, scale=scale)
    return dict(op="sparse", inputs=inputs, attrs=attrs, total_sequence_length=total)


def sparse_prompt(seed=4, batch=2, seq=8192):
    """SparseAttention prompt: B=2 S=8192 N=32 kvN=8 H=128 fp16 block 64, 4 layouts."""
    rng = np.random.default_rng(seed)
    B, S, N, kvN, H, bs = batch, seq, 32, 8, 128, 64
    q = normal(rng, (B, S, N * H), F16)
    k = normal(rng, (B, S, kvN * H), F16)
    v = normal(rng, (B, S, kvN * H), F16)
    pk = np.zeros((B, kvN, S, H), F16)
    pv = np.zeros((B, kvN, S, H), F16)
    rp, cols = local_vertical_layouts(4, S // bs, local=8, stride=8)
    c, s_ = rope_cache(S, H, F16)
    inputs = dict(query=q, key=k, value=v, past_key=pk, past_value=pv,
                  block_row_indices=rp, block_col_indices=cols,
                  key_total_sequence_lengths=np.full(B, S, np.int32),
                  cos_cache=c, sin_cache=s_)
    attrs = dict(num_heads=N, kv_num_heads=kvN, sparse_block_size=bs, do_rotary=1,
                 rotary_interleaved=0, scale=0.0)
    return dict(op="sparse", name="sparse_prompt", inputs=inputs, attrs=attrs,
                total_sequence_length=S)


def sparse_generation(seed=5, batch=2, context=8192):
    """SparseAttention token generation: the sparse prompt's configuration
    (N=32 kvN=8 H=128 fp16, block 64, the same four layouts, NeoX rotary)
    continued by one new token per sample after a past of context - 1 rows
    (cache ~ N(0,1))."""
    rng = np.random.default_rng(seed)
    B, S, N, kvN, H, bs = batch, 1, 32, 8, 128, 64
    q = normal(rng, (B, S, N * H), F16)
    k = normal(rng, (B, S, kvN * H), F16)
    v = normal(rng, (B, S, kvN * H), F16)
    pk = normal(rng, (B, kvN, context, H), F16)
    pv = normal(rng, (B, kvN, context, H), F16)
    rp, cols = local_vertical_layouts(4, context // bs, local=8, stride=8)
    c, s_ = rope_cache(context, H, F16)
    inputs = dict(query=q, key=k, value=v, past_key=pk, past_value=pv,
                  block_row_indices=rp, block_col_indices=cols,
                  key_total_sequence_lengths=np.full(B, context, np.int32),
                  cos_cache=c, sin_cache=s_)
    attrs = dict(num_heads=N, kv_num_heads=kvN, sparse_block_size=bs, do_rotary=1,
                 rotary_interleaved=0, scale=0.0)
    return dict(op="sparse", name="sparse_generation", inputs=inputs, attrs=attrs,
                total_sequence_length=context)


# --------------------------------------------------------------------------
# PackedAttention
# --------------------------------------------------------------------------

def packed_schedule_inputs(lengths, padded_seq):
    """token_offset (B, S) and cumulative_sequence_length (B+1) from lengths.

    token_offset lists each packed token's flat padded index b*S + s (s < L_b)
    in packed order, then the remaining padding positions in order.
    """
    lengths = np.asarray(lengths, np.int64)
    B = len(lengths)
    S = int(padded_seq)
    tok = [b * S + s for b in range(B) for s in range(int(lengths[b]))]
    pad = [b * S + s for b in range(B) for s in range(int(lengths[b]), S)]
    token_offset = np.array(tok + pad, np.int32).reshape(B, S)
    cum = np.zeros(B + 1, np.int32)
    cum[1:] = np.cumsum(lengths)
    return token_offset, cum


def packed_case(rng, *, lengths, padded_seq, D, N, H, dtype=F16, bias_attn=None,
                wstd=0.02, scale=0.0):
    lengths = np.asarray(lengths, np.int64)
    T = int(lengths.sum())
    x = normal(rng, (T, D), dtype)
    w = normal(rng, (D, 3 * N * H), dtype, std=wstd)
    bvec = normal(rng, (3 * N * H,), dtype, std=wstd)
    tok, cum = packed_schedule_inputs(lengths, padded_seq)
    inputs = dict(input=x, weights=w, bias=bvec, token_offset=tok,
                  cumulative_sequence_length=cum)
    if bias_attn is not None:
        B = len(lengths)
        bshape = {"full": (B, N), "b1": (1, N), "h1": (B, 1), "11": (1, 1)}[bias_attn]
        inputs["attention_bias"] = normal(rng, bshape + (padded_seq, padded_seq), dtype)
    attrs = dict(num_heads=N, scale=scale)
    return dict(op="packed", inputs=inputs, attrs=attrs)


def packed_varlen(seed=5, n_seq=64, padded_seq=512):
    """PackedAttention: 64 sequences of 32..512 tokens, hidden 768, 12 heads of 64, fp16."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(32, padded_seq + 1, n_seq)
    case = packed_case(rng, lengths=lengths, padded_seq=padded_seq, D=768, N=12, H=64,
                       dtype=F16, wstd=0.02)
    case["name"] = "packed_varlen"
    case["lengths"] = lengths
    return case


WORKLOADS = {
    "gqa_prompt_small": gqa_prompt_small,
    "gqa_decode": gqa_decode,
    "gqa_window_decode": gqa_window_decode,
    "gqa_decode_int8": gqa_decode_int8,
    "gqa_decode_int4": gqa_decode_int4,
    "gqa_long_prefill": gqa_long_prefill,
    "sparse_prompt": sparse_prompt,
    "sparse_generation": sparse_generation,
    "packed_varlen": packed_varlen,
}
