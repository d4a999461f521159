"""Helpers for the GPU parity tests: run a generated case through the HIP
library (via the Python binding) and through the oracle, and compare with the
tolerances of the attention outputs and the exactness rules of the caches.

Output tolerance (per element, against the float64 oracle):
  float16 storage: |gpu - ref| <= 2e-3 + 2e-3 * |ref|
  float32 storage: |gpu - ref| <= 1e-4 * |ref| + 1e-6 * max(1, V)
where V is the largest magnitude among the values the outputs average (an
output is a weighted average of value rows, so the float32 error of the sum
scales with them, not with the output, which may cancel far below them); V
is taken for quantised caches, whose values code * scale reach about 5.
Cache rows: copied rows (values, untouched and copied past rows, keys without
norm/rotary) bit-exact; keys transformed by norm and/or rotary within 1 ulp of
T (float16) of the float64 result rounded to T, plus 8 float32 ulps of the
largest element of their row (the float32 arithmetic's error, which matters
only where a pair cancels to a value far below its operands).  For float16
caches at most MAX_OFF_FRACTION of the transformed elements may differ from
the oracle's rounding at all (a double rounding lands on the other side of a
float16 tie only when the float32 result sits within its error of the tie).
"""

import numpy as np
import torch

import oracle

DEV = "cuda:0"


def dev(a):
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    return t.detach().cpu().numpy()


def tolerance(ref, dtype, value_max=1.0):
    ref = np.abs(np.asarray(ref, np.float64))
    if np.dtype(dtype) == np.float16:
        return 2e-3 + 2e-3 * ref
    return 1e-4 * ref + 1e-6 * max(1.0, float(value_max))


def check_output(got, ref, dtype, what="output", value_max=1.0):
    got = np.asarray(got).astype(np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    tol = tolerance(ref, dtype, value_max)
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} elements outside tolerance; worst at {i}: "
            f"gpu {got[i]!r} ref {ref[i]!r} (|d| {err[i]:.3g} > tol {tol[i]:.3g})")
    return float(np.max(err)) if err.size else 0.0


def ulp_distance(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    if a.dtype == np.float16:
        ia = a.view(np.uint16).astype(np.int64)
        ib = b.view(np.uint16).astype(np.int64)
        sign, mag = 0x8000, 0x7FFF
    else:
        ia = a.view(np.uint32).astype(np.int64)
        ib = b.view(np.uint32).astype(np.int64)
        sign, mag = 0x80000000, 0x7FFFFFFF
    oa = np.where(ia & sign, sign - (ia & mag), sign + ia)
    ob = np.where(ib & sign, sign - (ib & mag), sign + ib)
    return np.abs(oa - ob)


def check_cache(got, ref, transformed_rows=None, what="cache"):
    """Bit-exact everywhere except ``transformed_rows`` (bool mask over the
    first three axes), which get the bound described in the module docstring.
    Returns the number of transformed elements that are not bit-identical."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape and got.dtype == ref.dtype, f"{what}: shape/dtype"
    d = ulp_distance(got, ref)
    nan_g = np.isnan(got.astype(np.float64))
    nan_r = np.isnan(ref.astype(np.float64))
    assert np.array_equal(nan_g, nan_r), f"{what}: NaN pattern differs"
    d = np.where(nan_g, 0, d)
    if transformed_rows is None:
        transformed_rows = np.zeros(got.shape[:3], bool)
    exact = ~transformed_rows[..., None]
    bad_exact = (d > 0) & exact
    assert not bad_exact.any(), (
        f"{what}: {int(bad_exact.sum())} copied elements differ (first at "
        f"{np.argwhere(bad_exact)[0].tolist()})")
    tr = (~exact) & np.ones_like(d, bool)
    if not tr.any():
        return 0
    # Transformed rows are computed in float32 and rounded once to T.  The
    # float32 error is relative to the operands (a rotated or normed pair can
    # cancel to a value far below them), so the bound is: 1 ulp of T at the
    # reference value (float16) plus 8 float32 ulps of the row's largest
    # element (both storage types).
    g64 = got.astype(np.float64)
    r64 = ref.astype(np.float64)
    scale = np.max(np.abs(r64), axis=-1, keepdims=True)
    err = np.abs(g64 - r64)
    lim = 8 * 2.0 ** -24 * scale
    if got.dtype == np.float16:
        ulp16 = np.spacing(np.abs(np.where(np.isnan(ref), 0, ref))).astype(np.float64)
        lim = lim + ulp16
    bad = tr & (err > lim)
    assert not bad.any(), (f"{what}: {int(bad.sum())} transformed elements beyond the bound "
                           f"(worst {float(np.max(np.where(tr, err - lim, -1))):.3g} over)")
    n_off = int(np.sum(d[tr] > 0))
    if got.dtype == np.float16:
        n_tr = int(tr.sum())
        assert n_off <= MAX_OFF_FRACTION * n_tr + 2, (
            f"{what}: {n_off} of {n_tr} transformed elements differ from the oracle's rounding")
    return n_off


# ---------------------------------------------------------------------------
# GroupQueryAttention
# ---------------------------------------------------------------------------
def gqa_oracle(case, query_rows=None, info=None, stored_key_codes=None):
    i = dict(case["inputs"])
    a = dict(case["attrs"])
    a["softcap_value"] = a.pop("softcap")
    return oracle.gqa(i.pop("query"), i.pop("key"), i.pop("value"),
                      total_sequence_length=case["total_sequence_length"],
                      query_rows=query_rows, info=info, stored_key_codes=stored_key_codes,
                      **i, **a)


def gqa_gpu(case, workspace=None):
    import kv_cache_transformer_amd as kv
    i = case["inputs"]
    a = case["attrs"]
    t = {k: dev(v) for k, v in i.items() if k not in ("present_key", "present_value")}
    if case.get("shared"):
        pk, pv = t["past_key"], t["past_value"]
    else:
        pk, pv = dev(i["present_key"]), dev(i["present_value"])
    out, pk, pv = kv.gqa_attention(
        t["query"], t["key"], t["value"], t.get("past_key"), t.get("past_value"),
        t["seqlens_k"], case["total_sequence_length"], t.get("cos_cache"), t.get("sin_cache"),
        t.get("attention_bias"), t.get("head_sink"), t.get("q_norm_weight"),
        t.get("k_norm_weight"), t.get("k_scale"), t.get("v_scale"),
        num_heads=a["num_heads"], kv_num_heads=a["kv_num_heads"],
        causal=a["causal"], do_rotary=a["do_rotary"], local_window_size=a["local_window_size"],
        qk_norm_epsilon=a["qk_norm_epsilon"], scale=a["scale"],
        smooth_softmax=a["smooth_softmax"], softcap=a["softcap"],
        sliding_window_cache=a.get("sliding_window_cache", 0),
        k_quant_type=a.get("k_quant_type", 0), v_quant_type=a.get("v_quant_type", 0),
        kv_cache_bit_width=a.get("kv_cache_bit_width", 0), present_key=pk,
        present_value=pv, workspace=workspace)
    torch.cuda.synchronize()
    return host(out), host(pk), host(pv)


def gqa_new_rows(case):
    """Cache row of each new token: int array (B, S)."""
    i = case["inputs"]
    B, S = i["query"].shape[:2]
    total = i["seqlens_k"].astype(np.int64) + 1
    past = total - S if i.get("past_key") is not None else np.zeros(B, np.int64)
    if case["attrs"].get("sliding_window_cache"):
        cap = i["present_key"].shape[2]
        held = np.minimum(past, cap)
        past = held - np.maximum(0, held + S - cap)      # rows kept before the new ones
    return past[:, None] + np.arange(S)[None, :]


# Rounding slack of transformed keys in quantised caches (code units): the
# GPU computes a normed/rotated key in float32, the oracle in float64 rounded
# once to float32, so their quotients by the scale may differ by float32
# rounding of the operands (about 1e-5 here); a code may differ only where the
# oracle's quotient lies this close to a rounding boundary.
QUANT_SLACK = 1e-3

# Largest fraction of norm/rotary-transformed float16 cache elements allowed
# to differ (by one ulp) from the float64 result rounded once: measured about
# 2e-4 on the long prefill (normed and rotated keys), 1.5e-5 on the rotated
# block-sparse keys.
MAX_OFF_FRACTION = 1e-3


def check_quant_gqa(case, got, ref, info, query_rows=None):
    """Compare a quantised-cache call: codes of values and of untransformed
    keys bit-exact; codes of normed/rotated keys bit-exact except within
    QUANT_SLACK of a rounding boundary, where they may differ by one; every
    other cache row untouched or copied exactly; the output within the float32
    tolerance everywhere: against the oracle for every (sample, kv head) whose
    codes all match the oracle's, and for the others against the oracle
    evaluated on the codes the kernel stored (the tie's side decides what the
    attention reads).  Returns the number of codes taken on the other side of
    a near tie."""
    from oracle import quant
    out, pk, pv = got
    rout, rpk, rpv = ref
    a = case["attrs"]
    bits = a["kv_cache_bit_width"]
    transformed = bool(a["do_rotary"] or case["inputs"].get("q_norm_weight") is not None)
    assert pk.dtype == rpk.dtype and pk.shape == rpk.shape
    assert np.array_equal(pv, rpv), f"present_value: {int(np.sum(pv != rpv))} bytes differ"
    rows = gqa_new_rows(case)                       # (B, S)
    B, S = rows.shape
    # key rows other than the new ones: exact
    new = np.zeros(pk.shape[:3], bool)
    for b in range(B):
        for s_ in range(S):
            if 0 <= rows[b, s_] < pk.shape[2]:
                new[b, :, rows[b, s_]] = True
    assert np.array_equal(pk[~new], rpk[~new]), "present_key: rows other than the new ones differ"
    gc = quant.load_codes(pk, bits)
    rc = quant.load_codes(rpk, bits)
    diff = gc != rc                                 # (B, kvN, cap, H)
    n_off = 0
    bad_units = np.zeros(pk.shape[:2], bool)
    if diff.any():
        assert transformed, f"present_key: {int(diff.sum())} codes of untransformed keys differ"
        margin = quant.rounding_margin(info["k_quotient"])   # (B, kvN, S, H)
        for b, kh, r, d in np.argwhere(diff):
            s_ = int(np.nonzero(rows[b] == r)[0][0])
            assert margin[b, kh, s_, d] < QUANT_SLACK and abs(int(gc[b, kh, r, d]) - int(rc[b, kh, r, d])) == 1, (
                f"present_key code at {(b, kh, r, d)}: gpu {gc[b, kh, r, d]} oracle {rc[b, kh, r, d]} "
                f"(quotient {info['k_quotient'][b, kh, s_, d]!r})")
            bad_units[b, kh] = True
            n_off += 1
    N, kvN = a["num_heads"], a["kv_num_heads"]
    H = out.shape[-1] // N
    o = out if query_rows is None else out[:, query_rows]
    o = o.reshape(o.shape[0], o.shape[1], N, H)
    r = rout.reshape(rout.shape[0], rout.shape[1], N, H)
    keep = np.repeat(~bad_units, N // kvN, axis=1)  # (B, N)
    vs = quant.channel_scales(case["inputs"]["v_scale"], a["v_quant_type"], kvN, H)
    vmax = float(np.max(np.abs(quant.load_codes(rpv, bits)) * vs[None, :, None, :]))
    check_output(o.transpose(0, 2, 1, 3)[keep], r.transpose(0, 2, 1, 3)[keep], np.float32,
                 value_max=vmax)
    if bad_units.any():
        r2, _, _ = gqa_oracle(case, query_rows=query_rows, stored_key_codes=pk)
        r2 = r2.reshape(r2.shape[0], r2.shape[1], N, H)
        check_output(o.transpose(0, 2, 1, 3)[~keep], r2.transpose(0, 2, 1, 3)[~keep], np.float32,
                     "output of units whose key codes sit across a near tie", value_max=vmax)
    return n_off


def gqa_transformed_rows(case):
    """Bool mask (B, kvN, seq) of key-cache rows written from normed/rotated keys."""
    i = case["inputs"]
    a = case["attrs"]
    pk = i["present_key"]
    B, S = i["query"].shape[:2]
    m = np.zeros(pk.shape[:3], bool)
    if not (a["do_rotary"] or i.get("q_norm_weight") is not None):
        return m
    total = i["seqlens_k"].astype(np.int64) + 1
    cap = pk.shape[2]
    for b in range(B):
        past = int(total[b]) - S if i.get("past_key") is not None else 0
        if a.get("sliding_window_cache"):
            held = min(past, cap)
            past = held - max(0, held + S - cap)      # rows kept before the new ones
        m[b, :, past:past + S] = True
    return m


# ---------------------------------------------------------------------------
# DecoderMaskedMultiHeadAttention
# ---------------------------------------------------------------------------
def dmmha_oracle(case):
    i = dict(case["inputs"])
    a = dict(case["attrs"])
    a.pop("past_present_share_buffer", None)
    return oracle.dmmha(i.pop("query"), i.pop("key"), i.pop("value"), **i, **a)


def dmmha_gpu(case):
    import kv_cache_transformer_amd as kv
    i = case["inputs"]
    a = case["attrs"]
    t = {k: dev(v) for k, v in i.items()}
    out, qk = kv.decode_mha(t["query"], t["key"], t["value"], t.get("mask_index"),
                            t.get("attention_bias"), t.get("past_key"), t.get("past_value"),
                            t.get("past_sequence_length"), num_heads=a["num_heads"],
                            mask_filter_value=a["mask_filter_value"], output_qk=a["output_qk"],
                            past_present_share_buffer=a["past_present_share_buffer"],
                            scale=a["scale"], qk_dtype=case.get("qk_dtype"))
    torch.cuda.synchronize()
    pk = host(t["past_key"]) if "past_key" in t else None
    pv = host(t["past_value"]) if "past_value" in t else None
    return host(out), pk, pv, (host(qk) if qk is not None else None)


# ---------------------------------------------------------------------------
# SparseAttention
# ---------------------------------------------------------------------------
def sparse_oracle(case, query_rows=None):
    i = dict(case["inputs"])
    return oracle.sparse(i.pop("query"), i.pop("key"), i.pop("value"), i.pop("past_key"),
                         i.pop("past_value"), total_sequence_length=case["total_sequence_length"],
                         query_rows=query_rows, **i, **case["attrs"])


def sparse_gpu(case):
    import kv_cache_transformer_amd as kv
    i = case["inputs"]
    a = case["attrs"]
    t = {k: dev(v) for k, v in i.items()}
    out = kv.sparse_attention(t["query"], t.get("key"), t.get("value"), t["past_key"],
                              t["past_value"], t["block_row_indices"], t["block_col_indices"],
                              case["total_sequence_length"], t["key_total_sequence_lengths"],
                              t.get("cos_cache"), t.get("sin_cache"), num_heads=a["num_heads"],
                              kv_num_heads=a["kv_num_heads"],
                              sparse_block_size=a["sparse_block_size"], do_rotary=a["do_rotary"],
                              rotary_interleaved=a["rotary_interleaved"], scale=a["scale"])
    torch.cuda.synchronize()
    return host(out), host(t["past_key"]), host(t["past_value"])


# ---------------------------------------------------------------------------
# PackedAttention
# ---------------------------------------------------------------------------
def packed_oracle(case, sequences=None):
    i = dict(case["inputs"])
    return oracle.packed(i.pop("input"), i.pop("weights"), i.pop("bias"), i.pop("token_offset"),
                         i.pop("cumulative_sequence_length"), sequences=sequences, **i,
                         **case["attrs"])


def packed_gpu(case):
    import kv_cache_transformer_amd as kv
    i = case["inputs"]
    a = case["attrs"]
    t = {k: dev(v) for k, v in i.items()}
    out = kv.packed_attention(t["input"], t["weights"], t["bias"], t["token_offset"],
                              t["cumulative_sequence_length"], t.get("attention_bias"),
                              num_heads=a["num_heads"], scale=a["scale"])
    torch.cuda.synchronize()
    return host(out)
