"""Pins of the DecoderMaskedMultiHeadAttention, SparseAttention and
PackedAttention oracles: brute force, torch float64 SDPA on the CPU, special
cases that reduce to plain attention, and invariants.  CPU only."""

import numpy as np
import pytest
import torch

import oracle
from oracle.brute import brute_dmmha, brute_packed, brute_sparse
from kv_cache_transformer_amd import workloads as wl


def _dm(case, **kw):
    i = dict(case["inputs"])
    a = dict(case["attrs"])
    a.pop("past_present_share_buffer", None)
    a.update(kw)
    return oracle.dmmha(i.pop("query"), i.pop("key"), i.pop("value"), **i, **a)


def _dm_brute(case):
    i = dict(case["inputs"])
    a = dict(case["attrs"])
    a.pop("past_present_share_buffer", None)
    return brute_dmmha(i.pop("query"), i.pop("key"), i.pop("value"), **i, **a)


# ---------------------------------------------------------------------------
# DecoderMaskedMultiHeadAttention
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mask,bias,dtype", [(False, None, np.float32), (True, None, np.float16),
                                             (True, "full", np.float32), (False, "h1", np.float16),
                                             (True, "b1", np.float32)])
def test_dmmha_self_matches_brute(mask, bias, dtype):
    rng = np.random.default_rng(30)
    case = wl.dmmha_self_case(rng, B=2, N=3, H=8, cap=9, past_len=5, dtype=dtype, mask=mask,
                              bias=bias, mask_filter_value=-3.0)
    o, pk, pv, _ = _dm(case)
    ob, pkb, pvb, _ = _dm_brute(case)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(pk, pkb)
    np.testing.assert_array_equal(pv, pvb)
    # the append writes one row; all the others still hold the past cache
    keep = np.ones(9, bool)
    keep[5] = False
    np.testing.assert_array_equal(pk[:, :, keep], case["inputs"]["past_key"][:, :, keep])


@pytest.mark.parametrize("mask,output_qk", [(False, 1), (True, 1), (True, 0)])
def test_dmmha_cross_matches_brute(mask, output_qk):
    rng = np.random.default_rng(31)
    case = wl.dmmha_cross_case(rng, B=2, N=2, H=8, kv_len=6, dtype=np.float32, mask=mask,
                               output_qk=output_qk, mask_filter_value=-2.0)
    o, _, _, qk = _dm(case)
    ob, _, _, qkb = _dm_brute(case)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-13)
    if output_qk:
        np.testing.assert_allclose(qk, qkb, rtol=1e-12, atol=1e-13)
    else:
        assert qk is None


def test_dmmha_all_zero_mask_equals_no_mask():
    # the mask is additive: an all-zero mask shifts every score equally and
    # cancels; dropping masked keys instead would leave nothing to attend.
    rng = np.random.default_rng(32)
    case = wl.dmmha_self_case(rng, B=2, N=2, H=8, cap=8, past_len=6, dtype=np.float32, mask=True)
    case["inputs"]["mask_index"][...] = 0
    o_zero, _, _, _ = _dm(case)
    i = dict(case["inputs"])
    i.pop("mask_index")
    o_none, _, _, _ = _dm(dict(case, inputs=i))
    # a shift of 1e4 costs ~1e-12 of absolute score precision in float64
    np.testing.assert_allclose(o_zero, o_none, rtol=1e-9, atol=1e-12)


def test_dmmha_single_zero_entry_closed_form():
    rng = np.random.default_rng(33)
    case = wl.dmmha_self_case(rng, B=1, N=1, H=4, cap=4, past_len=2, dtype=np.float32, mask=True,
                              mask_filter_value=-1.0)
    case["inputs"]["mask_index"][...] = 1
    case["inputs"]["mask_index"][0, 1] = 0
    o, pk, pv, _ = _dm(case)
    q = case["inputs"]["query"].astype(np.float64).reshape(4)
    x = 0.5 * (pk[0, 0, :3].astype(np.float64) @ q)
    x[1] -= 1.0
    p = np.exp(x - x.max())
    p /= p.sum()
    np.testing.assert_allclose(o[0, 0], p @ pv[0, 0, :3].astype(np.float64), rtol=1e-13)


def test_dmmha_self_equals_gqa_mha_on_same_cache():
    rng = np.random.default_rng(34)
    B, N, H, cap, P = 2, 4, 8, 12, 7
    case = wl.dmmha_self_case(rng, B=B, N=N, H=H, cap=cap, past_len=P, dtype=np.float16)
    o, pk, pv, _ = _dm(case)
    i = case["inputs"]
    og, pkg, pvg = oracle.gqa(i["query"], i["key"], i["value"],
                              seqlens_k=np.full(B, P, np.int32), total_sequence_length=P + 1,
                              past_key=i["past_key"], past_value=i["past_value"],
                              present_key=i["past_key"], present_value=i["past_value"],
                              num_heads=N, kv_num_heads=N)
    np.testing.assert_allclose(o, og, rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(pk, pkg)
    np.testing.assert_array_equal(pv, pvg)


def test_dmmha_cross_matches_torch_sdpa():
    rng = np.random.default_rng(35)
    case = wl.dmmha_cross_case(rng, B=2, N=3, H=16, kv_len=11, dtype=np.float32)
    o, _, _, _ = _dm(case)
    i = case["inputs"]
    q = torch.tensor(i["query"].astype(np.float64)).view(2, 1, 3, 16).transpose(1, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, torch.tensor(i["key"].astype(np.float64)), torch.tensor(i["value"].astype(np.float64)))
    np.testing.assert_allclose(o.reshape(2, 1, 3, 16).transpose(0, 2, 1, 3), ref.numpy(),
                               rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# SparseAttention
# ---------------------------------------------------------------------------

def _sp(case, **kw):
    i = dict(case["inputs"])
    a = dict(case["attrs"])
    a.update(kw)
    return oracle.sparse(i.pop("query"), i.pop("key"), i.pop("value"), i.pop("past_key"),
                         i.pop("past_value"), total_sequence_length=case["total_sequence_length"],
                         **i, **a)


def _sp_brute(case):
    i = dict(case["inputs"])
    return brute_sparse(i.pop("query"), i.pop("key"), i.pop("value"), i.pop("past_key"),
                        i.pop("past_value"), total_sequence_length=case["total_sequence_length"],
                        **i, **case["attrs"])


@pytest.mark.parametrize("rot,inter,rot_dim,packed,past,bs", [
    (False, 0, None, False, None, 2), (True, 0, None, False, None, 2),
    (True, 1, None, False, None, 4), (True, 0, 4, False, None, 2),
    (True, 1, 4, True, None, 2), (False, 0, None, True, [2, 3], 2),
    (True, 0, None, False, [1, 4], 4),
])
def test_sparse_matches_brute(rot, inter, rot_dim, packed, past, bs):
    rng = np.random.default_rng(40)
    case = wl.sparse_case(rng, B=2, S=5, N=4, kvN=2, H=8, bs=bs, dtype=np.float32, cap=10,
                          past_lens=past, rotary=rot, rot_dim=rot_dim, interleaved=inter,
                          packed_qkv=packed, key_total=[5, 4] if past is None else None)
    o, pk, pv = _sp(case)
    ob, pkb, pvb = _sp_brute(case)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(pk, pkb)
    np.testing.assert_array_equal(pv, pvb)


def test_sparse_full_lower_triangle_equals_causal_gqa():
    rng = np.random.default_rng(41)
    B, S, N, kvN, H, bs = 2, 12, 4, 2, 8, 4
    nb = S // bs
    rp = np.zeros((1, nb + 1), np.int32)
    cols = []
    for r in range(nb):
        rp[0, r + 1] = rp[0, r] + r + 1
        cols += list(range(r + 1))
    layouts = (rp, np.array([cols], np.int32))
    case = wl.sparse_case(rng, B=B, S=S, N=N, kvN=kvN, H=H, bs=bs, dtype=np.float16,
                          layouts=layouts, rotary=True)
    o, pk, pv = _sp(case)
    i = case["inputs"]
    og, pkg, pvg = oracle.gqa(i["query"], i["key"], i["value"],
                              seqlens_k=np.full(B, S - 1, np.int32), total_sequence_length=S,
                              present_key=np.zeros_like(i["past_key"]),
                              present_value=np.zeros_like(i["past_value"]),
                              cos_cache=i["cos_cache"], sin_cache=i["sin_cache"],
                              num_heads=N, kv_num_heads=kvN, do_rotary=1)
    np.testing.assert_allclose(o, og, rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(pk, pkg)


def test_sparse_identical_layouts_equal_one_layout_and_csr_expansion():
    rng = np.random.default_rng(42)
    B, S, N, kvN, H, bs = 1, 16, 4, 1, 8, 4
    rp, cols = wl.local_vertical_layouts(1, S // bs, local=2, stride=3)
    case1 = wl.sparse_case(rng, B=B, S=S, N=N, kvN=kvN, H=H, bs=bs, dtype=np.float32,
                           layouts=(rp, cols))
    o1, _, _ = _sp(case1)
    i4 = dict(case1["inputs"], block_row_indices=np.repeat(rp, 4, 0),
              block_col_indices=np.repeat(cols, 4, 0))
    o4, _, _ = _sp(dict(case1, inputs=i4))
    np.testing.assert_array_equal(o1, o4)
    # garbage in the padding past a row's count is ignored
    cols_g = cols.copy()
    cols_g = np.concatenate([cols_g, np.full((1, 3), 99, np.int32)], axis=1)
    og, _, _ = _sp(dict(case1, inputs=dict(case1["inputs"], block_col_indices=cols_g)))
    np.testing.assert_array_equal(o1, og)
    # expansion of the CSR layout into an elementwise mask, then torch SDPA
    i = case1["inputs"]
    dense = np.zeros((S, S), bool)
    for r in range(S // bs):
        for c in cols[0, rp[0, r]:rp[0, r + 1]]:
            dense[r * bs:(r + 1) * bs, c * bs:(c + 1) * bs] = True
    dense &= np.tril(np.ones((S, S), bool))
    q = torch.tensor(i["query"].astype(np.float64)).view(S, N, H).transpose(0, 1)
    k = torch.tensor(i["key"].astype(np.float64)).view(S, 1, H).transpose(0, 1)
    v = torch.tensor(i["value"].astype(np.float64)).view(S, 1, H).transpose(0, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=torch.tensor(dense))
    np.testing.assert_allclose(o1[0].reshape(S, N, H).transpose(1, 0, 2), ref.numpy(),
                               rtol=1e-12, atol=1e-14)


def test_sparse_layouts_cycle_over_heads():
    rng = np.random.default_rng(43)
    B, S, N, kvN, H, bs = 1, 8, 4, 4, 4, 2
    rp, cols = wl.local_vertical_layouts(2, S // bs, local=1, stride=2)
    case = wl.sparse_case(rng, B=B, S=S, N=N, kvN=kvN, H=H, bs=bs, dtype=np.float32,
                          layouts=(rp, cols))
    o, _, _ = _sp(case)
    for h in range(N):
        one = dict(case["inputs"], block_row_indices=rp[h % 2:h % 2 + 1],
                   block_col_indices=cols[h % 2:h % 2 + 1])
        oh, _, _ = _sp(dict(case, inputs=one))
        np.testing.assert_array_equal(o[..., h * H:(h + 1) * H], oh[..., h * H:(h + 1) * H])


def test_csr_visible_blocks():
    rp = np.array([[0, 1, 3, 3]], np.int32)
    cols = np.array([[0, 1, 0, 7]], np.int32)
    assert oracle.csr_visible_blocks(rp, cols, 0, 0) == {0}
    assert oracle.csr_visible_blocks(rp, cols, 0, 1) == {0, 1}
    assert oracle.csr_visible_blocks(rp, cols, 0, 2) == set()


# ---------------------------------------------------------------------------
# PackedAttention
# ---------------------------------------------------------------------------

def _pk(case, **kw):
    i = dict(case["inputs"])
    a = dict(case["attrs"])
    a.update(kw)
    return oracle.packed(i.pop("input"), i.pop("weights"), i.pop("bias"), i.pop("token_offset"),
                         i.pop("cumulative_sequence_length"), **i, **a)


@pytest.mark.parametrize("bias_attn", [None, "full", "b1", "h1", "11"])
def test_packed_matches_brute(bias_attn):
    rng = np.random.default_rng(50)
    case = wl.packed_case(rng, lengths=[3, 1, 4], padded_seq=5, D=6, N=2, H=4,
                          dtype=np.float32, bias_attn=bias_attn, wstd=0.5)
    o = _pk(case)
    i = dict(case["inputs"])
    ob = brute_packed(i.pop("input"), i.pop("weights"), i.pop("bias"), i.pop("token_offset"),
                      i.pop("cumulative_sequence_length"), **i, **case["attrs"])
    np.testing.assert_allclose(o, ob, rtol=1e-11, atol=1e-13)


def test_packed_equals_per_sequence_sdpa_and_padded_bias_gather():
    rng = np.random.default_rng(51)
    lengths = [5, 2, 7]
    case = wl.packed_case(rng, lengths=lengths, padded_seq=8, D=16, N=2, H=8,
                          dtype=np.float32, bias_attn="full", wstd=0.3)
    o = _pk(case)
    i = case["inputs"]
    qkv = i["input"].astype(np.float64) @ i["weights"].astype(np.float64) + i["bias"].astype(np.float64)
    cum = i["cumulative_sequence_length"]
    for b in range(3):
        t0, t1 = cum[b], cum[b + 1]
        L = t1 - t0
        q = torch.tensor(qkv[t0:t1, :16]).view(L, 2, 8).transpose(0, 1)
        k = torch.tensor(qkv[t0:t1, 16:32]).view(L, 2, 8).transpose(0, 1)
        v = torch.tensor(qkv[t0:t1, 32:]).view(L, 2, 8).transpose(0, 1)
        # generator schedules: padded position of token t is t - cum[b]
        bias = torch.tensor(i["attention_bias"][b, :, :L, :L].astype(np.float64))
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=bias)
        np.testing.assert_allclose(o[t0:t1].reshape(L, 2, 8).transpose(1, 0, 2), ref.numpy(),
                                   rtol=1e-12, atol=1e-14)


def test_packed_single_sequence_is_plain_mha():
    rng = np.random.default_rng(52)
    case = wl.packed_case(rng, lengths=[6], padded_seq=6, D=8, N=2, H=4, dtype=np.float32,
                          wstd=0.4)
    o = _pk(case)
    i = case["inputs"]
    qkv = i["input"].astype(np.float64) @ i["weights"].astype(np.float64) + i["bias"].astype(np.float64)
    og, _, _ = oracle.gqa(qkv[None, :, :8], qkv[None, :, 8:16], qkv[None, :, 16:],
                          seqlens_k=np.array([5], np.int32), total_sequence_length=6,
                          present_key=np.zeros((1, 2, 6, 4)), present_value=np.zeros((1, 2, 6, 4)),
                          num_heads=2, kv_num_heads=2, causal=0)
    np.testing.assert_allclose(o, og[0], rtol=1e-13, atol=1e-15)


def test_packed_schedule_and_qkv_sizes():
    tok, cum = wl.packed_schedule_inputs([2, 0, 3], 4)
    seq, pos = oracle.packed_schedule(cum, 5)
    np.testing.assert_array_equal(seq, [0, 0, 2, 2, 2])
    np.testing.assert_array_equal(pos, [0, 1, 0, 1, 2])
    np.testing.assert_array_equal(tok.reshape(-1)[:5], [0, 1, 8, 9, 10])
    # explicit qkv_hidden_sizes equal to the default split give the same result
    rng = np.random.default_rng(53)
    case = wl.packed_case(rng, lengths=[3, 2], padded_seq=4, D=4, N=2, H=2, dtype=np.float32)
    o1 = _pk(case)
    o2 = _pk(case, qkv_hidden_sizes=[4, 4, 4])
    np.testing.assert_array_equal(o1, o2)
    # value head size may differ from the query head size
    x = rng.standard_normal((5, 4)).astype(np.float32)
    w = rng.standard_normal((4, 4 + 4 + 6)).astype(np.float32)
    bv = rng.standard_normal(14).astype(np.float32)
    tok, cum = wl.packed_schedule_inputs([3, 2], 4)
    o = oracle.packed(x, w, bv, tok, cum, num_heads=2, qkv_hidden_sizes=[4, 4, 6])
    ob = brute_packed(x, w, bv, tok, cum, num_heads=2, qkv_hidden_sizes=[4, 4, 6])
    assert o.shape == (5, 6)
    np.testing.assert_allclose(o, ob, rtol=1e-11, atol=1e-13)
