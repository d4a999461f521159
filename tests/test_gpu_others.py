"""GPU parity of decode_mha, sparse_attention and packed_attention against the
oracle, small cases plus the named sparse and packed workloads at full size,
every output element compared."""

import numpy as np
import pytest
import torch

import oracle
from kv_cache_transformer_amd import workloads as wl

from gpu_util import (check_cache, check_output, dev, dmmha_gpu, dmmha_oracle, host, packed_gpu,
                      packed_oracle, sparse_gpu, sparse_oracle)

pytestmark = pytest.mark.gpu

F16, F32 = np.float16, np.float32

# ---------------------------------------------------------------------------
# DecoderMaskedMultiHeadAttention
# ---------------------------------------------------------------------------
DMMHA_SELF = [
    dict(dtype=F16, B=2, N=4, H=64, cap=300, past_len=299),
    dict(dtype=F32, B=3, N=2, H=128, cap=40, past_len=17, mask=True, bias="full"),
    dict(dtype=F16, B=1, N=8, H=128, cap=2000, past_len=1500, mask=True,
         mask_filter_value=-3.0, bias="h1", scale=0.2),
    dict(dtype=F16, B=2, N=2, H=16, cap=8, past_len=0),
]
DMMHA_CROSS = [
    dict(dtype=F16, B=2, N=2, H=16, kv_len=1, output_qk=1),
    dict(dtype=F32, B=2, N=4, H=64, kv_len=77, mask=True, output_qk=1, mask_filter_value=-5.0),
    dict(dtype=F16, B=1, N=8, H=128, kv_len=1500, mask=True, output_qk=0),
    # qk in the other type (the page's QK type is float32 or float16, apart from T)
    dict(dtype=F16, B=2, N=4, H=64, kv_len=300, mask=True, output_qk=1, qk_dtype=F32),
    dict(dtype=F32, B=1, N=2, H=128, kv_len=50, output_qk=1, qk_dtype=F16),
]


@pytest.mark.parametrize("idx", range(len(DMMHA_SELF)))
def test_dmmha_self_parity(idx):
    spec = dict(DMMHA_SELF[idx])
    print(f"dmmha self {idx}: {spec}", flush=True)
    dtype = spec.pop("dtype")
    case = wl.dmmha_self_case(np.random.default_rng(400 + idx), dtype=dtype, **spec)
    out, pk, pv, _ = dmmha_gpu(case)
    ref, rpk, rpv, _ = dmmha_oracle(case)
    check_output(out, ref, dtype)
    check_cache(pk, rpk, None, "present_key")
    check_cache(pv, rpv, None, "present_value")


@pytest.mark.parametrize("idx", range(len(DMMHA_CROSS)))
def test_dmmha_cross_parity(idx):
    spec = dict(DMMHA_CROSS[idx])
    print(f"dmmha cross {idx}: {spec}", flush=True)
    dtype = spec.pop("dtype")
    qk_dtype = spec.pop("qk_dtype", dtype)
    case = wl.dmmha_cross_case(np.random.default_rng(500 + idx), dtype=dtype, **spec)
    case["qk_dtype"] = {F16: torch.float16, F32: torch.float32}[qk_dtype]
    out, _, _, qk = dmmha_gpu(case)
    ref, _, _, rqk = dmmha_oracle(case)
    check_output(out, ref, dtype)
    if spec.get("output_qk"):
        assert qk.dtype == qk_dtype
        check_output(qk, rqk, qk_dtype, "qk")


def test_dmmha_all_zero_mask_matches_unmasked():
    case = wl.dmmha_self_case(np.random.default_rng(450), B=2, N=4, H=64, cap=64, past_len=40,
                              dtype=F32, mask=True, mask_filter_value=-7.0)
    case["inputs"]["mask_index"][...] = 0
    out_z, _, _, _ = dmmha_gpu(case)
    i = dict(case["inputs"])
    i.pop("mask_index")
    case2 = dict(case, inputs=i)
    out_n, _, _, _ = dmmha_gpu(case2)
    check_output(out_z, out_n.astype(np.float64), F32, "all-zero mask vs none")


# ---------------------------------------------------------------------------
# SparseAttention
# ---------------------------------------------------------------------------
SPARSE = [
    dict(dtype=F16, B=2, S=256, N=8, kvN=2, H=64, bs=64, rotary=True),
    dict(dtype=F16, B=1, S=200, N=4, kvN=2, H=128, bs=16, rotary=True, interleaved=1),
    dict(dtype=F32, B=2, S=96, N=4, kvN=4, H=64, bs=32, rotary=True, rot_dim=32),
    dict(dtype=F16, B=1, S=300, N=8, kvN=2, H=128, bs=128, packed_qkv=True),
    dict(dtype=F16, B=2, S=130, N=4, kvN=1, H=64, bs=64, key_total=[130, 77], rotary=True),
    dict(dtype=F32, B=1, S=64, N=2, kvN=1, H=8, bs=16, packed_qkv=True),
    dict(dtype=F16, B=1, S=100, N=4, kvN=2, H=32, bs=32, rotary=True, rot_dim=16,
         interleaved=1),
]


# token generation (total_sequence_length != S): the new rows follow a past
# of key_total - S rows in the in-place cache
SPARSE_GEN = [
    dict(dtype=F16, B=2, S=1, N=8, kvN=2, H=64, bs=64, cap=512, past_lens=[300, 511], rotary=True),
    dict(dtype=F16, B=1, S=37, N=4, kvN=2, H=128, bs=16, cap=400, past_lens=[200], rotary=True,
         interleaved=1),
    dict(dtype=F32, B=2, S=5, N=4, kvN=4, H=64, bs=32, cap=256, past_lens=[3, 100]),
    dict(dtype=F16, B=1, S=1, N=8, kvN=2, H=128, bs=128, cap=1000, past_lens=[999],
         packed_qkv=True, rotary=True, rot_dim=64),
    dict(dtype=F32, B=3, S=1, N=4, kvN=1, H=64, bs=16, cap=300, past_lens=[5, 299, 100],
         rotary=True, rot_dim=32, interleaved=1),
    dict(dtype=F16, B=1, S=1, N=16, kvN=4, H=256, bs=32, cap=2000, past_lens=[1234]),
    dict(dtype=F16, B=80, S=1, N=4, kvN=2, H=64, bs=16, cap=128,
         past_lens=list(range(3, 128, 2)) + [0] * 17, rotary=True),
]


@pytest.mark.parametrize("idx", range(len(SPARSE_GEN)))
def test_sparse_generation_parity(idx):
    spec = dict(SPARSE_GEN[idx])
    print(f"sparse generation {idx}: {spec}", flush=True)
    dtype = spec.pop("dtype")
    case = wl.sparse_case(np.random.default_rng(650 + idx), dtype=dtype, **spec)
    out, pk, pv = sparse_gpu(case)
    ref, rpk, rpv = sparse_oracle(case)
    check_output(out, ref, dtype)
    tr = np.zeros(pk.shape[:3], bool)
    if spec.get("rotary"):
        for b, past in enumerate(spec["past_lens"]):
            tr[b, :, past:past + spec["S"]] = True
    check_cache(pk, rpk, tr, "key cache")
    check_cache(pv, rpv, None, "value cache")


def test_sparse_generation_wide_column_list():
    # one generated token whose column list is padded past 4096 entries:
    # the block-sparse flash route serves it (the decode route's block table
    # would not fit LDS); the padding is never read
    spec = dict(SPARSE_GEN[0])
    dtype = spec.pop("dtype")
    case = wl.sparse_case(np.random.default_rng(650), dtype=dtype, **spec)
    i = case["inputs"]
    cols = i["block_col_indices"]
    i["block_col_indices"] = np.concatenate(
        [cols, np.full((cols.shape[0], 4100 - cols.shape[1]), 7, np.int32)], axis=1)
    out, pk, pv = sparse_gpu(case)
    ref, rpk, rpv = sparse_oracle(case)
    check_output(out, ref, dtype)
    check_cache(pv, rpv, None, "value cache")


@pytest.mark.parametrize("idx", range(len(SPARSE)))
def test_sparse_parity(idx):
    spec = dict(SPARSE[idx])
    print(f"sparse {idx}: {spec}", flush=True)
    dtype = spec.pop("dtype")
    case = wl.sparse_case(np.random.default_rng(600 + idx), dtype=dtype, **spec)
    out, pk, pv = sparse_gpu(case)
    ref, rpk, rpv = sparse_oracle(case)
    check_output(out, ref, dtype)
    tr = np.zeros(pk.shape[:3], bool)
    if spec.get("rotary"):
        tr[:, :, :spec["S"]] = True
    check_cache(pk, rpk, tr, "key cache")
    check_cache(pv, rpv, None, "value cache")


def test_sparse_garbage_padding_and_column_order():
    rng = np.random.default_rng(650)
    case = wl.sparse_case(rng, B=1, S=128, N=4, kvN=2, H=64, bs=32, dtype=F16)
    rp, cols = case["inputs"]["block_row_indices"], case["inputs"]["block_col_indices"]
    cols2 = np.concatenate([cols, np.full((cols.shape[0], 5), 3, np.int32)], axis=1)
    for l in range(rp.shape[0]):             # reverse each row's columns
        for r in range(rp.shape[1] - 1):
            lo, hi = rp[l, r], rp[l, r + 1]
            cols2[l, lo:hi] = cols2[l, lo:hi][::-1]
    case2 = dict(case, inputs=dict(case["inputs"], block_col_indices=cols2))
    out, _, _ = sparse_gpu(case2)
    ref, _, _ = sparse_oracle(case)
    check_output(out, ref, F16)


def test_workload_sparse_prompt():
    """The block-sparse prompt at full size (B2 S8192 N32 kvN8 H128, block
    64, four layouts, rotary): every output element and every cache row
    against the oracle, which runs over row chunks in child processes."""
    from oracle import pool as oracle_pool
    case = wl.sparse_prompt()
    print("sparse_prompt: GPU call, then the oracle over 16 row chunks", flush=True)
    out, pk, pv = sparse_gpu(case)
    ref, rpk, rpv = oracle_pool.sparse_full("sparse_prompt", 8192)
    err = check_output(out, ref, F16)
    tr = np.ones(pk.shape[:3], bool)
    n1 = check_cache(pk, rpk, tr, "key cache")
    check_cache(pv, rpv, None, "value cache")
    print(f"max |d| {err:.3g}; rotated key elements off by 1 ulp: {n1} of {pk.size}")


def test_sparse_empty_batch():
    case = wl.sparse_case(np.random.default_rng(1), B=0, S=64, N=4, kvN=2, H=64, bs=16, dtype=F16)
    out, pk, pv = sparse_gpu(case)
    ref, rpk, rpv = sparse_oracle(case)
    assert out.shape == ref.shape == (0, 64, 4 * 64) and pk.shape == rpk.shape


def test_workload_sparse_generation():
    case = wl.sparse_generation()
    print("sparse_generation", flush=True)
    out, pk, pv = sparse_gpu(case)
    ref, rpk, rpv = sparse_oracle(case)
    check_output(out, ref, F16)
    tr = np.zeros(pk.shape[:3], bool)
    tr[:, :, 8191] = True                      # the new (rotated) key row
    check_cache(pk, rpk, tr, "key cache")
    check_cache(pv, rpv, None, "value cache")


# ---------------------------------------------------------------------------
# PackedAttention
# ---------------------------------------------------------------------------
PACKED = [
    dict(dtype=F16, lengths=[5, 130, 64, 1], padded_seq=160, D=64, N=2, H=64),
    dict(dtype=F32, lengths=[33, 70], padded_seq=80, D=48, N=4, H=32, bias_attn="full"),
    dict(dtype=F16, lengths=[200, 0, 17], padded_seq=256, D=128, N=3, H=128, bias_attn="h1"),
    dict(dtype=F16, lengths=[2, 1], padded_seq=4, D=8, N=1, H=8, wstd=0.3),
    # an input hidden size with a partial last k step of the projection, over
    # several k steps and two row tiles
    dict(dtype=F16, lengths=[300, 45, 129], padded_seq=320, D=104, N=2, H=64),
    dict(dtype=F32, lengths=[70, 3], padded_seq=96, D=72, N=2, H=32),
]


@pytest.mark.parametrize("idx", range(len(PACKED)))
def test_packed_parity(idx):
    spec = dict(PACKED[idx])
    print(f"packed {idx}: {spec}", flush=True)
    dtype = spec.pop("dtype")
    case = wl.packed_case(np.random.default_rng(700 + idx), dtype=dtype, **spec)
    out = packed_gpu(case)
    ref = packed_oracle(case)
    check_output(out, ref, dtype)


def test_packed_schedule_bit_exact():
    import kv_cache_transformer_amd as kv
    lengths = np.array([5, 0, 300, 128, 129, 1, 256])
    tok, cum = wl.packed_schedule_inputs(lengths, 300)
    T = int(lengths.sum())
    bounds, work, seq, pos = kv.packed_schedule(dev(cum), T, 300, tile_rows=128)
    torch.cuda.synchronize()
    rseq, rpos = oracle.packed_schedule(cum, T)
    np.testing.assert_array_equal(host(seq), rseq)
    np.testing.assert_array_equal(host(pos), rpos)
    np.testing.assert_array_equal(host(bounds), np.stack([cum[:-1], cum[1:]], 1))
    w = host(work)
    n = int(w[0])
    items = [tuple(x) for x in w[1:1 + 2 * n].reshape(n, 2)]
    # unique: the set of (sequence, tile) items covering every token once
    expect = {(b, t) for b in range(len(lengths)) for t in range(-(-int(lengths[b]) // 128))}
    assert set(items) == expect and len(items) == len(expect)
    # order: non-increasing sequence length, ties by index
    keys = [(-int(lengths[b]), b) for b, _ in items]
    assert keys == sorted(keys)


def test_workload_packed_varlen():
    """The packed varlen workload at full size (64 sequences, T = 16936):
    every output element of every sequence against the oracle."""
    case = wl.packed_varlen()
    out = packed_gpu(case)
    ref = packed_oracle(case)
    err = check_output(out, ref, F16)
    print(f"max |d| {err:.3g} over {out.size} elements")
