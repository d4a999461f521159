"""GPU parity of gqa_attention (prefill and decode paths) against the oracle.

Small cases span several key tiles, ragged tails and every feature; the named
workloads run at full size with every output element compared (the long
prefill's oracle runs over row chunks in child processes)."""

import numpy as np
import pytest

from kv_cache_transformer_amd import workloads as wl

from gpu_util import (check_cache, check_output, check_quant_gqa, gqa_gpu, gqa_oracle,
                      gqa_transformed_rows)

pytestmark = pytest.mark.gpu

F16, F32 = np.float16, np.float32

PREFILL = [
    dict(dtype=F16, B=2, S=150, N=8, kvN=2, H=64),
    dict(dtype=F32, B=1, S=128, N=8, kvN=2, H=64, scale=0.125),
    dict(dtype=F16, B=2, S=200, N=8, kvN=2, H=128, window=37, softcap=30.0, sink=True,
         norm=True, rotary=True),
    dict(dtype=F16, B=1, S=97, N=4, kvN=4, H=128, bias="full", smooth_softmax=1),
    dict(dtype=F16, B=2, S=70, N=6, kvN=3, H=64, bias="h1", window=0),
    dict(dtype=F32, B=2, S=90, N=4, kvN=1, H=128, rotary=True, norm=True, window=20,
         softcap=10.0, sink=True),
    dict(dtype=F16, B=2, S=100, N=8, kvN=2, H=64, causal=0, total_lens=[60, 100], bias="b1"),
    dict(dtype=F16, B=2, S=40, N=8, kvN=2, H=128, past="shared", cap=300, past_lens=[0, 200],
         rotary=True, window=64),
    dict(dtype=F32, B=2, S=17, N=4, kvN=2, H=64, past="concat", cap=60, past_lens=[5, 30],
         bias="full"),
    dict(dtype=F16, B=1, S=80, N=4, kvN=1, H=256, sink=True),
    dict(dtype=F16, B=1, S=50, N=4, kvN=2, H=72, rotary=True),
    dict(dtype=F16, B=2, S=9, N=2, kvN=1, H=8),
    dict(dtype=F32, B=1, S=40, N=2, kvN=1, H=256, window=5),
    dict(dtype=F16, B=2, S=64, N=8, kvN=2, H=128, total_lens=[40, 64]),
    dict(dtype=F16, B=1, S=130, N=6, kvN=2, H=64, softcap=5.0),
    dict(dtype=F16, B=1, S=33, N=32, kvN=1, H=64, scale=-0.3),
    dict(dtype=F16, B=1, S=1, N=8, kvN=2, H=128, rotary=True),
    # windows without softcap or bias: the per-lane key-offset masks of the
    # pipelined kernel, tiles partly visible to a workgroup's rows
    dict(dtype=F16, B=2, S=300, N=8, kvN=2, H=128, window=90),
    dict(dtype=F16, B=1, S=257, N=4, kvN=1, H=64, window=40, rotary=True),
    # more samples than a persistent prompt workgroup copies lengths of (1024)
    dict(dtype=F16, B=1100, S=3, N=2, kvN=1, H=64, past="shared", cap=12, rotary=True),
]

DECODE = [
    dict(dtype=F16, B=3, N=32, kvN=8, H=128, cap=600, past_lens=[1, 300, 599], rotary=True),
    dict(dtype=F32, B=2, N=8, kvN=2, H=64, cap=200, past_lens=[0, 150]),
    dict(dtype=F16, B=2, N=4, kvN=4, H=256, cap=1100, past_lens=[1099, 513], softcap=20.0,
         sink=True, window=100),
    dict(dtype=F16, B=1, N=32, kvN=1, H=64, cap=300, past_lens=[299], norm=True, rotary=True,
         bias="full"),
    dict(dtype=F16, B=2, N=8, kvN=2, H=128, past="concat", cap=151, past_lens=[150, 7]),
    dict(dtype=F32, B=1, N=16, kvN=2, H=128, cap=5000, past_lens=[4999], smooth_softmax=1),
    dict(dtype=F16, B=2, N=2, kvN=1, H=8, cap=8, past_lens=[7, 3]),
    dict(dtype=F16, B=4, N=16, kvN=4, H=128, cap=2100, past_lens=[2099, 1024, 128, 127],
         bias="h1", sink=True),
    # more than 64 samples: the deal scans the lengths in several 64-lane passes
    dict(dtype=F16, B=150, N=8, kvN=2, H=64, cap=96, rotary=True, past="shared"),
    dict(dtype=F32, B=70, N=4, kvN=4, H=64, cap=40, window=7, past="concat"),
]


def _case(spec, seed):
    spec = dict(spec)
    dtype = spec.pop("dtype")
    past = spec.pop("past", None)
    if "past_lens" in spec and past is None:
        past = "shared"
    rng = np.random.default_rng(seed)
    return wl.gqa_case(rng, dtype=dtype, past=past, **spec)


def _compare(case, rows=None):
    dtype = case["inputs"]["query"].dtype
    out, pk, pv = gqa_gpu(case)
    ref, rpk, rpv = gqa_oracle(case, query_rows=rows)
    got = out if rows is None else out[:, rows]
    err = check_output(got, ref, dtype)
    tr = gqa_transformed_rows(case)
    n1 = check_cache(pk, rpk, tr, "present_key")
    check_cache(pv, rpv, None, "present_value")
    return err, n1


@pytest.mark.parametrize("idx", range(len(PREFILL)))
def test_prefill_parity(idx):
    print(f"prefill case {idx}: {PREFILL[idx]}", flush=True)
    _compare(_case(PREFILL[idx], 100 + idx))


# Dense f16 prompts run one workgroup per CU over pairs of row blocks; with
# the (sample, head-group pair) slabs a multiple of eight, each XCD takes its
# own slabs through all row blocks, in several rounds here (38 row blocks x 8
# slabs over at most 256 workgroups).  Every seventh query row is compared.
# A prompt's present cache in its own float type (GroupQueryAttention page,
# Description): the attention reads the new rows in T, the cache holds them
# in its own type.
CACHE_TYPE = [
    dict(dtype=F16, cache_dtype=F32, B=2, S=150, N=8, kvN=2, H=64),
    dict(dtype=F16, cache_dtype=F32, B=2, S=200, N=8, kvN=2, H=128, cap=230, window=37,
         softcap=30.0, sink=True, norm=True, rotary=True),
    dict(dtype=F32, cache_dtype=F16, B=1, S=90, N=4, kvN=1, H=128, rotary=True, norm=True,
         window=20, bias="full"),
    dict(dtype=F32, cache_dtype=F16, B=2, S=64, N=8, kvN=2, H=72, causal=0, total_lens=[40, 64]),
    dict(dtype=F16, cache_dtype=F32, B=1, S=33, N=32, kvN=1, H=256),
]


@pytest.mark.parametrize("idx", range(len(CACHE_TYPE)))
def test_prompt_cache_in_its_own_type(idx):
    print(f"cache type case {idx}: {CACHE_TYPE[idx]}", flush=True)
    case = _case(CACHE_TYPE[idx], 5000 + idx)
    assert case["inputs"]["present_key"].dtype == CACHE_TYPE[idx]["cache_dtype"]
    err, n1 = _compare(case)
    print(f"max |d| {err:.3g}; transformed key elements off: {n1}")


def test_prefill_persistent_rounds():
    case = _case(dict(dtype=F16, B=8, S=1200, N=4, kvN=1, H=64, window=300, rotary=True, norm=True,
                      softcap=20.0), 150)
    _compare(case, rows=np.arange(0, 1200, 7))


@pytest.mark.parametrize("idx", range(len(DECODE)))
def test_decode_parity(idx):
    spec = dict(DECODE[idx])
    spec["S"] = 1
    print(f"decode case {idx}: {spec}", flush=True)
    _compare(_case(spec, 200 + idx))


def test_decode_repeat_is_deterministic():
    case = _case(dict(DECODE[0], S=1), 300)
    o1, _, _ = gqa_gpu(case)
    o2, _, _ = gqa_gpu(case)
    np.testing.assert_array_equal(o1, o2)


# Split-key decode (GroupQueryAttention page, Implementation variants: cached
# decode partitioned along the key axis, partial online-softmax results
# merged): one fixed input at several split targets, from one pair of waves
# per (sample, kv head) unit (no merge) to many pairs per unit, every output
# against the oracle.
SPLITS = [1, 2, 8, 32]


def test_decode_split_count_sweep():
    import kv_cache_transformer_amd as kv
    case = wl.gqa_decode()
    ref, rpk, rpv = gqa_oracle(case)
    outs = {}
    try:
        for w in SPLITS:
            kv.set_decode_split(w)
            print(f"gqa_decode at {w} waves per compute unit", flush=True)
            out, pk, pv = gqa_gpu(case)
            check_output(out, ref, np.float16, f"output at split {w}")
            check_cache(pk, rpk, gqa_transformed_rows(case), "present_key")
            check_cache(pv, rpv, None, "present_value")
            outs[w] = out
    finally:
        kv.set_decode_split(0)
    for w in SPLITS[1:]:
        print(f"split {w} vs 1: {int(np.sum(outs[w] != outs[1]))} elements differ in the last bit(s)")


def test_decode_workspace_reuse_leaves_counters_zero():
    """Decode calls keep per-unit arrival counters in the workspace and leave
    them zero: one zero-filled workspace serves a sequence of calls of
    different shapes, each checked against the oracle."""
    import torch
    ws = torch.zeros(16 << 20, dtype=torch.uint8, device="cuda:0")
    # a prompt whose cache has its own type puts its T rows in the workspace,
    # after the counters: the decode after it still finds them zero
    specs = [(DECODE[0], 310), (DECODE[7], 311), (CACHE_TYPE[0], 313), (DECODE[8], 312),
             (DECODE[0], 310)]
    for spec, seed in specs:
        case = _case(spec if "cache_dtype" in spec else dict(spec, S=1), seed)
        out, _, _ = gqa_gpu(case, workspace=ws)
        ref, _, _ = gqa_oracle(case)
        check_output(out, ref, case["inputs"]["query"].dtype)
        # the first 32 KiB hold the counters (one int32 per split unit); the
        # partials follow them
        assert int(torch.count_nonzero(ws[:32768])) == 0, f"counters left non-zero after {spec}"


def test_decode_split_setting_is_validated():
    import kv_cache_transformer_amd as kv
    with pytest.raises(kv.KvattnError):
        kv.set_decode_split(33)
    assert kv.set_decode_split(0) == 0


def test_workload_gqa_prompt_small():
    case = wl.gqa_prompt_small()
    print("gqa_prompt_small", flush=True)
    _compare(case)


def test_workload_gqa_decode():
    case = wl.gqa_decode()
    print("gqa_decode", flush=True)
    err, n1 = _compare(case)
    print(f"max |d| {err:.3g}; rotated key elements off by 1 ulp: {n1}")


def test_workload_gqa_long_prefill():
    """The long prefill at full size (B4 S4096 N32 kvN8 H128, window 1024,
    softcap, sink, q/k norm, rotary): every output element and every cache
    row against the oracle, which runs over row chunks in child processes."""
    from oracle import pool as oracle_pool
    case = wl.gqa_long_prefill()
    print("gqa_long_prefill: GPU call, then the oracle over 16 row chunks", flush=True)
    out, pk, pv = gqa_gpu(case)
    ref, rpk, rpv = oracle_pool.gqa_full("gqa_long_prefill", 4096)
    err = check_output(out, ref, np.float16)
    n1 = check_cache(pk, rpk, gqa_transformed_rows(case), "present_key")
    check_cache(pv, rpv, None, "present_value")
    print(f"max |d| {err:.3g}; normed+rotated key elements off by 1 ulp: {n1} of {pk.size}")


# Sliding-window cache (GroupQueryAttention page, Attributes table): shared
# buffers of capacity cap hold the most recent tokens; past_lens are the
# tokens seen before the call (above cap, rows are evicted from the front).
WINDOW = [
    dict(dtype=F16, B=3, S=1, N=8, kvN=2, H=128, cap=300, window=200,
         past_lens=[150, 299, 700], rotary=True, norm=True),
    dict(dtype=F16, B=2, S=40, N=8, kvN=2, H=64, cap=120, window=64,
         past_lens=[30, 500], softcap=10.0, sink=True),
    dict(dtype=F16, B=2, S=64, N=8, kvN=2, H=128, cap=200, window=100,
         past_lens=[150, 1000], rotary=True),
    dict(dtype=F32, B=2, S=1, N=4, kvN=2, H=64, cap=64, window=32, past_lens=[10, 100]),
    dict(dtype=F32, B=1, S=17, N=4, kvN=1, H=64, cap=50, window=33, past_lens=[90],
         rotary=True, norm=True),
]


@pytest.mark.parametrize("idx", range(len(WINDOW)))
def test_window_cache_parity(idx):
    case = _case(WINDOW[idx], 3000 + idx)
    case["attrs"]["sliding_window_cache"] = 1
    err, _ = _compare(case)
    assert err >= 0


# The same windows over separate past and present buffers: the rows that
# survive the eviction are copied to the front of the present buffer, the new
# rows follow, and its other rows keep what they held (NaN here).
@pytest.mark.parametrize("idx", range(len(WINDOW)))
def test_window_cache_separate_buffers(idx):
    case = _case(WINDOW[idx], 3100 + idx)
    case["attrs"]["sliding_window_cache"] = 1
    i = case["inputs"]
    fill = np.full_like(i["past_key"], np.nan)
    i["present_key"], i["present_value"] = fill, fill.copy()
    case["shared"] = False
    err, _ = _compare(case)
    assert err >= 0


def test_workload_window_decode():
    """The sliding-window decode workload at full size, every output checked."""
    case = wl.gqa_window_decode()
    err, _ = _compare(case)
    assert err >= 0


# Quantised caches (GroupQueryAttention page, Attributes table: k_quant_type,
# v_quant_type, kv_cache_bit_width; Inputs table: k_scale, v_scale): float32
# activations, int8 and packed int4 caches for prompts and decode.
Q8T = dict(bits=8, k="tensor", v="tensor")
Q8C = dict(bits=8, k="channel", v="channel")
Q4T = dict(bits=4, k="tensor", v="tensor")
Q4C = dict(bits=4, k="channel", v="channel")
QUANT = [
    dict(B=2, S=150, N=8, kvN=2, H=64, quant=Q8T),
    dict(B=2, S=130, N=8, kvN=2, H=128, window=37, softcap=30.0, sink=True, bias="full",
         quant=dict(bits=8, k="channel", v="tensor")),
    dict(B=2, S=100, N=8, kvN=2, H=128, causal=0, total_lens=[60, 100],
         quant=dict(bits=4, k="channel", v="channel")),
    dict(B=1, S=24, N=4, kvN=1, H=64, rotary=True, norm=True,
         quant=dict(bits=4, k="tensor", v="channel")),
    dict(B=1, S=20, N=4, kvN=1, H=128, rotary=True, quant=Q8C),
    dict(B=2, S=9, N=2, kvN=1, H=8, quant=dict(bits=4, k="tensor", v="tensor")),
    # prompts whose attention reads the codes of a cache longer than the
    # prompt: heads narrower than the padded tile, and the widest head
    dict(B=2, S=70, N=4, kvN=2, H=40, cap=100, quant=Q4C),
    dict(B=2, S=33, N=4, kvN=2, H=24, cap=48, total_lens=[20, 33], quant=Q8C),
    dict(B=1, S=40, N=2, kvN=1, H=256, cap=64, softcap=25.0,
         quant=dict(bits=8, k="channel", v="tensor")),
    dict(B=1, S=50, N=2, kvN=2, H=256, cap=50, quant=Q4T),
    # prompts continuing a quantised past (chunked prefill): codes of the
    # past read together with the new rows' codes, in place or copied
    dict(B=2, S=40, N=8, kvN=2, H=128, past="shared", cap=300, past_lens=[0, 200],
         rotary=True, window=64, quant=Q8C),
    dict(B=2, S=17, N=4, kvN=2, H=64, past="concat", cap=60, past_lens=[5, 30], bias="full",
         quant=Q4T),
    dict(B=1, S=33, N=4, kvN=1, H=72, past="shared", cap=100, past_lens=[50], rotary=True,
         norm=True, quant=Q4C),
    dict(B=2, S=64, N=8, kvN=2, H=40, past="concat", cap=200, past_lens=[100, 136], softcap=20.0,
         sink=True, quant=dict(bits=8, k="tensor", v="channel")),
    dict(B=3, S=1, N=32, kvN=8, H=128, cap=600, past_lens=[1, 300, 599], rotary=True, quant=Q8C),
    dict(B=2, S=1, N=8, kvN=2, H=64, past="concat", cap=200, past_lens=[0, 150],
         quant=dict(bits=8, k="tensor", v="channel")),
    dict(B=2, S=1, N=4, kvN=4, H=256, cap=1100, past_lens=[1099, 513], softcap=20.0, sink=True,
         window=100, quant=dict(bits=8, k="channel", v="tensor")),
    dict(B=1, S=1, N=8, kvN=2, H=72, cap=300, past_lens=[299], norm=True, rotary=True, quant=Q8C),
    dict(B=4, S=1, N=16, kvN=4, H=128, cap=2100, past_lens=[2099, 1024, 128, 127], bias="h1",
         smooth_softmax=1, quant=Q8T),
    dict(B=2, S=1, N=2, kvN=1, H=8, cap=8, past_lens=[7, 3], quant=Q8C),
    dict(B=90, S=1, N=8, kvN=2, H=128, cap=64, rotary=True, quant=Q8T, past="shared"),
    # int4 decode: two codes per byte, runs of Hp / 8 dims per lane
    dict(B=3, S=1, N=32, kvN=8, H=128, cap=600, past_lens=[1, 300, 599], rotary=True, quant=Q4C),
    dict(B=2, S=1, N=8, kvN=2, H=64, past="concat", cap=200, past_lens=[0, 150],
         quant=dict(bits=4, k="tensor", v="channel")),
    dict(B=2, S=1, N=4, kvN=4, H=256, cap=1100, past_lens=[1099, 513], softcap=20.0, sink=True,
         window=100, quant=dict(bits=4, k="channel", v="tensor")),
    dict(B=1, S=1, N=8, kvN=2, H=80, cap=300, past_lens=[299], norm=True, rotary=True, quant=Q4C),
    dict(B=1, S=1, N=4, kvN=2, H=192, cap=100, past_lens=[99], rotary=True, quant=Q4T),
    dict(B=4, S=1, N=16, kvN=4, H=128, cap=2100, past_lens=[2099, 1024, 128, 127], bias="h1",
         smooth_softmax=1, quant=Q4T),
    dict(B=2, S=1, N=2, kvN=1, H=8, cap=8, past_lens=[7, 3], quant=Q4C),
    dict(B=70, S=1, N=8, kvN=2, H=128, cap=64, rotary=True, quant=Q4T, past="shared"),
]


@pytest.mark.parametrize("idx", range(len(QUANT)))
def test_quant_cache_parity(idx):
    print(f"quant case {idx}: {QUANT[idx]}", flush=True)
    case = _case(dict(QUANT[idx], dtype=F32), 400 + idx)
    got = gqa_gpu(case)
    info = {}
    ref = gqa_oracle(case, info=info)
    n = check_quant_gqa(case, got, ref, info)
    print(f"key codes on the other side of a near tie: {n}")


# Sliding-window caches of codes: the eviction moves code rows (H bytes for
# int8, H / 2 for int4: 40-wide heads give 40- and 20-byte rows), in place or
# by the copy into a separate present buffer.
QWINDOW = [
    dict(B=3, S=1, N=8, kvN=2, H=128, cap=300, window=200, past_lens=[150, 299, 700],
         rotary=True, norm=True, quant=Q8C),
    dict(B=2, S=1, N=4, kvN=2, H=40, cap=64, window=32, past_lens=[10, 100], quant=Q4C),
    dict(B=2, S=40, N=8, kvN=2, H=40, cap=120, window=64, past_lens=[30, 500], softcap=10.0,
         sink=True, quant=Q8T),
    dict(B=1, S=17, N=4, kvN=1, H=128, cap=50, window=33, past_lens=[90], rotary=True,
         quant=Q4T),
]


@pytest.mark.parametrize("separate", [False, True])
@pytest.mark.parametrize("idx", range(len(QWINDOW)))
def test_quant_window_cache_parity(idx, separate):
    print(f"quant window case {idx} separate={separate}: {QWINDOW[idx]}", flush=True)
    case = _case(dict(QWINDOW[idx], dtype=F32, past="shared"), 4200 + idx + 10 * separate)
    case["attrs"]["sliding_window_cache"] = 1
    if separate:
        i = case["inputs"]
        fill = np.full(i["past_key"].shape, 0x5A, np.uint8).view(i["past_key"].dtype)
        i["present_key"], i["present_value"] = fill, fill.copy()
        case["shared"] = False
    got = gqa_gpu(case)
    info = {}
    ref = gqa_oracle(case, info=info)
    n = check_quant_gqa(case, got, ref, info)
    print(f"key codes on the other side of a near tie: {n}")


def test_workload_gqa_decode_int8():
    case = wl.gqa_decode_int8()
    print("gqa_decode_int8", flush=True)
    got = gqa_gpu(case)
    info = {}
    ref = gqa_oracle(case, info=info)
    n = check_quant_gqa(case, got, ref, info)
    print(f"key codes on the other side of a near tie: {n}")


def test_workload_gqa_decode_int4():
    case = wl.gqa_decode_int4()
    print("gqa_decode_int4", flush=True)
    got = gqa_gpu(case)
    info = {}
    ref = gqa_oracle(case, info=info)
    n = check_quant_gqa(case, got, ref, info)
    print(f"key codes on the other side of a near tie: {n}")


def _empty_case(B, S, past=None, cap=64, N=8, kvN=2, H=64, dtype=F16):
    """A call over an empty batch (B = 0) or with no new tokens (S = 0)."""
    rng = np.random.default_rng(900 + B + S)
    inputs = dict(query=wl.normal(rng, (B, S, N * H), dtype),
                  key=wl.normal(rng, (B, S, kvN * H), dtype),
                  value=wl.normal(rng, (B, S, kvN * H), dtype))
    lens = np.full(B, 20, np.int64)
    if past is None:
        inputs.update(present_key=np.zeros((B, kvN, max(S, 1), H), dtype),
                      present_value=np.zeros((B, kvN, max(S, 1), H), dtype))
        inputs["seqlens_k"] = np.full(B, S - 1, np.int32)
    else:
        pk = wl.normal(rng, (B, kvN, cap, H), dtype)
        pv = wl.normal(rng, (B, kvN, cap, H), dtype)
        if past == "shared":
            inputs.update(past_key=pk, past_value=pv, present_key=pk, present_value=pv)
        else:
            inputs.update(past_key=pk, past_value=pv,
                          present_key=np.full((B, kvN, cap + S, H), np.nan, dtype),
                          present_value=np.full((B, kvN, cap + S, H), np.nan, dtype))
        inputs["seqlens_k"] = (lens + S - 1).astype(np.int32)
    attrs = dict(num_heads=N, kv_num_heads=kvN, causal=1, do_rotary=0, local_window_size=-1,
                 qk_norm_epsilon=1e-6, scale=0.0, smooth_softmax=-1, softcap=0.0)
    return dict(op="gqa", inputs=inputs, attrs=attrs, total_sequence_length=21,
                shared=past == "shared")


@pytest.mark.parametrize("B,S,past", [(0, 16, None), (0, 1, "shared"), (2, 0, None),
                                      (2, 0, "concat"), (2, 0, "shared")])
def test_empty_batch_or_sequence(B, S, past):
    """Degenerate calls: nothing to attend; the output is empty and the caches
    hold what the definition says (past rows copied to a separate present)."""
    case = _empty_case(B, S, past)
    out, pk, pv = gqa_gpu(case)
    ref, rpk, rpv = gqa_oracle(case)
    assert out.shape == ref.shape == (B, S, 8 * 64)
    if past == "concat":
        live = np.zeros(pk.shape[:3], bool)
        live[:, :, :20] = True                   # rows [0, past_b) are copied
        assert np.array_equal(pk[live], rpk[live]) and np.array_equal(pv[live], rpv[live])
    else:
        check_cache(pk, rpk, None, "present_key")
        check_cache(pv, rpv, None, "present_value")
