"""Benchmark of the MI355X attention library on its named workloads.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME ...] [--no-cpu]

Prints ONE JSON line.  The headline ("value") is the GroupQueryAttention
decode workload: B=16, N=32, kvN=8, H=128, fp16, shared BNSH cache of
capacity 4096 with past lengths uniform in [1024, 4095], rotary on; one step
is one gqa_attention call, and the value is live key/value bytes read per
second (K and V rows 0..past_b of every sample and kv head).  The decode call
rotates over several independently generated caches so that every call
streams from HBM rather than from the 256 MB last-level cache.

The other workloads (long prefill, small fp32 prompt, block-sparse prompt
and token generation, packed varlen, sliding-window decode, int8 and packed
int4 cache decode) are timed in the same run and reported under "workloads",
each with its own roofline object.

Timing.  `ms_per_step` (and `graph_call_ms` in each workload line) come
from a HIP graph of `steps` calls replayed between two events (no host
launch overhead).  `eager_ms` holds p10 / p50 / p90 / mean over `steps` eager
calls, each bracketed by torch events on the stream, with its dominant
kernel bracketed by HIP events the library records on the same stream
(kvattn_profile_events); a workload line's `call_ms` is that eager call
mean.  Kernel and call come from the same calls, so kernel <= call; the
graph replay runs the same calls without the events between kernels and
reads lower.  The roofline's `achieved` uses
the eager kernel mean, which includes the kernel's dispatch (about 2 us more
than rocprofv3's kernel duration).

CPU baselines: the float64 oracle on the host, on whole decode passes for
about 12 s (the headline's `cpu_baseline`), and on the full outputs of the
long prefill, block-sparse prompt, small prompt and packed batch (their
`cpu_baseline`); `--no-cpu` skips them.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFS = 2500.0     # MI355X dense fp16 MFMA
MFMA_F32_PEAK_TFS = 157.3      # MI355X fp32 matrix
ROOT = os.path.dirname(os.path.abspath(__file__))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", nargs="*", default=None)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--rotations", type=int, default=4)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first copy this many MiB device to device (a plain copy of known size, "
                         "to scale the HBM byte counters of a profiler run)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                    help="CPU only: summarise two rocprofv3 --pmc output folders (FETCH_SIZE, then "
                         "WRITE_SIZE, each from a run with --copy-probe-mib) into profiles/traffic.json")
    ap.add_argument("--counters-from", nargs=2, metavar=("DIR", "COMMAND"), default=None,
                    help="CPU only: summarise one rocprofv3 --pmc run of SQ/GRBM counters (made by "
                         "COMMAND) into profiles/sq_counters_all_workloads.txt")
    ap.add_argument("--traffic-merge", action="store_true",
                    help="CPU only, with --traffic-from: keep the entries of profiles/traffic.json this run "
                         "does not measure")
    ap.add_argument("--traffic-cmd", nargs=2, default=None,
                    help="the two profiler commands, recorded in the traffic summary")
    return ap.parse_args()


class HipEvents:
    """hipEvent_t handles from the HIP runtime (the library records them on
    the stream it launches on; torch events cannot be read after a foreign
    record)."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = self.ct.c_void_p()
        if self.hip.hipEventCreate(self.ct.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev)


class Timer:
    """Per-call timing of one workload.

    Eager calls: each call is bracketed by torch events on the current stream
    and its dominant kernel by HIP events that the library records on the same
    stream around that kernel's launch (kvattn_profile_events), so for every
    call the kernel interval lies inside the call interval (kernel <= call).
    The calls are enqueued behind a spin kernel, so they run back to back on
    the GPU and the intervals hold GPU time only.
    Graph: the same number of calls captured in one HIP graph and replayed
    between two events, so that host launch overhead is not part of the time
    (the figure `value` is computed from)."""

    def __init__(self, torch, lib, kind, hip):
        self.torch, self.lib, self.kind, self.hip = torch, lib, kind, hip

    def run(self, fn, steps, warmup):
        torch = self.torch
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        ks = [self.hip.create() for _ in range(steps)]
        ke = [self.hip.create() for _ in range(steps)]
        cs = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ce = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        # A spin kernel ahead of the timed calls keeps the GPU busy while the
        # host enqueues them, so the calls then run back to back and no host
        # launch latency falls inside an event interval.
        torch.cuda._sleep(int(1e6 + 2e5 * steps))
        for i in range(steps):
            cs[i].record()
            self.lib.kvattn_profile_events(ks[i], ke[i], self.kind)
            fn(warmup + i)
            ce[i].record()
        self.lib.kvattn_profile_events(None, None, 0)
        torch.cuda.synchronize()
        kern = np.array([self.hip.elapsed_ms(ks[i], ke[i]) for i in range(steps)])
        call = np.array([cs[i].elapsed_time(ce[i]) for i in range(steps)])
        for e in ks + ke:
            self.hip.destroy(e)
        if np.any(kern > call + 1e-3):
            print("# warning: a kernel interval exceeds its call interval", file=sys.stderr)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(steps):
                fn(i)
        graph.replay()
        torch.cuda.synchronize()
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record()
        graph.replay()
        c1.record()
        torch.cuda.synchronize()
        graph_ms = c0.elapsed_time(c1) / steps
        del graph
        return dict(call_ms=graph_ms, kern_ms=float(np.mean(kern)), kern_samples=kern,
                    call_samples=call)


def eager_stats(r, scale=1.0, digits=4):
    """p10 / p50 / p90 / mean of the eager per-call samples (kernel <= call per call)."""
    def q(x):
        x = np.asarray(x) * scale
        return {"p10": round(float(np.percentile(x, 10)), digits),
                "p50": round(float(np.median(x)), digits),
                "p90": round(float(np.percentile(x, 90)), digits),
                "mean": round(float(np.mean(x)), digits)}
    return {"kernel": q(r["kern_samples"]), "call": q(r["call_samples"])}


def decode_workload(torch, kv, wl, args, timer):
    case = wl.gqa_decode()
    i = case["inputs"]
    dev = "cuda:0"
    t = {k: torch.from_numpy(v).to(dev) for k, v in i.items() if k not in ("present_key", "present_value")}
    sets = [(t["past_key"], t["past_value"])]
    g = torch.Generator(device=dev)
    g.manual_seed(12345)
    for _ in range(args.rotations - 1):
        sets.append((torch.randn(t["past_key"].shape, generator=g, device=dev).half(),
                     torch.randn(t["past_value"].shape, generator=g, device=dev).half()))
    a = case["attrs"]
    out = torch.empty_like(t["query"])
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=dev)

    def step(n):
        pk, pv = sets[n % len(sets)]
        kv.gqa_attention(t["query"], t["key"], t["value"], pk, pv, t["seqlens_k"],
                         case["total_sequence_length"], t["cos_cache"], t["sin_cache"],
                         num_heads=a["num_heads"], kv_num_heads=a["kv_num_heads"],
                         do_rotary=1, output=out, present_key=pk, present_value=pv, workspace=ws)

    tm = timer.run(step, args.steps, args.warmup)
    lens = i["seqlens_k"].astype(np.int64) + 1
    kvN, H = 8, 128
    kv_bytes = int(lens.sum()) * kvN * H * 2 * 2
    return dict(case=case, **tm,
                kv_bytes=kv_bytes)


def decode_quant_workload(torch, kv, wl, args, timer, bits=8):
    """The decode over an int8 or packed int4 cache (float32 Q/K/V,
    per-channel scales): rotations of random caches as for the float16 decode."""
    case = wl.gqa_decode_int8() if bits == 8 else wl.gqa_decode_int4()
    i = case["inputs"]
    dev = "cuda:0"
    t = {k: torch.from_numpy(v).to(dev) for k, v in i.items() if k not in ("present_key", "present_value")}
    sets = [(t["past_key"], t["past_value"])]
    g = torch.Generator(device=dev)
    g.manual_seed(54321)
    for _ in range(args.rotations - 1):
        lo, hi, cdt = (-128, 128, torch.int8) if bits == 8 else (0, 256, torch.uint8)
        sets.append(tuple(torch.randint(lo, hi, t["past_key"].shape, generator=g, device=dev,
                                        dtype=cdt) for _ in range(2)))
    a = case["attrs"]
    out = torch.empty_like(t["query"])
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=dev)

    def step(n):
        pk, pv = sets[n % len(sets)]
        kv.gqa_attention(t["query"], t["key"], t["value"], pk, pv, t["seqlens_k"],
                         case["total_sequence_length"], t["cos_cache"], t["sin_cache"],
                         k_scale=t["k_scale"], v_scale=t["v_scale"],
                         num_heads=a["num_heads"], kv_num_heads=a["kv_num_heads"], do_rotary=1,
                         k_quant_type=2, v_quant_type=2, kv_cache_bit_width=bits,
                         output=out, present_key=pk, present_value=pv, workspace=ws)

    tm = timer.run(step, args.steps, args.warmup)
    lens = i["seqlens_k"].astype(np.int64) + 1
    kvN, H = 8, 128
    kv_bytes = int(lens.sum()) * kvN * H * 2 * bits // 8   # K and V codes
    return dict(**tm, kv_bytes=kv_bytes)


def window_decode_workload(torch, kv, wl, args, timer):
    """Decode steps on a full sliding-window cache: each call evicts one row
    (the shift moves the other 1023 rows of every slab) and attends the 1024
    rows held.  Repeated calls shift the same amount, so every call costs the
    same."""
    case = wl.gqa_window_decode()
    i = case["inputs"]
    a = case["attrs"]
    dev = "cuda:0"
    t = {k: torch.from_numpy(v).to(dev) for k, v in i.items() if k not in ("present_key", "present_value")}
    out = torch.empty_like(t["query"])
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=dev)

    def step(n):
        kv.gqa_attention(t["query"], t["key"], t["value"], t["past_key"], t["past_value"],
                         t["seqlens_k"], case["total_sequence_length"], t["cos_cache"],
                         t["sin_cache"], num_heads=a["num_heads"], kv_num_heads=a["kv_num_heads"],
                         do_rotary=1, local_window_size=a["local_window_size"],
                         sliding_window_cache=1, output=out, present_key=t["past_key"],
                         present_value=t["past_value"], workspace=ws)

    tm = timer.run(step, args.steps, args.warmup)
    B, kvN, H = 16, 8, 128
    cap = i["past_key"].shape[2]
    row = H * 2                                      # bytes of one fp16 row
    shift_bytes = B * kvN * 2 * (cap - 1) * row * 2  # K and V: read and written once
    read_bytes = B * kvN * 2 * cap * row             # rows attended (K and V)
    return dict(**tm, shift_bytes=shift_bytes,
                read_bytes=read_bytes)


def causal_window_pairs(S, W):
    p = np.arange(S, dtype=np.int64)
    return int(np.minimum(p + 1, W + 1 if W >= 0 else S).sum())


def prefill_workload(torch, kv, wl, args, timer):
    case = wl.gqa_long_prefill()
    i = case["inputs"]
    a = case["attrs"]
    dev = "cuda:0"
    t = {k: torch.from_numpy(v).to(dev) for k, v in i.items()}
    out = torch.empty_like(t["query"])
    ws = torch.zeros(256 << 20, dtype=torch.uint8, device=dev)

    def step(n):
        kv.gqa_attention(t["query"], t["key"], t["value"], None, None, t["seqlens_k"],
                         case["total_sequence_length"], t["cos_cache"], t["sin_cache"], None,
                         t["head_sink"], t["q_norm_weight"], t["k_norm_weight"],
                         num_heads=a["num_heads"], kv_num_heads=a["kv_num_heads"],
                         do_rotary=1, local_window_size=a["local_window_size"],
                         softcap=a["softcap"], output=out, present_key=t["present_key"],
                         present_value=t["present_value"], workspace=ws)

    tm = timer.run(step, args.steps, args.warmup)
    B, S, N, H = 4, 4096, 32, 128
    flops = 4 * H * causal_window_pairs(S, a["local_window_size"]) * B * N
    return dict(**tm, flops=flops)


def prompt_small_workload(torch, kv, wl, args, timer):
    case = wl.gqa_prompt_small()
    i = case["inputs"]
    a = case["attrs"]
    dev = "cuda:0"
    t = {k: torch.from_numpy(v).to(dev) for k, v in i.items()}
    out = torch.empty_like(t["query"])

    def step(n):
        kv.gqa_attention(t["query"], t["key"], t["value"], None, None, t["seqlens_k"], 128,
                         num_heads=8, kv_num_heads=2, scale=0.125, output=out,
                         present_key=t["present_key"], present_value=t["present_value"])

    tm = timer.run(step, args.steps, args.warmup)
    flops = 4 * 64 * causal_window_pairs(128, -1) * 8
    return dict(**tm, flops=flops)


def sparse_pairs(rp, cols, N, B, S, bs):
    L = rp.shape[0]
    per_layout = []
    for l in range(L):
        tot = 0
        for r in range(rp.shape[1] - 1):
            for c in cols[l, rp[l, r]:rp[l, r + 1]]:
                if c < r:
                    tot += bs * bs
                elif c == r:
                    tot += bs * (bs + 1) // 2
        per_layout.append(tot)
    return B * sum(per_layout[h % L] for h in range(N))


def sparse_workload(torch, kv, wl, args, timer):
    case = wl.sparse_prompt()
    i = case["inputs"]
    a = case["attrs"]
    dev = "cuda:0"
    t = {k: torch.from_numpy(v).to(dev) for k, v in i.items()}
    out = torch.empty_like(t["query"])
    ws = torch.zeros(256 << 20, dtype=torch.uint8, device=dev)

    def step(n):
        kv.sparse_attention(t["query"], t["key"], t["value"], t["past_key"], t["past_value"],
                            t["block_row_indices"], t["block_col_indices"], 8192,
                            t["key_total_sequence_lengths"], t["cos_cache"], t["sin_cache"],
                            num_heads=32, kv_num_heads=8, sparse_block_size=64, do_rotary=1,
                            output=out, workspace=ws)

    tm = timer.run(step, args.steps, args.warmup)
    pairs = sparse_pairs(i["block_row_indices"], i["block_col_indices"], 32, 2, 8192, 64)
    return dict(**tm, flops=4 * 128 * pairs)


def sparse_generation_workload(torch, kv, wl, args, timer):
    """One generated token per sample over the sparse layouts: the K/V rows
    of the blocks any query head of a kv head sees are the bytes that must
    be read.  (The decode kernel serves it; its traffic is not split from the
    float16 decode's in the counter runs, which launch the same kernel.)"""
    case = wl.sparse_generation()
    i = case["inputs"]
    dev = "cuda:0"
    t = {k: torch.from_numpy(v).to(dev) for k, v in i.items()}
    out = torch.empty_like(t["query"])
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=dev)
    total = case["total_sequence_length"]

    def step(n):
        kv.sparse_attention(t["query"], t["key"], t["value"], t["past_key"], t["past_value"],
                            t["block_row_indices"], t["block_col_indices"], total,
                            t["key_total_sequence_lengths"], t["cos_cache"], t["sin_cache"],
                            num_heads=32, kv_num_heads=8, sparse_block_size=64, do_rotary=1,
                            output=out, workspace=ws)

    tm = timer.run(step, args.steps, args.warmup)
    rp, cols = i["block_row_indices"], i["block_col_indices"]
    B, N, kvN, H, bs = 2, 32, 8, 128, 64
    row = (total - 1) // bs
    blocks = 0
    for kh in range(kvN):
        seen = set()
        for h in range(kh * (N // kvN), (kh + 1) * (N // kvN)):
            l = h % rp.shape[0]
            seen |= set(int(c) for c in cols[l, rp[l, row]:rp[l, row + 1]])
        blocks += len(seen)
    kv_bytes = B * blocks * bs * H * 2 * 2
    return dict(**tm, kv_bytes=kv_bytes)


def packed_workload(torch, kv, wl, args, timer):
    case = wl.packed_varlen()
    i = case["inputs"]
    dev = "cuda:0"
    t = {k: torch.from_numpy(v).to(dev) for k, v in i.items()}
    T = i["input"].shape[0]
    out = torch.empty((T, 768), dtype=torch.float16, device=dev)
    ws = torch.zeros(256 << 20, dtype=torch.uint8, device=dev)

    def step(n):
        kv.packed_attention(t["input"], t["weights"], t["bias"], t["token_offset"],
                            t["cumulative_sequence_length"], num_heads=12, output=out,
                            workspace=ws)

    tm = timer.run(step, args.steps, args.warmup)
    L = case["lengths"].astype(np.int64)
    gemm = 2 * T * 768 * 2304
    attn = 4 * 64 * 12 * int((L * L).sum())
    return dict(**tm, gemm_flops=gemm,
                attn_flops=attn, tokens=T)


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(case, budget_s=12.0):
    """Time the oracle on the decode workload (all 16 samples per pass),
    repeating passes until about budget_s seconds of CPU work; report live KV
    GB/s of the oracle."""
    import oracle
    threads = _blas_threads()
    i = case["inputs"]
    lens = i["seqlens_k"].astype(np.int64) + 1
    B = lens.shape[0]
    per_pass = int(lens.sum()) * 8 * 128 * 2 * 2
    elapsed = 0.0
    passes = 0
    while elapsed < budget_s and passes < 100:
        for b in range(B):
            sl = slice(b, b + 1)
            t0 = time.perf_counter()
            oracle.gqa(i["query"][sl], i["key"][sl], i["value"][sl],
                       seqlens_k=i["seqlens_k"][sl],
                       total_sequence_length=case["total_sequence_length"],
                       past_key=i["past_key"][sl], past_value=i["past_value"][sl],
                       present_key=i["past_key"][sl], present_value=i["past_value"][sl],
                       cos_cache=i["cos_cache"], sin_cache=i["sin_cache"],
                       num_heads=32, kv_num_heads=8, do_rotary=1)
            elapsed += time.perf_counter() - t0
        passes += 1
    return {"value": round(per_pass * passes / elapsed / 1e9, 4), "unit": "GB/s",
            "cores": int(threads), "kind": "oracle",
            "sample": f"float64 numpy oracle over the whole decode workload (16 samples, "
                      f"{per_pass / 1e6:.1f} MB of live K/V per pass), {passes} passes in "
                      f"{elapsed:.1f} s"}


def cpu_baseline_workload(name, wl, flops):
    """The oracle's full outputs of one prompt workload, timed on the host:
    the long prefill and the block-sparse prompt over row chunks in child
    processes (one BLAS thread each, one per core up to 16), the small prompt
    and the packed batch in this process (best of three).  Reported as
    algorithmic TFLOP/s of the oracle."""
    import oracle
    from oracle import pool
    if name in ("gqa_long_prefill", "sparse_prompt"):
        S = 4096 if name == "gqa_long_prefill" else 8192
        t0 = time.perf_counter()
        if name == "gqa_long_prefill":
            pool.gqa_full(name, S)
        else:
            pool.sparse_full(name, S)
        best, runs, cores = time.perf_counter() - t0, 1, pool.workers()
        how = f"{cores} child processes over row chunks, 1 run"
    else:
        case = getattr(wl, name)()
        i = dict(case["inputs"])
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            if name == "packed_varlen":
                j = dict(i)
                oracle.packed(j.pop("input"), j.pop("weights"), j.pop("bias"), j.pop("token_offset"),
                              j.pop("cumulative_sequence_length"), **j, **case["attrs"])
            else:
                j = dict(i)
                a = dict(case["attrs"])
                a["softcap_value"] = a.pop("softcap")
                oracle.gqa(j.pop("query"), j.pop("key"), j.pop("value"),
                           total_sequence_length=case["total_sequence_length"], **j, **a)
            times.append(time.perf_counter() - t0)
        best, runs, cores = min(times), 3, _blas_threads()
        how = f"this process, BLAS on {cores} threads, best of {runs}"
    return {"value": round(flops / best / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"float64 numpy oracle, full outputs of the whole workload in {best:.2f} s ({how})"}


# Kernels whose HBM traffic is summarised, keyed as bench lines look them up:
# (key, pattern on the mangled kernel name, sources whose hash pins the figure)
_KERNEL_SOURCES = ["kv_cache_transformer_amd/csrc/device_common.hpp",
                   "kv_cache_transformer_amd/csrc/kvattn_internal.hpp",
                   "kv_cache_transformer_amd/csrc/api.cpp"]
TRAFFIC_KERNELS = [
    ("decode", r"decode_kernelIDF16_Li128ELi0E", "kv_cache_transformer_amd/csrc/decode.hip", "gqa_decode"),
    ("flash_gqa_long_prefill", r"flash_pp_kernel(?:ILi128ELi0E|<128, 0,)", "kv_cache_transformer_amd/csrc/flash.hip",
     "gqa_long_prefill"),
    ("flash_sparse_prompt", r"flash_kernelIDF16_Li128ELi\d+ELi1E", "kv_cache_transformer_amd/csrc/flash.hip",
     "sparse_prompt", lambda grid: grid >= 1 << 20),
    ("qkv_gemm_packed_varlen", r"qkv_gemm_dma_kernel", "kv_cache_transformer_amd/csrc/packed.hip",
     "packed_varlen"),
    ("window_shift_gqa_window_decode", r"window_shift_kernel", "kv_cache_transformer_amd/csrc/prep.hip",
     "gqa_window_decode"),
    ("decode_gqa_decode_int8", r"decode_kernel(?:INS0_7QuantI8ELi128E|<[^<>]*QuantI8, 128,)",
     "kv_cache_transformer_amd/csrc/decode.hip", "gqa_decode_int8"),
    ("decode_gqa_decode_int4", r"decode_kernel(?:INS0_7QuantI4ELi128E|<[^<>]*QuantI4, 128,)",
     "kv_cache_transformer_amd/csrc/decode.hip", "gqa_decode_int4"),
]


def _sources_sha(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()


def summarise_traffic(fetch_dir, write_dir, cmds, probe_mib, merge=False):
    """Per-launch HBM bytes of the library's kernels from two rocprofv3
    counter runs.  Each counter is scaled by what it reads for the largest
    device-to-device copy of the same run (a copy of known size), and the
    figure is stored with a hash of the kernel's sources.  With ``merge`` the
    entries of profiles/traffic.json that this run does not measure are kept
    (workloads launching the same kernel are counted in runs of their own)."""
    import csv
    import glob
    import re

    def load(d, counter):
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            rows += [r for r in csv.DictReader(open(f)) if r["Counter_Name"] == counter]
        if not rows:
            raise SystemExit(f"no {counter} rows under {d}")
        copies = [r for r in rows if "copyBuffer" in r["Kernel_Name"]]
        if not copies:
            raise SystemExit(f"no copy-probe dispatch under {d} (run with --copy-probe-mib)")
        probe = max(copies, key=lambda r: float(r["Counter_Value"]))
        return rows, float(probe["Counter_Value"])

    probe_kib = probe_mib * 1024
    fetch, f_probe = load(fetch_dir, "FETCH_SIZE")
    write, w_probe = load(write_dir, "WRITE_SIZE")
    f_scale, w_scale = probe_kib / f_probe, probe_kib / w_probe
    path = os.path.join(ROOT, "profiles", "traffic.json")
    out = json.load(open(path)) if (merge and os.path.exists(path)) else {}
    # a run measures the workloads its command names (bench.py --only ...), or all
    ran = set()
    for c in cmds or []:
        toks = c.split()
        if "--only" in toks:
            for t in toks[toks.index("--only") + 1:]:
                if t.startswith("--"):
                    break
                ran.add(t)
    for key, pat, src, workload, *grid_ok in TRAFFIC_KERNELS:
        if ran and workload not in ran:
            continue
        # kernels that two workloads share are told apart by their grid size (threads)
        ok = grid_ok[0] if grid_ok else (lambda grid: True)
        fr = [float(r["Counter_Value"]) for r in fetch
              if re.search(pat, r["Kernel_Name"]) and ok(int(r["Grid_Size"]))]
        wr = [float(r["Counter_Value"]) for r in write
              if re.search(pat, r["Kernel_Name"]) and ok(int(r["Grid_Size"]))]
        if not fr or not wr:
            continue
        fk, wk = sum(fr) / len(fr), sum(wr) / len(wr)
        rb, wb = fk * 1024 * f_scale, wk * 1024 * w_scale
        sources = [src] + _KERNEL_SOURCES
        out[key] = {"bytes_per_launch": int(round(rb + wb)), "fetch_bytes": int(round(rb)),
                    "write_bytes": int(round(wb)), "fetch_kib": fk, "write_kib": wk,
                    "fetch_scale": f_scale, "write_scale": w_scale, "probe_mib": probe_mib,
                    "probe_fetch_kib": f_probe, "probe_write_kib": w_probe,
                    "launches": len(fr), "sources": sources, "source_sha256": _sources_sha(sources),
                    "workload": workload, "commands": list(cmds or ["(not recorded)"]),
                    "profile": "profiles/traffic_all_workloads.txt"}
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    lines = ["# HBM traffic per launch of the library's kernels (bench workloads)",
             "# each group: the commands (on the GPU host, from the repository root), one counter per",
             "# run, and the calibration of that group's counters by its device-to-device copy"]
    groups = {}
    for key, e in out.items():
        groups.setdefault(tuple(e.get("commands", [])), []).append((key, e))
    for cmd_group, ents in groups.items():
        e0 = ents[0][1]
        lines += [f"#   {c}" for c in cmd_group]
        lines += [f"# calibration: the {e0.get('probe_mib', probe_mib)} MiB copy reads FETCH_SIZE "
                  f"{e0.get('probe_fetch_kib', 0):.0f} KiB (scale {e0['fetch_scale']:.4f}) and WRITE_SIZE "
                  f"{e0.get('probe_write_kib', 0):.0f} KiB (scale {e0['write_scale']:.4f})",
                  f"{'kernel':<32} {'launches':>8} {'FETCH KiB':>12} {'WRITE KiB':>12} {'read MB':>10} {'written MB':>10}"]
        for key, e in ents:
            lines.append(f"{key:<32} {e['launches']:>8} {e.get('fetch_kib', 0):>12.1f} {e.get('write_kib', 0):>12.1f} "
                         f"{e['fetch_bytes'] / 1e6:>10.2f} {e['write_bytes'] / 1e6:>10.2f}")
        lines.append("")
    with open(os.path.join(ROOT, "profiles", "traffic_all_workloads.txt"), "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def summarise_counters(d, cmd):
    """Per-kernel averages of one rocprofv3 counter run, with the MFMA and VALU
    busy fractions.  GRBM_GUI_ACTIVE sums the eight XCDs' busy clocks, so the
    SIMD-cycles of a launch are GRBM_GUI_ACTIVE / 8 * 1024 SIMDs;
    SQ_ACTIVE_INST_VALU counts quad-cycles."""
    import csv
    import glob
    import re
    pat = re.compile(r"(flash_pp_kernel|flash_kernel|decode_kernel|qkv_gemm_dma_kernel|qkv_gemm_kernel|prep_kv_kernel|"
                     r"window_shift_kernel|prep_kernel|packed_sched_kernel)(?:I(DF16_|f)(?:Li(\d+)ELi(\d+)(?:ELi(\d+))?)?)?")
    agg, dur = {}, {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            m = pat.search(r["Kernel_Name"])
            if not m:
                continue
            t = {"DF16_": "f16", "f": "f32", None: ""}[m.group(2)]
            hd, md = m.group(3), m.group(5)
            pm = re.search(r"flash_pp_kernel(?:ILi(\d+)ELi(\d+)E|<(\d+), (\d+),)", r["Kernel_Name"])
            if pm:  # f16 only; template arguments (head, mode, ...)
                t, hd, md = "f16", pm.group(1) or pm.group(3), pm.group(2) or pm.group(4)
            dm = re.search(r"<float(?:, (\d+), (\d+), (\d+))?", r["Kernel_Name"])
            if not t and dm:  # names of float instances come demangled
                t, hd, md = "f32", dm.group(1), dm.group(3)
            qm = re.search(r"QuantI([48])(?:E|, )(?:Li)?(\d+)", r["Kernel_Name"])
            if qm:  # quantised-cache decode
                t, hd, md = "q" + qm.group(1), qm.group(2), None
            mode = {"0": "dense", "1": "csr", "2": "varlen"}.get(md, "")
            if m.group(1) == "decode_kernel" and m.group(4) is not None and not qm:
                mode = "feat" + m.group(4)  # decode_kernel<type, head, features>
            key = m.group(1) + (f"<{t},{hd},{mode}>" if hd else (f"<{t}>" if t else ""))
            agg.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                dur.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines = ["# SQ / GRBM counters per launch, all bench workloads (one counter run, averages over launches)",
             "# command (on the GPU host, from the repository root):", f"#   {cmd}",
             "# mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / SIMD-cycles; valu_busy = 4 * SQ_ACTIVE_INST_VALU / SIMD-cycles;",
             "# SIMD-cycles = GRBM_GUI_ACTIVE (summed over the 8 XCDs) / 8 * 1024 SIMDs; clock = GRBM_GUI_ACTIVE / 8 / duration",
             "# (GRBM_GUI_ACTIVE also counts a few microseconds of dispatch around the kernel, so the clock",
             "# column reads high on short kernels; the long kernels show the clock under load)",
             f"{'kernel':<28} {'launches':>8} {'dur_us':>8} {'clock_GHz':>9} {'mfma_busy':>9} {'valu_busy':>9} "
             f"{'lds_bank_conf':>13} {'lds_active':>11} {'mfma_insts':>11} {'valu_insts':>11}"]
    for key in sorted(agg):
        g = {c: sum(v) / len(v) for c, v in agg[key].items()}
        gui = g.get("GRBM_GUI_ACTIVE", 0.0)
        ns = sum(dur.get(key, [0])) / max(1, len(dur.get(key, [])))
        simd_cyc = gui / 8 * 1024
        if simd_cyc <= 0 or ns <= 0:
            continue
        lines.append(f"{key:<28} {len(agg[key].get('GRBM_GUI_ACTIVE', [])):>8} {ns / 1e3:>8.1f} "
                     f"{gui / 8 / ns:>9.2f} {g.get('SQ_VALU_MFMA_BUSY_CYCLES', 0) / simd_cyc:>9.3f} "
                     f"{4 * g.get('SQ_ACTIVE_INST_VALU', 0) / simd_cyc:>9.3f} "
                     f"{g.get('SQ_LDS_BANK_CONFLICT', 0):>13.4g} {g.get('SQ_ACTIVE_INST_LDS', 0):>11.4g} "
                     f"{g.get('SQ_INSTS_MFMA', 0):>11.4g} {g.get('SQ_INSTS_VALU', 0):>11.4g}")
    with open(os.path.join(ROOT, "profiles", "sq_counters_all_workloads.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def traffic_for(kernel_key):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    when the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
        ent = data.get(kernel_key)
        if not ent:
            return None
        if _sources_sha(ent["sources"]) != ent["source_sha256"]:
            return None
        return ent["bytes_per_launch"]
    except Exception:
        return None


def main():
    args = parse()
    if args.counters_from:
        summarise_counters(args.counters_from[0], args.counters_from[1])
        return
    if args.traffic_from:
        summarise_traffic(args.traffic_from[0], args.traffic_from[1], args.traffic_cmd,
                          args.copy_probe_mib or 512, merge=args.traffic_merge)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has "
              "no multi-GPU path: every workload here is one GPU's share.", file=sys.stderr)
        sys.exit(2)
    import torch
    import kv_cache_transformer_amd as kv
    from kv_cache_transformer_amd import workloads as wl
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    lib = kv.library()
    hip = HipEvents()
    only = set(args.only) if args.only else None

    def want(name):
        return only is None or name in only

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"# copy probe: {args.copy_probe_mib} MiB read and written", file=sys.stderr, flush=True)
        del src, dst

    res = {}
    if want("gqa_decode"):
        res["gqa_decode"] = decode_workload(torch, kv, wl, args, Timer(torch, lib, 1, hip))
        print(f"# gqa_decode done: {res['gqa_decode']['call_ms']*1e3:.1f} us/call", file=sys.stderr, flush=True)
    if want("gqa_long_prefill"):
        res["gqa_long_prefill"] = prefill_workload(torch, kv, wl, args, Timer(torch, lib, 2, hip))
        print("# gqa_long_prefill done", file=sys.stderr, flush=True)
    if want("gqa_prompt_small"):
        res["gqa_prompt_small"] = prompt_small_workload(torch, kv, wl, args, Timer(torch, lib, 2, hip))
        print("# gqa_prompt_small done", file=sys.stderr, flush=True)
    if want("sparse_prompt"):
        res["sparse_prompt"] = sparse_workload(torch, kv, wl, args, Timer(torch, lib, 2, hip))
        print("# sparse_prompt done", file=sys.stderr, flush=True)
    if want("sparse_generation"):
        res["sparse_generation"] = sparse_generation_workload(torch, kv, wl, args, Timer(torch, lib, 1, hip))
        print("# sparse_generation done", file=sys.stderr, flush=True)
    if want("gqa_window_decode"):
        res["gqa_window_decode"] = window_decode_workload(torch, kv, wl, args, Timer(torch, lib, 5, hip))
        print("# gqa_window_decode done", file=sys.stderr, flush=True)
    for bits in (8, 4):
        name = f"gqa_decode_int{bits}"
        if want(name):
            res[name] = decode_quant_workload(torch, kv, wl, args, Timer(torch, lib, 1, hip), bits)
            print(f"# {name} done: {res[name]['call_ms']*1e3:.1f} us/call", file=sys.stderr, flush=True)
    if want("packed_varlen"):
        res["packed_varlen"] = packed_workload(torch, kv, wl, args, Timer(torch, lib, 4, hip))
        print("# packed_varlen done", file=sys.stderr, flush=True)

    workloads = {}

    def timing(r):
        """Per call, in ms: the eager call mean (the calls the kernel time
        comes from, so kernel <= call), the eager samples, and the graph
        replay."""
        e = eager_stats(r, digits=5)
        return {"call_ms": e["call"]["mean"], "eager_ms": e, "graph_call_ms": round(r["call_ms"], 5)}

    def mfma_line(name, config, r, flops, peak, kernel, traffic_key, extra=None):
        tf_k = flops / (r["kern_ms"] * 1e-3) / 1e12
        d = {"config": config, **timing(r),
             "graph_call_TFLOPs": round(flops / (r["call_ms"] * 1e-3) / 1e12, 3),
             "roofline": {"bound": "mfma", "kernel": kernel, "achieved": round(tf_k, 3),
                          "peak": peak, "unit": "TFLOP/s", "frac": round(tf_k / peak, 5),
                          "kernel_ms": round(r["kern_ms"], 5), "algorithmic_flops": flops,
                          "traffic": traffic_for(traffic_key) if traffic_key else None}}
        if extra:
            d.update(extra)
        if not args.no_cpu:
            d["cpu_baseline"] = cpu_baseline_workload(name, wl, r.get("all_flops", flops))
        workloads[name] = d

    if "gqa_long_prefill" in res:
        r = res["gqa_long_prefill"]
        mfma_line("gqa_long_prefill",
                  "B4 S4096 N32 kvN8 H128 fp16 causal window 1024 softcap 50 sink qk-norm rotary",
                  r, r["flops"], MFMA_F16_PEAK_TFS, "flash", "flash_gqa_long_prefill")
        print("# gqa_long_prefill reported", file=sys.stderr, flush=True)
    if "gqa_prompt_small" in res:
        r = res["gqa_prompt_small"]
        mfma_line("gqa_prompt_small", "B1 S128 N8 kvN2 H64 fp32 causal", r, r["flops"],
                  MFMA_F32_PEAK_TFS, "flash", None)
    if "sparse_prompt" in res:
        r = res["sparse_prompt"]
        mfma_line("sparse_prompt", "B2 S8192 N32 kvN8 H128 fp16 block 64, 4 CSR layouts, NeoX rotary",
                  r, r["flops"], MFMA_F16_PEAK_TFS, "flash", "flash_sparse_prompt")
        print("# sparse_prompt reported", file=sys.stderr, flush=True)
    if "packed_varlen" in res:
        r = res["packed_varlen"]
        r["all_flops"] = r["gemm_flops"] + r["attn_flops"]
        mfma_line("packed_varlen",
                  f"64 seqs of 32..512 tokens (T={r['tokens']}), D768, QKV 768x2304, 12x64 fp16",
                  r, r["gemm_flops"], MFMA_F16_PEAK_TFS, "qkv_gemm", "qkv_gemm_packed_varlen",
                  {"graph_call_TFLOPs": round(r["all_flops"] / (r["call_ms"] * 1e-3) / 1e12, 3),
                   "algorithmic_flops_call": r["all_flops"]})

    def hbm_line(name, config, r, nbytes, kernel, traffic_key, call_bytes=None):
        gbs_k = nbytes / (r["kern_ms"] * 1e-3) / 1e9
        cb = call_bytes if call_bytes is not None else nbytes
        workloads[name] = {
            "config": config, **timing(r),
            "graph_call_GBs": round(cb / (r["call_ms"] * 1e-3) / 1e9, 2), "algorithmic_bytes_call": cb,
            "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(gbs_k, 2),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs_k / HBM_PEAK_GBS, 4),
                         "kernel_ms": round(r["kern_ms"], 5), "algorithmic_bytes": nbytes,
                         "traffic": traffic_for(traffic_key) if traffic_key else None}}

    if "gqa_window_decode" in res:
        r = res["gqa_window_decode"]
        hbm_line("gqa_window_decode",
                 "B16 N32 kvN8 H128 fp16, sliding-window cache 1024 (window 1023), past tokens U[1024,4095], rotary",
                 r, r["shift_bytes"], "window_shift", "window_shift_gqa_window_decode",
                 call_bytes=r["shift_bytes"] + r["read_bytes"])
    if "sparse_generation" in res:
        r = res["sparse_generation"]
        hbm_line("sparse_generation",
                 "B2 S1 after 8191 past rows, N32 kvN8 H128 fp16 block 64, 4 CSR layouts, NeoX rotary",
                 r, r["kv_bytes"], "decode", None)
    for bits, cname in ((8, "int8"), (4, "packed int4")):
        name = f"gqa_decode_int{bits}"
        if name in res:
            hbm_line(name, f"B16 N32 kvN8 H128 fp32 Q/K/V, shared {cname} cache 4096, per-channel scales, "
                           "past lengths U[1024,4095], rotary", res[name], res[name]["kv_bytes"],
                     "decode", f"decode_{name}")

    line = {"metric": "GQA prefill TFLOP/s and decode KV GB/s on 1 MI355X, % of roofline",
            "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
            "config": {"workload": "gqa_decode: GroupQueryAttention decode, B16 N32 kvN8 H128 fp16, "
                                   "shared BNSH cache 4096, past lengths U[1024,4095], rotary theta 1e4",
                       "batch": 16, "cache_capacity": 4096}}
    if "gqa_decode" in res:
        r = res["gqa_decode"]
        gbs_call = r["kv_bytes"] / (r["call_ms"] * 1e-3) / 1e9
        gbs_k = r["kv_bytes"] / (r["kern_ms"] * 1e-3) / 1e9
        line["value"] = round(gbs_call, 2)
        line["ms_per_step"] = round(r["call_ms"], 5)
        line["config"]["live_kv_bytes"] = r["kv_bytes"]
        line["config"]["cache_rotations"] = args.rotations
        line["timing"] = {"ms_per_step": "graph replay of `steps` calls, per call",
                          "eager_ms": eager_stats(r, digits=5)}
        line["roofline"] = {"bound": "hbm", "kernel": "decode", "achieved": round(gbs_k, 2),
                            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs_k / HBM_PEAK_GBS, 4),
                            "kernel_us": round(r["kern_ms"] * 1e3, 3),
                            "algorithmic_bytes": r["kv_bytes"], "traffic": traffic_for("decode")}
        if not args.no_cpu:
            line["cpu_baseline"] = cpu_baseline(r["case"])
    line["workloads"] = workloads
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
