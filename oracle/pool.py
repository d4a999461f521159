"""The oracle over chunks of a named full-size workload, in child processes.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): no arithmetic of the
method lives here.  The full-size parity tests compare every output element
of the long prefill (4 x 4096 query rows) and the block-sparse prompt
(2 x 8192 rows) with the oracle, and the benchmark's CPU baseline times the
same full-output runs.  The oracle computes a chunk of query rows
exactly as it computes the whole (rows are independent), so the chunks run
in separate Python processes, at most one per core (16 at most).  Each child
generates the workload itself from its seed, limits its BLAS to one thread,
computes its rows and saves them to a temporary .npy file; the parent starts
the children as plain subprocesses (they inherit no GPU state), waits for
each with a time limit and fails on any non-zero exit.

Run as a script it is one such child:
    python oracle/pool.py {gqa|sparse} WORKLOAD ROW0 ROW1 OUT.npy WANT_CACHE
"""

import os
import subprocess
import sys
import tempfile
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def workers():
    """Child processes at a time: the host's cores, at most 16 (a GPU machine's CPU share)."""
    return max(1, min(16, os.cpu_count() or 1))


def _workloads():
    """The seeded input generators (kv_cache_transformer_amd/workloads.py),
    loaded from their file alone so that nothing of the HIP library's package
    is imported here."""
    import importlib.util
    path = os.path.join(ROOT, "kv_cache_transformer_amd", "workloads.py")
    spec = importlib.util.spec_from_file_location("_seeded_workloads", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _child(kind, name, r0, r1, out_path, want_cache):
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass
    import oracle
    case = getattr(_workloads(), name)()
    i = dict(case["inputs"])
    rows = list(range(r0, r1))
    if kind == "gqa":
        a = dict(case["attrs"])
        a["softcap_value"] = a.pop("softcap")
        out, pk, pv = oracle.gqa(i.pop("query"), i.pop("key"), i.pop("value"),
                                 total_sequence_length=case["total_sequence_length"],
                                 query_rows=rows, **i, **a)
    elif kind == "sparse":
        out, pk, pv = oracle.sparse(i.pop("query"), i.pop("key"), i.pop("value"),
                                    i.pop("past_key"), i.pop("past_value"),
                                    total_sequence_length=case["total_sequence_length"],
                                    query_rows=rows, **i, **case["attrs"])
    else:
        raise SystemExit(f"unknown kind {kind}")
    np.save(out_path, out)
    if want_cache:
        np.save(out_path + ".pk.npy", pk)
        np.save(out_path + ".pv.npy", pv)


def _run(kind, name, S, chunk, timeout_s=900):
    tasks = [(r0, min(r0 + chunk, S)) for r0 in range(0, S, chunk)]
    with tempfile.TemporaryDirectory(prefix="oracle_pool_") as tmp:
        paths = [os.path.join(tmp, f"rows_{r0}.npy") for r0, _ in tasks]
        pending = list(range(len(tasks)))
        running = {}
        t0 = time.time()
        try:
            while pending or running:
                while pending and len(running) < workers():
                    k = pending.pop(0)
                    r0, r1 = tasks[k]
                    cmd = [sys.executable, os.path.abspath(__file__), kind, name, str(r0), str(r1),
                           paths[k], "1" if k == 0 else "0"]
                    running[k] = subprocess.Popen(cmd, cwd=ROOT)
                for k, p in list(running.items()):
                    rc = p.poll()
                    if rc is None:
                        continue
                    del running[k]
                    if rc != 0:
                        raise RuntimeError(f"oracle child for rows {tasks[k]} exited with {rc}")
                if time.time() - t0 > timeout_s:
                    raise TimeoutError(f"oracle children not done after {timeout_s} s")
                time.sleep(0.05)
        finally:
            for p in running.values():
                p.kill()
                p.wait()
        out = np.concatenate([np.load(p) for p in paths], axis=1)
        pk = np.load(paths[0] + ".pk.npy")
        pv = np.load(paths[0] + ".pv.npy")
    return out, pk, pv


def gqa_full(name, S, chunk=256):
    """(output over all rows, present_key, present_value) of a GroupQueryAttention workload."""
    return _run("gqa", name, S, chunk)


def sparse_full(name, S, chunk=512):
    """(output over all rows, key cache, value cache) of a SparseAttention workload."""
    return _run("sparse", name, S, chunk)


if __name__ == "__main__":
    kind, name, r0, r1, out_path, want = sys.argv[1:7]
    _child(kind, name, int(r0), int(r1), out_path, want == "1")
