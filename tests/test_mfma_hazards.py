"""Every MFMA result in the library's kernels is read only after enough wait
states on every control-flow path (tests/mfma_hazards.py states the rule).
The kernels are compiled to gfx950 assembly here with the library's own
flags; CPU only (hipcc cross-compiles)."""

import concurrent.futures as cf
import os
import shutil
import subprocess
import tempfile

import pytest

import mfma_hazards as mh
from kv_cache_transformer_amd import build

KERNELS = ["decode.hip", "flash.hip", "packed.hip", "prep.hip"]


def _asm(src, out_dir):
    out = os.path.join(out_dir, src + ".s")
    cmd = [build.HIPCC, *build.FLAGS, "--cuda-device-only", "-S",
           os.path.join(build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} to assembly failed:\n{r.stderr[-2000:]}")
    return open(out).read()


@pytest.fixture(scope="module")
def listings():
    if shutil.which(build.HIPCC) is None and not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not available")
    d = tempfile.mkdtemp(prefix="kvattn_asm_")
    try:
        with cf.ThreadPoolExecutor(len(KERNELS)) as ex:
            texts = list(ex.map(lambda s: _asm(s, d), KERNELS))
    finally:
        shutil.rmtree(d, ignore_errors=True)
    return dict(zip(KERNELS, texts))


SYNTHETIC = """
_Z4testv:
	v_mfma_f32_32x32x16_f16 v[0:15], v[20:23], v[24:27], v[0:15]
	s_cbranch_scc1 .LBB0_2
	s_nop 7
	s_nop 7
.LBB0_2:
	v_add_f32_e32 v30, v3, v31
	s_endpgm
.Lfunc_end0:
"""


def test_checker_flags_a_short_path_through_a_branch():
    # fall-through: 1 + 8 + 8 = 17 wait states; the taken branch: 1
    found = mh.violations(SYNTHETIC)
    assert [(op, w, need) for _, _, op, w, need in found] == [("v_mfma_f32_32x32x16_f16", 1, 12)]
    assert mh.violations(SYNTHETIC.replace("s_cbranch_scc1 .LBB0_2", "s_nop 0")) == []


def test_checker_knows_every_mfma_the_kernels_use(listings):
    import re
    used = set()
    for text in listings.values():
        used |= set(re.findall(r"\bv_mfma_\w+", text))
    assert used and used <= set(mh.PASSES), sorted(used - set(mh.PASSES))


@pytest.mark.parametrize("src", KERNELS)
def test_no_early_mfma_result_reads(listings, src):
    found = mh.violations(listings[src])
    assert not found, "\n".join(f"{k[:70]} #{i} {op}: {w} wait states < {need}"
                                for k, i, op, w, need in found[:10])
