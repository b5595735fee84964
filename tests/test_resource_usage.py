"""Register, scratch and LDS budgets of every kernel, read from the compiler.

Each HIP source is compiled for gfx950 with the library's own flags and the
compiler's per-kernel resource report.  The checks hold the facts the kernels'
launch shapes rely on:

* no kernel spills to scratch memory;
* the direct-to-LDS prefill kernels fit three waves per SIMD (at most 168
  VGPRs) and three workgroups per CU in LDS (the tile ring of three stages is
  sized for that residency; a build that fell to two waves per SIMD ran 20 %
  slower with bitwise-identical output, which no parity test would notice);
* the persistent decode kernels fit one wave per SIMD.

Runs on the CPU (hipcc cross-compiles); skipped where hipcc is absent.
"""
import importlib.util
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_85_amd", "csrc")
LDS_PER_CU = 160 * 1024


def _build_flags():
    spec = importlib.util.spec_from_file_location(
        "pa_build_flags", os.path.join(ROOT, "paged_kv_cache_85_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.hipcc(), list(mod.COMMON)


def _report(hipcc, flags, src, out_dir):
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [hipcc] + flags + ["--cuda-device-only", "-c", src, "-o", obj,
                             "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"compile failed: {' '.join(cmd)}\n{r.stderr[-4000:]}"
    kernels, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+)\s*(?:\[|$)", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = int(m.group(2))
    return kernels


@pytest.fixture(scope="module")
def usage(tmp_path_factory):
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    hipcc, flags = _build_flags()
    out_dir = str(tmp_path_factory.mktemp("resource_usage"))
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        reports = list(ex.map(lambda s: _report(hipcc, flags, s, out_dir), srcs))
    merged = {}
    for rep in reports:
        merged.update(rep)
    return merged


def test_reports_cover_the_hot_kernels(usage):
    names = list(usage)
    for part in ("store_kv_kernel", "decode_persistent_kernel", "decode_combine_kernel",
                 "decode_gqa_mfma_kernel", "prefill_bf16_kernel", "row_attn_kernel"):
        assert any(part in n for n in names), part
    for n, u in usage.items():
        for key in ("VGPRs", "ScratchSize", "Occupancy", "VGPRs Spill"):
            assert key in u, (n, key, u)


def test_no_kernel_spills_to_scratch(usage):
    bad = {n: (u["ScratchSize"], u["VGPRs Spill"]) for n, u in usage.items()
           if u["ScratchSize"] != 0 or u["VGPRs Spill"] != 0}
    assert not bad, bad


def test_direct_to_lds_prefill_fits_three_workgroups_per_cu(usage):
    # prefill_bf16_kernel<D, HPW, DMA, BN, NST, POL>: DMA = true (b1) kernels.
    dma = {n: u for n, u in usage.items()
           if re.search(r"prefill_bf16_kernelILi(64|128)ELi\dELb1E", n)}
    assert len(dma) == 18, sorted(dma)
    for n, u in dma.items():
        assert u["VGPRs"] <= 168, (n, u["VGPRs"])
        assert u["Occupancy"] >= 3, (n, u["Occupancy"])
        assert 3 * u["LDS Size"] <= LDS_PER_CU, (n, u["LDS Size"])


def test_persistent_decode_fits_one_wave_per_simd(usage):
    pers = {n: u for n, u in usage.items() if "decode_persistent_kernel" in n}
    assert pers
    for n, u in pers.items():
        assert u["Occupancy"] >= 1, (n, u)
        assert u["LDS Size"] <= LDS_PER_CU // 4, (n, u["LDS Size"])
