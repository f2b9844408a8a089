"""Register use of every HIP kernel, from the compiler's resource report
(device-only compile for gfx950 with -Rpass-analysis=kernel-resource-usage;
no GPU needed).

No kernel may spill vector registers: a spill moves values through scratch
memory inside the hot loops, and it appears silently when a shared piece of
code (the tile store, the fused expand) grows.  The FP8 LoRA GEMM, at the
register file's limit with 256 accumulators, is the first to show it."""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from rank_adapter_gemm_amd import build

HIPCC = build.HIPCC


def _report(src: str, outdir: str) -> str:
    flags = [f for f in build.FLAGS if f != "-shared"]
    cmd = [HIPCC] + flags + ["--offload-device-only", "-c", os.path.join(build.CSRC, src),
                             "-o", os.path.join(outdir, src + ".o"), "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return res.stderr


def _parse(text: str) -> dict:
    kernels, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark:\s+(VGPRs Spill|VGPRs|AGPRs|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and cur:
            kernels[cur][m.group(1)] = int(m.group(2))
    return kernels


@pytest.fixture(scope="module")
def resources():
    if not (os.path.exists(HIPCC) or shutil.which(HIPCC)):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        with ThreadPoolExecutor(max_workers=min(8, len(build.SOURCES))) as ex:
            texts = list(ex.map(lambda s: _report(s, d), build.SOURCES))
    out = {}
    for src, text in zip(build.SOURCES, texts):
        for name, info in _parse(text).items():
            out[(src, name)] = info
    return out


def test_reports_cover_the_kernels(resources):
    names = " ".join(n for _, n in resources)
    for k in ("k_gemm_bf16", "k_gemm_fp8", "k_splitk_reduce", "k_shrink_rows", "k_shrink_grouped",
              "k_expand_short", "k_seg_scan", "k_upload"):
        assert k in names, k


def test_no_kernel_spills_vector_registers(resources):
    spilled = {name: info for (src, name), info in resources.items() if info.get("VGPRs Spill", 0) > 0}
    assert not spilled, spilled


def test_large_tiles_keep_one_workgroup_per_cu_resident(resources):
    """The 256x256 GEMM tiles run eight wavefronts (two per SIMD) or four
    (one per SIMD, accumulators in AGPRs); both need their registers to fit
    that occupancy."""
    for (src, name), info in resources.items():
        if "k_gemm_bf16ILb1ELi256ELi256ELi64" in name or "k_gemm_bf16ILb0ELi256ELi256ELi64" in name:
            assert info["VGPRs"] + info.get("AGPRs", 0) <= 256, (name, info)
        if "k_gemm_fp8ILb1ELi256ELi256" in name or "k_gemm_fp8ILb0ELi256ELi256" in name:
            assert info["VGPRs"] <= 256 and info.get("AGPRs", 0) <= 256, (name, info)
