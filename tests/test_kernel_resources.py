"""Register budget of the gfx950 kernels, read from the compiler (no GPU).

Every kernel runs one 256-thread workgroup per CU with up to 512 registers a
lane; a change that pushes one over makes the compiler spill to scratch
memory, which costs HBM writes and time without changing any result.  This
compiles each source for the device only with the compiler's resource-usage
report and checks that the kernels of the fused path (direct-to-LDS GEMM,
row passes, gradient scaling, RMSNorm, fp32 GEMM) neither spill nor use
scratch.
The register-staged bf16 GEMM, taken only when a contraction length is not
a multiple of 64, is compiled and reported but not held to this.
"""

import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_cross_entropy_06_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")

SOURCES = ["gemm_bf16_dma.hip", "gemm_bf16.hip", "gemm_f32.hip", "ce_rows.hip",
           "grad_scale.hip", "rmsnorm.hip", "orpo.hip", "mfma_rate.hip", "flce_api.hip"]
FUSED = ["gemm_bf16_dma.hip", "gemm_f32.hip", "ce_rows.hip", "grad_scale.hip", "rmsnorm.hip",
         "orpo.hip", "mfma_rate.hip"]


def _report(src, out):
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, src),
           "-o", out, "-Rpass-analysis=kernel-resource-usage"]
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def _parse(text):
    """{kernel name: {field: int}} from the resource-usage remarks."""
    kernels, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+(.+?)(?: \[[^\]]*\])?: (\d+)", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = int(m.group(2))
    return kernels


@pytest.fixture(scope="module")
def reports():
    if HIPCC is None:
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as tmp:
        procs = {s: _report(s, os.path.join(tmp, s + ".o")) for s in SOURCES}
        out = {}
        for s, p in procs.items():
            text, _ = p.communicate(timeout=600)
            assert p.returncode == 0, f"{s} failed to compile:\n{text[-2000:]}"
            out[s] = _parse(text)
    return out


@pytest.mark.parametrize("src", FUSED)
def test_no_spills_or_scratch(reports, src):
    kernels = reports[src]
    assert kernels, f"no kernel reported for {src}"
    for name, f in kernels.items():
        assert f.get("VGPRs Spill", 0) == 0, (name, f)
        assert f.get("SGPRs Spill", 0) == 0, (name, f)
        assert f.get("ScratchSize", 0) == 0, (name, f)


def test_every_source_compiles_with_kernels(reports):
    for src in SOURCES:
        if src != "flce_api.hip":
            assert reports[src], src


def test_fused_path_kernels_fit_one_workgroup_per_cu(reports):
    for name, f in reports["gemm_bf16_dma.hip"].items():
        assert f["LDS Size"] <= 160 * 1024, (name, f)
        assert f["VGPRs"] <= 256 and f.get("AGPRs", 0) <= 256, (name, f)
