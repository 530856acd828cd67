"""Build checks for the gfx950 kernels (no GPU): every kernel compiles without
register spills or scratch memory, and fits the residency the launch assumes.

The kernels sit close to the 256-register budget of two waves per SIMD (one
eight-wave workgroup per CU), so a source change that tips one into spilling
would slow it down silently;
this test makes that loud. The figures come from the compiler's
kernel-resource-usage remarks for our own gfx950 build.
"""

import os
import re
import subprocess

import pytest

import moe_ragged_grouped_amd.build as hb

pytestmark = pytest.mark.skipif(not os.path.exists(hb.HIPCC), reason="hipcc not available")


def _resources():
    cmd = [hb.HIPCC, *[f for f in hb.FLAGS if f not in ("-shared",)], "--offload-device-only",
           "-c", "-Rpass-analysis=kernel-resource-usage", "-o", os.devnull, *hb.SOURCES]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels = {}
    cur = None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z /\[\]]+?):\s+(\d+)", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = int(m.group(2))
    return kernels


@pytest.fixture(scope="module")
def resources():
    return _resources()


def test_no_spills_no_scratch(resources):
    gemm = {k: v for k, v in resources.items() if "grouped_gemm_kernel" in k}
    # five single heights + the per-expert mix, each for fp32 C, bf16 C,
    # bf16 SwiGLU output, fp32 C with gathered / scattered rows, the weighted
    # combine, fp8 weights, and fp8 activations with fp8 weights (fp32 C,
    # bf16 C and bf16 SwiGLU output)
    assert len(gemm) == 54, sorted(resources)
    for name, r in resources.items():
        assert r.get("VGPRs Spill", 0) == 0, (name, r)
        assert r.get("SGPRs Spill", 0) == 0, (name, r)
        assert r.get("ScratchSize [bytes/lane]", 0) == 0, (name, r)


def test_two_waves_per_simd(resources):
    # eight waves per workgroup and one workgroup per CU: two waves per SIMD,
    # so at most 256 registers (VGPR + AGPR) per wave
    for name, r in resources.items():
        if "grouped_gemm_kernel" in name:
            assert r.get("VGPRs", 0) + r.get("AGPRs", 0) <= 256, (name, r)
            assert r.get("Occupancy [waves/SIMD]", 0) >= 2, (name, r)
