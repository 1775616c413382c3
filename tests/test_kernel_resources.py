"""Build check: every HIP kernel of the library compiles for gfx950 without
scratch memory or register spills (a private-memory slot in a hot loop, e.g. from
a by-reference lambda output, silently costs a large part of the GEMM's speed)."""

import os
import re
import subprocess

import pytest

from bit_w4a4_quantized_quantize_amd import build

HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", ["gemm_lds.hip", "gemm_bf16.hip", "gemm_w4a4.hip", "gemm_mx.hip", "quant_lora.hip",
                                 "quant_act.hip", "repack.hip", "prep.hip", "calib.hip"])
def test_no_scratch_no_spills(src, tmp_path):
    path = os.path.join(build.CSRC, src)
    cmd = [HIPCC, *build.COMMON_FLAGS, "-I", build.INCLUDE, "-I", build.CSRC, "--cuda-device-only", "-c", path,
           "-o", str(tmp_path / "k.o"), "-Rpass-analysis=kernel-resource-usage"]
    out = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stderr[-2000:]
    names = re.findall(r"Function Name: (\S+)", out.stderr)
    scratch = [int(v) for v in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", out.stderr)]
    spills = [int(v) for v in re.findall(r"VGPRs Spill: (\d+)", out.stderr)]
    assert names and len(names) == len(scratch) == len(spills)
    bad = [(n, sc, sp) for n, sc, sp in zip(names, scratch, spills) if sc or sp]
    assert not bad, f"kernels with scratch/spills: {bad}"
