"""The kernels' compile-time variants (the -D switches the measured
alternatives are built with, `python -m geometric_context_attention_amd.build
-D NAME=V`) still compile for gfx950: a semantic check of the device and host
code of gca_kernels.hip for each, no code generation."""
import os
import subprocess

import pytest

from geometric_context_attention_amd import build as B

VARIANTS = [
    ["GCA_PINGPONG=0"],
    ["GCA_RING=5", "GCA_AHEAD=3"],
    ["GCA_SOFT_EXP=4"],
    ["GCA_SOFT_EXP=8"],
    ["GCA_ASYM_ARGS=1"],
    ["GCA_QSCALE=1"],
    ["GCA_KPREFETCH=1"],
    ["GCA_SUM_CHAINS=2"],
    ["GCA_SUM_CHAINS=4"],
    ["GCA_STAGE_MFMA=1"],
    ["GCA_FRAME_RING=0"],
    ["GCA_FRAME_PERSIST=0"],
    ["GCA_WS_VROW=0"],
    ["GCA_WS_BATCH_MAX=2"],
    ["GCA_PHASE_TIMING=1"],
]


@pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("defines", VARIANTS, ids=lambda d: ",".join(d))
def test_variant_compiles(defines):
    cmd = [B.HIPCC, *B.DEVICE_FLAGS, *[f"-D{d}" for d in defines], "-I", os.path.join(B.ROOT, "include"),
           "-fsyntax-only", os.path.join(B.CSRC, "gca_kernels.hip")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
