"""The matrix-core kernels accumulate in AGPRs.

Compiled so that its accumulators lived in VGPRs (a forced occupancy of two
wavefronts per SIMD), the staged matrix-core gate/up kernel gave wrong outputs
on one layer shape, and its assembly held MFMAs whose VGPR destination was also
their A source (v_mfma_f32_16x16x32_bf16 v[2:5], v[2:5], ...).  Every MFMA of
the shipped kernels writes an AGPR destination, which cannot alias the VGPR
operands; this test compiles the GEMV source for gfx950 and checks that it
stays so."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from hbm_expert_slot_amd import build as B

SRC = os.path.join(B.HERE, "csrc", "expert_gemv.hip")


def _assembly():
    cc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cc):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "expert_gemv.s")
        cmd = [cc] + B.FLAGS + ["-I" + os.path.join(B.HERE, "csrc"), "--cuda-device-only", "-S", SRC, "-o", out]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        assert r.returncode == 0, r.stdout[-2000:]
        return open(out).read()


def test_every_mfma_accumulates_in_agprs():
    asm = _assembly()
    mfma = re.findall(r"^\s*(v_mfma\S*)\s+([^,\s]+),", asm, flags=re.M)
    assert len(mfma) > 100, "no matrix-core kernels found"
    vgpr_dst = [(op, d) for op, d in mfma if not d.startswith("a")]
    assert not vgpr_dst, "MFMAs with VGPR destinations: %s" % vgpr_dst[:5]
