"""Register and scratch budget of the Newton-Schulz GEMM kernels (CPU: hipcc
cross-compiles for gfx950).

Every instantiation of ns_gemm_kernel must run without scratch memory: no
spilled VGPRs or SGPRs and no private segment.  A spill or an accumulator
array indexed dynamically (a loop the compiler failed to unroll) shows up
here as a nonzero count in the code object's metadata, long before it shows
up as lost time on the GPU.  The flags are the library build's own.
"""

import os
import re
import shutil
import subprocess

import pytest

from matrix_aware_optimizer_step_amd import build as B


def _metadata(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path / "ns_gemm.s"
    cmd = [hipcc, *[f for f in B.COMMON if f != "-fPIC"], *B.EXTRA.get("ns_gemm.hip", []), "-x", "hip",
           "--cuda-device-only", "-S", os.path.join(B.CSRC, "ns_gemm.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert res.returncode == 0, res.stderr[-3000:]
    assert "loop not unrolled" not in res.stderr, res.stderr[-3000:]
    text = out.read_text()
    kernels = {}
    for block in re.split(r"\n\s+- \.", text):
        m = re.search(r"\.name:\s+(\S*ns_gemm_kernel\S*)", block)
        if not m:
            continue
        vals = {k: int(v) for k, v in re.findall(r"\.(private_segment_fixed_size|vgpr_spill_count|sgpr_spill_count|"
                                                   r"vgpr_count):\s+(\d+)", block)}
        kernels[m.group(1)] = vals
    return kernels


def test_ns_gemm_kernels_use_no_scratch(tmp_path):
    kernels = _metadata(tmp_path)
    # 2 element types x 2 tile sizes x (Gram, polynomial, update, last step,
    # last step with the update applied)
    assert len(kernels) == 20, sorted(kernels)
    for name, v in kernels.items():
        assert v.get("private_segment_fixed_size", 0) == 0, (name, v)
        assert v.get("vgpr_spill_count", 0) == 0, (name, v)
        assert v.get("sgpr_spill_count", 0) == 0, (name, v)
        assert 0 < v["vgpr_count"] <= 256, (name, v)
