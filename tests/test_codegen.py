"""Code-generation guard for the fused indexer kernel (CPU; needs hipcc).

The fused kernel keeps q, the head weights and the 2048-entry top-k state in
registers across the compaction code.  Under register pressure the compiler has
been seen to split a live range by a copy placed inside a lane-divergent region,
so that the lanes inactive there lost a loop-invariant copy address and later key
tiles landed in the wrong LDS rows.  Every instantiation must therefore stay below
the register limit without VGPR spills.
"""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "..", "dsa_indexer_indexcache_amd", "csrc", "indexer_fused.hip")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_fused_indexer_has_no_vgpr_spills(tmp_path):
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "--cuda-device-only", "-c", SRC, "-o", str(tmp_path / "k.o"),
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels, name = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"VGPRs Spill: (\d+)", line)
        if m and name and "idx_topk_fused_kernel" in name:
            kernels[name] = int(m.group(1))
    assert len(kernels) == 9, kernels
    assert all(v == 0 for v in kernels.values()), kernels
