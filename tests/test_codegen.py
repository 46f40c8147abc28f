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


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_decode_score_kernel_keeps_four_waves_per_simd(tmp_path):
    """The decode score pass is bound by how many key loads are in flight: its 64-head bf16
    instantiation must fit four waves per SIMD (at most 128 VGPRs) without spilling."""
    src = os.path.join(HERE, "..", "dsa_indexer_indexcache_amd", "csrc", "indexer_slab.hip")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "--cuda-device-only", "-c", src, "-o", str(tmp_path / "k.o"),
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    stats, name = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        if name and "idx_score_bf16_kernelILi4ELi128" in name:
            for key in ("VGPRs", "AGPRs", "VGPRs Spill", "Occupancy \\[waves/SIMD\\]"):
                m = re.search(r"remark:\s+" + key + r": (\d+)", line)
                if m:
                    stats[key.split(" ")[0] if key != "VGPRs Spill" else "spill"] = int(m.group(1))
    assert stats, "no idx_score_bf16_kernel<4, 128> in the resource report"
    assert stats.get("spill", 0) == 0, stats
    assert stats["VGPRs"] + stats.get("AGPRs", 0) <= 128, stats
    assert stats["Occupancy"] >= 4, stats


def _kernel_bodies(asm: str, name_part: str):
    """Assembly text of every kernel whose mangled name contains name_part."""
    out, cur = [], None
    for line in asm.splitlines():
        if cur is None:
            if re.match(r"^_Z\S*:", line) and name_part in line:
                cur = []
        else:
            cur.append(line)
            if "s_endpgm" in line:
                out.append(cur)
                cur = None
    return out


def _scratch_reload_with_copies_in_flight(body):
    """Inside every loop that issues direct-to-LDS copies, a scratch reload between a
    copy and the next s_waitcnt vmcnt(0) would wait for all copies in flight (the
    counter completes in order) and serialise them.  Returns the offending lines."""
    bad = []
    headers = [(i, l.split(":")[0]) for i, l in enumerate(body) if re.match(r"^\.LBB\S+:", l) and "Loop Header" in l]
    for h, label in headers:
        ends = [i for i, l in enumerate(body) if i > h and re.search(r"s_c?branch\w*\s+" + re.escape(label) + r"\b", l)]
        if not ends:
            continue
        seg = body[h:max(ends) + 1]
        if not any("global_load_lds" in l for l in seg):
            continue
        inflight = False
        for l in seg:
            if "global_load_lds" in l:
                inflight = True
            elif re.search(r"s_waitcnt\s+vmcnt\(0\)", l):
                inflight = False
            elif inflight and "scratch_load" in l:
                bad.append(l.strip())
    return bad


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src,kernel", [("sparse_attn.hip", "sparse_attn_pair_kernel"),
                                        ("sparse_attn.hip", "sparse_attn_pair2_kernel"),
                                        ("indexer_fused.hip", "idx_topk_fused_kernel")])
def test_no_spill_reload_while_lds_copies_are_in_flight(tmp_path, src, kernel):
    path = os.path.join(HERE, "..", "dsa_indexer_indexcache_amd", "csrc", src)
    out = tmp_path / "k.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "--cuda-device-only", "-S", path, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    bodies = _kernel_bodies(out.read_text(), kernel)
    assert bodies, "no %s in the assembly" % kernel
    for body in bodies:
        assert not _scratch_reload_with_copies_in_flight(body)


def _scratch_reload_in_copy_loops(body):
    """Every scratch reload inside a loop that issues direct-to-LDS copies (a loop-invariant
    value spilled and reloaded each iteration puts a memory wait on every pass)."""
    bad = []
    headers = [(i, l.split(":")[0]) for i, l in enumerate(body) if re.match(r"^\.LBB\S+:", l) and "Loop Header" in l]
    for h, label in headers:
        ends = [i for i, l in enumerate(body) if i > h and re.search(r"s_c?branch\w*\s+" + re.escape(label) + r"\b", l)]
        if not ends:
            continue
        seg = body[h:max(ends) + 1]
        if any("global_load_lds" in l for l in seg):
            bad += [l.strip() for l in seg if "scratch_load" in l]
    return bad


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_attention_block_loop_has_no_spill_reload(tmp_path):
    path = os.path.join(HERE, "..", "dsa_indexer_indexcache_amd", "csrc", "sparse_attn.hip")
    out = tmp_path / "k.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "--cuda-device-only", "-S", path, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    bodies = _kernel_bodies(asm, "sparse_attn_pair_kernel") + _kernel_bodies(asm, "sparse_attn_pair2_kernel")
    assert len(bodies) == 4  # 16 heads per pair (decode) and 32 heads per pair with 2, 4 and 8 waves
    for body in bodies:
        assert not _scratch_reload_in_copy_loops(body)


def test_reload_scanner_flags_a_reload_after_a_copy():
    loop = [".LBB0_3:                                ; =>This Inner Loop Header: Depth=1",
            "\ts_waitcnt vmcnt(0)", "\ts_barrier", "\tglobal_load_lds_dwordx4 v[2:3], off",
            "\tv_mfma_f32_16x16x32_bf16 v[4:7], v[8:11], v[12:15], v[4:7]",
            "\tscratch_load_dword v0, off, off offset:8", "\ts_cbranch_scc0 .LBB0_3"]
    assert _scratch_reload_with_copies_in_flight(loop) == ["scratch_load_dword v0, off, off offset:8"]
    ok = loop[:5] + ["\ts_waitcnt vmcnt(0)"] + loop[5:]
    assert _scratch_reload_with_copies_in_flight(ok) == []
    assert _scratch_reload_in_copy_loops(ok) == ["scratch_load_dword v0, off, off offset:8"]
