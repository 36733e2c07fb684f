"""Codegen guard for the grouped GEMM and the router GEMM (CPU only:
cross-compiles for gfx950).

The K loop waits for its direct-to-LDS loads with explicit vmcnt counts, which
is only correct if those loads are the only vector-memory instructions inside
the loop (no compiler loads, stores or register spills to scratch).  This test
compiles gemm.hip and route.hip to gfx950 assembly and checks exactly that for
every K loop.
"""

import os
import re
import shutil
import subprocess
from collections import defaultdict

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("/opt/rocm/bin/hipcc") is None and shutil.which("hipcc") is None,
                    reason="hipcc not available")
@pytest.mark.parametrize("src,pattern,count,min_loops", [
    ("gemm.hip", r"^(_ZN3moe9k_gemm_q4ILi\dEEEvNS_8GemmArgsE):", 3, 2),
    ("route.hip", r"^(_ZN3moe\d+k_router_gemm\w*EPKtS1_PKfS3_iiiiPfS4_):", 2, 1),
])
def test_k_loops_issue_only_direct_lds_loads(tmp_path, src, pattern, count, min_loops):
    from sparse_moe_softmax_amd import build as B
    asm = tmp_path / (src + ".s")
    cmd = [B.HIPCC, *B.FLAGS, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", str(asm)]
    subprocess.run(cmd, check=True, capture_output=True)
    s = asm.read_text()
    kernels = re.findall(pattern, s, re.M)
    assert len(kernels) == count
    assert "scratch_" not in s, "register spills to scratch memory"
    for k in kernels:
        a = s.index(k + ":")
        b = s.index(".Lfunc_end", a)
        ops = defaultdict(list)
        cur = None
        for line in s[a:b].split("\n"):
            if line.startswith(".LBB") or line.startswith("; %bb"):
                cur = None
                m = re.search(r"Header=(\S+)", line)
                if "Loop Header" in line:
                    cur = line.split(":")[0].strip().lstrip(".").lstrip("L")
                elif m:
                    cur = m.group(1)
                continue
            text = line.strip()
            op = text.split(" ")[0]
            if cur and re.match(r"(global_|buffer_|scratch_|flat_)", op):
                ops[cur].append("lds-load" if re.match(r"(global|buffer)_load_\w+ .* lds$", text) else text)
        k_loops = {h: v for h, v in ops.items() if "lds-load" in v}
        assert len(k_loops) >= min_loops, k
        for h, v in k_loops.items():
            others = [o for o in v if o != "lds-load"]
            assert not others, (k, h, others)


@pytest.mark.skipif(shutil.which("/opt/rocm/bin/hipcc") is None and shutil.which("hipcc") is None,
                    reason="hipcc not available")
def test_fused_layer_keeps_its_arrays_in_registers(tmp_path):
    """The fused 1-4-token layer holds x, the prefetched weight rows and the
    partial sums in register arrays.  A code change can silently turn them into
    per-lane stack memory (a lambda capturing them by reference that is not
    inlined, a helper with too many call sites): the layer then ran ~60%
    slower.  Every form but the widest (k > 8 with hidden and inter both at
    their largest) must use no private segment."""
    from sparse_moe_softmax_amd import build as B
    asm = tmp_path / "decode.s"
    cmd = [B.HIPCC, *B.FLAGS, "--cuda-device-only", "-S", os.path.join(B.CSRC, "decode.hip"), "-o", str(asm)]
    subprocess.run(cmd, check=True, capture_output=True)
    s = asm.read_text()
    meta = re.findall(r"\.name:\s+(_ZN3moe14k_decode_layerILi(\d)ELi(\d)ELi(\d+)ELi(\d)EEEvNS_7DecArgsE)"
                      r"[\s\S]*?\.private_segment_fixed_size:\s+(\d+)", s)
    if not meta:   # metadata keys in the other order
        meta = re.findall(r"\.private_segment_fixed_size:\s+(\d+)[\s\S]*?\.name:\s+"
                          r"(_ZN3moe14k_decode_layerILi(\d)ELi(\d)ELi(\d+)ELi(\d)EEEvNS_7DecArgsE)", s)
        meta = [(n, a, b, c, d, p) for p, n, a, b, c, d in meta]
    assert len(meta) == 9, meta
    for name, kcg, kcd, kmax, tm, priv in meta:
        if (kcg, kcd, kmax) == ("2", "2", "16"):
            continue
        assert int(priv) == 0, (name, priv)
