"""Codegen guard for the grouped GEMM (CPU only: cross-compiles for gfx950).

The K loop waits for its direct-to-LDS loads with explicit vmcnt counts, which
is only correct if those loads are the only vector-memory instructions inside
the loop (no compiler loads, stores or register spills to scratch).  This test
compiles gemm.hip to gfx950 assembly and checks exactly that for every K loop,
and that the steady-state loops are single basic blocks.
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
def test_k_loops_issue_only_direct_lds_loads(tmp_path):
    from sparse_moe_softmax_amd import build as B
    asm = tmp_path / "gemm.s"
    cmd = [B.HIPCC, *B.FLAGS, "--cuda-device-only", "-S", os.path.join(B.CSRC, "gemm.hip"), "-o", str(asm)]
    subprocess.run(cmd, check=True, capture_output=True)
    s = asm.read_text()
    kernels = re.findall(r"^(_ZN3moe9k_gemm_q4ILi\dEEEvNS_8GemmArgsE):", s, re.M)
    assert len(kernels) == 3
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
        assert len(k_loops) >= 2, k
        for h, v in k_loops.items():
            others = [o for o in v if o != "lds-load"]
            assert not others, (k, h, others)
