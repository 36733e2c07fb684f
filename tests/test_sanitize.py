"""Sanitizer builds of the host code (CPU only).

* The oracle, built with AddressSanitizer and UndefinedBehaviorSanitizer by
  g++, runs every entry point on small inputs (tests/sanitize/oracle_driver.cpp).
* The HIP library, its host code instrumented the same way (device code as
  usual), drives every C-ABI entry point's argument checks, workspace carving,
  host block map and queries (tests/sanitize/abi_driver.cpp).  Without a GPU
  the launch paths end in MOE_ERR_HIP and are checked to do so.

Any report (out-of-bounds access, use after free, leak, undefined behaviour)
fails the run: the instrumented code aborts on the first one.
"""

from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
SAN = "address,undefined"
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
CSRC = os.path.join(ROOT, "sparse_moe_softmax_amd", "csrc")


def _digest(paths, extra=""):
    h = hashlib.sha256(extra.encode())
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def _env():
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_oracle_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    srcs = [os.path.join(ROOT, "oracle", "moe_oracle.cpp"), os.path.join(ROOT, "tests", "sanitize", "oracle_driver.cpp")]
    exe = os.path.join(OUT, f"oracle_driver_{_digest(srcs)}")
    if not os.path.exists(exe):
        _run(["g++", "-std=c++17", "-O1", "-g", f"-fsanitize={SAN}", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer", "-ffp-contract=off", *srcs, "-o", exe, "-lpthread"])
    r = subprocess.run([exe], capture_output=True, text=True, env=_env(), timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "oracle driver: ok" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not available")
def test_abi_host_code_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    from sparse_moe_softmax_amd import build as B
    hip = [os.path.join(CSRC, f) for f in B.SOURCES]
    hdrs = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith(".hpp")]
    drv = os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp")
    tag = _digest(hip + hdrs + [drv, os.path.join(ROOT, "include", "moe.h")])
    exe = os.path.join(OUT, f"abi_driver_{tag}")
    if not os.path.exists(exe):
        # host code instrumented: each sanitizer flag applies to the host pass only
        host_san = f"-Xarch_host -fsanitize={SAN} -Xarch_host -fno-sanitize-recover=all".split()
        common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Wno-inline-asm",
                  "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

        def obj(src):
            o = os.path.join(OUT, os.path.basename(src) + f".{tag}.o")
            _run([HIPCC, *common, *host_san, "-c", src, "-o", o])
            return o

        with ThreadPoolExecutor(max_workers=6) as ex:
            objs = list(ex.map(obj, hip))
        dobj = os.path.join(OUT, f"abi_driver.{tag}.o")
        _run([HIPCC, "-x", "c++", "-std=c++17", "-O1", "-g", f"-fsanitize={SAN}", "-fno-sanitize-recover=all",
              "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-c", drv, "-o", dobj])
        _run([CLANG, f"-fsanitize={SAN}", dobj, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
              "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True, env=_env(), timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "abi driver: ok" in r.stdout
