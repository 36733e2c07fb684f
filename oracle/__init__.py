"""CPU oracle for the sparse-MoE layer (test infrastructure).

Only the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and its
binding) never does, and this package never imports the product path.

The arithmetic lives in ``moe_oracle.cpp`` (plain C++, double accumulation,
explicit bfloat16 rounding points); this module only marshals numpy arrays into
it.  Each wrapper names the step of the layer it computes; the step definitions
follow the pages' description of the MoE layer ("Lily: Perplexity's Custom
Inference Engine for Apple Silicon", section "The architecture that forces the
issue: MoE plus Gated DeltaNet"; "Inside Lily ...", section "Performance Gains
and Workload Patterns") with the readings listed in the oracle source header.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.cpp")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

_lib_handle = None


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (-O2, no FP contraction, no fast-math)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp"
    cmd = ["g++", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c++17", "-fPIC", "-shared",
           "-pthread", _SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_LIB):
            build()
        _lib_handle = ctypes.CDLL(_LIB)
        _declare(_lib_handle)
    return _lib_handle


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int


def _declare(lib):
    lib.oracle_abi_version.restype = _INT
    sigs = {
        "oracle_round_bf16": [_P, _P, _I64],
        "oracle_bf16_bits": [_P, _P, _I64],
        "oracle_half_to_double": [_P, _P, _I64],
        "oracle_bf16_to_double": [_P, _P, _I64],
        "oracle_dequant": [_P, _P, _P, _I64, _I64, _I64, _P],
        "oracle_router": [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _INT],
        "oracle_topk": [_P, _I64, _I64, _I64, _P, _P],
        "oracle_sigmoid": [_P, _I64, _P],
        "oracle_group": [_P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _I64, _P],
        "oracle_grouped_swiglu": [_I64, _I64, _I64, _I64, _I64, _P, _INT, _P, _P, _P, _P, _P, _P, _INT],
        "oracle_grouped_down": [_I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _INT],
        "oracle_moe_tokens": [_I64] * 6 + [_P] * 16 + [_P, _I64, _P, _P, _P, _P, _INT],
        "oracle_gqa_decode": [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, ctypes.c_double, _P, _INT],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = _INT if name == "oracle_group" else None


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------- numbers

def round_bf16(v) -> np.ndarray:
    """Nearest-even bfloat16 value of each double (returned as float64)."""
    v = _c(v, np.float64)
    out = np.empty_like(v)
    _lib().oracle_round_bf16(_ptr(v), _ptr(out), v.size)
    return out


def bf16_bits(v) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of nearest-even rounding of doubles."""
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    _lib().oracle_bf16_bits(_ptr(v), _ptr(out), v.size)
    return out


def half_to_double(h) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float64)
    _lib().oracle_half_to_double(_ptr(h), _ptr(out), h.size)
    return out


def bf16_to_double(b) -> np.ndarray:
    b = _c(b, np.uint16)
    out = np.empty(b.shape, np.float64)
    _lib().oracle_bf16_to_double(_ptr(b), _ptr(out), b.size)
    return out


def dequant(codes, scales, biases, N: int, K: int, G: int) -> np.ndarray:
    """Dequantised [N][K] matrix (bf16 values as float64) of one expert."""
    codes = _c(codes, np.uint8).reshape(-1)
    scales = _c(scales, np.uint16).reshape(-1)
    biases = _c(biases, np.uint16).reshape(-1)
    assert codes.size == N * K // 2 and scales.size == N * K // G and biases.size == scales.size
    out = np.empty((N, K), np.float64)
    _lib().oracle_dequant(_ptr(codes), _ptr(scales), _ptr(biases), N, K, G, _ptr(out))
    return out


# --------------------------------------------------------------------- routing

def router(x_bits, W, bias=None, wsg=None, threads: int = 0):
    """Router logits [T][E] (fp32) and shared-gate logits [T] (fp32, or None)."""
    x_bits = _c(x_bits, np.uint16)
    T, H = x_bits.shape
    W = _c(W, np.float32)
    E = W.shape[0]
    assert W.shape == (E, H)
    bias = None if bias is None else _c(bias, np.float32)
    wsg = None if wsg is None else _c(wsg, np.float32)
    logits = np.empty((T, E), np.float32)
    s = np.empty((T,), np.float32) if wsg is not None else None
    _lib().oracle_router(_ptr(x_bits), T, H, E, _ptr(W), _ptr(bias), _ptr(wsg), _ptr(logits), _ptr(s), threads)
    return logits, s


def topk(logits, k: int):
    """(ids int32 [T][k], weights fp32 [T][k]): softmax, top-k by logit, renormalised."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _lib().oracle_topk(_ptr(logits), T, E, k, _ptr(ids), _ptr(w))
    return ids, w


def sigmoid(s) -> np.ndarray:
    s = _c(s, np.float32)
    g = np.empty_like(s)
    _lib().oracle_sigmoid(_ptr(s), s.size, _ptr(g))
    return g


@dataclass
class Grouping:
    counts: np.ndarray
    offsets: np.ndarray
    perm: np.ndarray
    inv_perm: np.ndarray
    block_map: np.ndarray
    n_tiles: int


def max_tiles(T: int, k: int, E: int, BM: int) -> int:
    """Upper bound on the number of tiles of height BM: ceil(T*k/BM) + E."""
    return (T * k + BM - 1) // BM + E


def group(ids, E: int, BM: int, n_max_tiles: int | None = None) -> Grouping:
    ids = _c(ids, np.int32)
    T, k = ids.shape
    F = T * k
    mt = max_tiles(T, k, E, BM) if n_max_tiles is None else n_max_tiles
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(F, np.int32)
    inv = np.empty(F, np.int32)
    bmap = np.empty((mt, 2), np.int32)
    nt = np.zeros(1, np.int32)
    rc = _lib().oracle_group(_ptr(ids), T, k, E, BM, _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv),
                             _ptr(bmap), mt, _ptr(nt))
    if rc != 0:
        raise ValueError("block map does not fit in max_tiles")
    return Grouping(counts, offsets, perm, inv, bmap, int(nt[0]))


# --------------------------------------------------------------------- experts

def grouped_swiglu(a_bits, rows_are_tokens: bool, k: int, perm, offsets, q4, H: int, I: int, G: int,
                   threads: int = 0) -> np.ndarray:
    """h [n_rows][I] (bf16 bits) for every grouped position p (see oracle source)."""
    codes, scales, biases = (_c(q4[0], np.uint8), _c(q4[1], np.uint16), _c(q4[2], np.uint16))
    a_bits = _c(a_bits, np.uint16)
    offsets = _c(offsets, np.int32)
    perm = _c(perm, np.int32)
    E = offsets.size - 1
    n_rows = int(offsets[-1])
    h = np.zeros((n_rows, I), np.uint16)
    _lib().oracle_grouped_swiglu(H, I, E, G, k, _ptr(a_bits), int(rows_are_tokens), _ptr(perm), _ptr(offsets),
                                 _ptr(codes), _ptr(scales), _ptr(biases), _ptr(h), threads)
    return h


def grouped_down(h_bits, offsets, q4, H: int, I: int, G: int, threads: int = 0) -> np.ndarray:
    """o [n_rows][H] (float64) = h[p] . Wd[e(p)]^T for every grouped position p."""
    codes, scales, biases = (_c(q4[0], np.uint8), _c(q4[1], np.uint16), _c(q4[2], np.uint16))
    h_bits = _c(h_bits, np.uint16)
    offsets = _c(offsets, np.int32)
    E = offsets.size - 1
    n_rows = int(offsets[-1])
    o = np.zeros((n_rows, H), np.float64)
    _lib().oracle_grouped_down(H, I, E, G, _ptr(h_bits), _ptr(offsets), _ptr(codes), _ptr(scales), _ptr(biases),
                               _ptr(o), threads)
    return o


@dataclass
class LayerWeights:
    """Host copies of one layer's weights in the canonical layout.

    gate_up/down/sh_gate_up/sh_down are (codes uint8, scales uint16, biases uint16)
    with codes [n_exp][N][K/2] and scales/biases [n_exp][N][K/G] (fp16 bits).
    """
    gate_up: tuple
    down: tuple
    sh_gate_up: tuple
    sh_down: tuple
    router_w: np.ndarray          # [E][H] fp32
    shared_gate_w: np.ndarray     # [H] fp32
    router_bias: np.ndarray | None = None  # [E] fp32


@dataclass
class Dims:
    hidden: int = 2048
    inter: int = 512
    n_experts: int = 256
    top_k: int = 8
    group_size: int = 64
    shared_inter: int = 512


def moe_tokens(d: Dims, x_bits, ids, w, g, lw: LayerWeights, tokens=None, threads: int = 0,
               want_y: bool = False, want_h: bool = False):
    """Layer output for the listed tokens given routing (ids, w, g).

    Returns (out bf16 bits [n][H], y float64 [n][H] or None, h or None, h_sh or None).
    """
    x_bits = _c(x_bits, np.uint16)
    T = x_bits.shape[0]
    ids = _c(ids, np.int32)
    w = _c(w, np.float32)
    g = _c(g, np.float32)
    tokens = np.arange(T, dtype=np.int32) if tokens is None else _c(tokens, np.int32)
    n = tokens.size
    H, I, E, k, G, Is = d.hidden, d.inter, d.n_experts, d.top_k, d.group_size, d.shared_inter
    out = np.empty((n, H), np.uint16)
    y = np.empty((n, H), np.float64) if want_y else None
    h = np.empty((n, k, I), np.uint16) if want_h else None
    hs = np.empty((n, Is), np.uint16) if want_h else None
    q = [tuple(_c(a, dt) for a, dt in zip(m, (np.uint8, np.uint16, np.uint16)))
         for m in (lw.gate_up, lw.down, lw.sh_gate_up, lw.sh_down)]
    flat = [p for m in q for p in (_ptr(m[0]), _ptr(m[1]), _ptr(m[2]))]
    _lib().oracle_moe_tokens(H, I, E, k, G, Is, _ptr(x_bits), _ptr(ids), _ptr(w), _ptr(g), *flat, _ptr(tokens), n,
                             _ptr(out), _ptr(y), _ptr(h), _ptr(hs), threads)
    return out, y, h, hs


def layer(d: Dims, x_bits, lw: LayerWeights, tokens=None, logits=None, s=None, threads: int = 0):
    """Whole layer: router -> top-k -> experts -> combine.

    ``logits``/``s`` may be supplied (e.g. another implementation's fp32
    logits) so that routing is taken from exactly those values.
    Returns dict with logits, s, ids, w, g, out (bf16 bits for ``tokens``).
    """
    if logits is None:
        logits, s = router(x_bits, lw.router_w, lw.router_bias, lw.shared_gate_w, threads)
    ids, w = topk(logits, d.top_k)
    g = sigmoid(s)
    out, _, _, _ = moe_tokens(d, x_bits, ids, w, g, lw, tokens=tokens, threads=threads)
    return {"logits": logits, "s": s, "ids": ids, "w": w, "g": g, "out": out}


# --------------------------------------------------------------------- attention

def gqa_decode(q_bits, k_bits, v_bits, lens, scale: float, threads: int = 0) -> np.ndarray:
    """One decode step of grouped-query attention, [B][Hq][D] float64 (unrounded).

    q_bits [B][Hq][D], k_bits / v_bits [B][Hkv][S][D] (bf16 bit patterns),
    lens [B] positions in use.  Query head h reads key/value head h // (Hq // Hkv)
    (Lily page, section "The architecture that forces the issue": 16 query heads
    share 2 key/value heads)."""
    q_bits = _c(q_bits, np.uint16)
    k_bits = _c(k_bits, np.uint16)
    v_bits = _c(v_bits, np.uint16)
    lens = _c(lens, np.int32)
    B, Hq, D = q_bits.shape
    _, Hkv, S, _ = k_bits.shape
    assert k_bits.shape == (B, Hkv, S, D) and v_bits.shape == k_bits.shape and lens.shape == (B,)
    assert Hq % Hkv == 0 and np.all((lens >= 0) & (lens <= S))
    out = np.empty((B, Hq, D), np.float64)
    _lib().oracle_gqa_decode(_ptr(q_bits), _ptr(k_bits), _ptr(v_bits), _ptr(lens), B, Hq, Hkv, S, D,
                             float(scale), _ptr(out), threads)
    return out
