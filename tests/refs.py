"""Independent reference helpers used to pin the oracle (CPU only).

Nothing here calls the oracle.  Rounding to bfloat16 uses torch's float32 ->
bfloat16 conversion (a library routine, nearest-even); doubles are first
rounded to float32 *to odd*, which makes the later nearest-even rounding to
bfloat16 equal to a single rounding of the double (Boldo & Melquiond, "When
double rounding is odd", 2005: rounding to odd at p+2 or more bits followed by
rounding to nearest at p bits is a correct rounding).
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch


def round_to_odd_f32(v) -> np.ndarray:
    v = np.asarray(v, np.float64)
    f = v.astype(np.float32)
    # truncate toward zero
    over = np.abs(f.astype(np.float64)) > np.abs(v)
    f = np.where(over, np.nextafter(f, np.float32(0)), f)
    inexact = f.astype(np.float64) != v
    bits = f.view(np.uint32)
    even = (bits & 1) == 0
    away = np.where(v < 0, np.float32(-np.inf), np.float32(np.inf))
    f = np.where(inexact & even, np.nextafter(f, away), f)
    return f.astype(np.float32)


def bf16_rn_f32(f) -> np.ndarray:
    """Nearest-even bfloat16 of float32 values (torch), returned as float64."""
    t = torch.from_numpy(np.ascontiguousarray(f, np.float32))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def bf16_rn(v) -> np.ndarray:
    """Single nearest-even rounding of doubles to bfloat16 (returned as float64)."""
    return bf16_rn_f32(round_to_odd_f32(v))


def bf16_bits_of(v) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(round_to_odd_f32(v)))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_rn_fraction(x: float) -> Fraction:
    """Exact nearest-even bfloat16 rounding by rational arithmetic (slow)."""
    q = Fraction(x)
    if q == 0:
        return q
    sign = -1 if q < 0 else 1
    a = abs(q)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    spacing_exp = max(e - 7, -133)
    unit = Fraction(2) ** spacing_exp
    n = a / unit
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * unit


def unpack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] codes, low nibble = even element."""
    lo = codes & 0x0F
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)


def dequant_ref(codes, scales_u16, biases_u16, G: int) -> np.ndarray:
    """Dequantised bf16 weights (float64) via numpy float32 arithmetic + torch rounding."""
    c = unpack_nibbles(np.asarray(codes, np.uint8)).astype(np.float32)
    s = np.asarray(scales_u16, np.uint16).view(np.float16).astype(np.float32)
    b = np.asarray(biases_u16, np.uint16).view(np.float16).astype(np.float32)
    s = np.repeat(s, G, axis=-1)
    b = np.repeat(b, G, axis=-1)
    v = (c * s).astype(np.float32) + b        # two float32 roundings, as the format defines
    return bf16_rn_f32(v.astype(np.float32))


def topk_ref(logits: np.ndarray, k: int):
    """Brute force: full ranking by (-logit, expert) with Python's sort; scipy softmax."""
    from scipy.special import softmax
    T, E = logits.shape
    ids = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float32)
    for t in range(T):
        row = [float(v) for v in logits[t]]
        order = sorted(range(E), key=lambda e: (-row[e], e))[:k]
        p = softmax(logits[t].astype(np.float64))
        sel = p[order]
        ids[t] = order
        w[t] = (sel / sel.sum()).astype(np.float32)
    return ids, w


def silu(z):
    return z / (1.0 + np.exp(-z))


def layer_ref(x_bits, ids, w, g, W, dims):
    """Dense numpy fp64 reference of the expert part of the layer (tiny dims).

    W: dict with dequantised float64 matrices: gu[E][2I][H], dn[E][H][I],
    sgu[2Is][H], sdn[H][Is].  Returns (out bf16 float64 values, y float64).
    """
    H, I, k, Is = dims.hidden, dims.inter, dims.top_k, dims.shared_inter
    x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).double().numpy()
    T = x.shape[0]
    y = np.zeros((T, H), np.float64)
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            gu = W["gu"][e] @ x[t]
            h = bf16_rn(silu(gu[:I]) * gu[I:])
            o = W["dn"][e] @ h
            y[t] += np.float64(w[t, j]) * o
        gu = W["sgu"] @ x[t]
        h = bf16_rn(silu(gu[:Is]) * gu[Is:])
        o = W["sdn"] @ h
        y[t] += np.float64(g[t]) * o
    return bf16_rn(y), y
