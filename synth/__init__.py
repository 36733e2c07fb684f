"""Seeded synthetic inputs for the sparse-MoE layer.

Shared by the tests, the benchmark and the smoke check, for both the HIP path
and the CPU oracle.  This module only draws numbers; it contains none of the
layer's arithmetic.

Recipe (every draw is a pure function of the seed, so any part can be rebuilt):

* activations x ~ N(0, 1), rounded to bfloat16 (torch CPU generator);
* router weights W_r ~ N(0, 1/H) fp32 [E][H]; shared-gate weights w_sg ~ N(0, 1/H) fp32 [H];
* int4 codes uniform on {0..15}; fp16 scales uniform on [0.005, 0.02) (drawn on
  the 2^-18 grid, then rounded to fp16); biases = -8 * scale (exact in fp16).
  Codes and scales come from a counter-based generator -- splitmix64's output
  function applied to key + (i+1) * 0x9E3779B97F4A7C15 (Steele, Lea & Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014) -- written
  with torch int64 tensor operations so that CPU and GPU produce the same bytes;
* skewed routing: a per-expert logit bias b[e] = -1.2 * ln(1 + pi(e)) for a
  seeded permutation pi of the experts (Zipf exponent 1.2 over a random order).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

_GOLDEN = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK64 = (1 << 64) - 1


def _s64(u: int) -> int:
    """uint64 bit pattern -> the int64 with the same bits."""
    u &= _MASK64
    return u - (1 << 64) if u >= (1 << 63) else u


def mix64_int(z: int) -> int:
    """splitmix64 output function on a Python int (uint64 semantics)."""
    z &= _MASK64
    z = ((z ^ (z >> 30)) * _M1) & _MASK64
    z = ((z ^ (z >> 27)) * _M2) & _MASK64
    return z ^ (z >> 31)


def splitmix64_int(key: int, i: int) -> int:
    """i-th output (i >= 0) of a splitmix64 stream whose state starts at key."""
    return mix64_int((key + (i + 1) * _GOLDEN) & _MASK64)


def _lsr(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 tensors holding uint64 bit patterns."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def mix64(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _lsr(z, 30)) * _s64(_M1)
    z = (z ^ _lsr(z, 27)) * _s64(_M2)
    return z ^ _lsr(z, 31)


def splitmix64(keys: torch.Tensor, idx: torch.Tensor) -> torch.Tensor:
    """splitmix64 outputs for int64 keys (broadcast) and counters idx >= 0."""
    return mix64(keys + (idx + 1) * _s64(_GOLDEN))


def stream_key(*parts: int) -> int:
    """Fold integers into one 64-bit stream key."""
    k = 0x243F6A8885A308D3
    for p in parts:
        k = mix64_int(k ^ (p & _MASK64))
    return k


# ---------------------------------------------------------------------- dims & configs

@dataclass(frozen=True)
class Dims:
    hidden: int = 2048
    inter: int = 512
    n_experts: int = 256
    top_k: int = 8
    group_size: int = 64
    shared_inter: int = 512


MODEL_DIMS = Dims()


@dataclass(frozen=True)
class Config:
    name: str
    T: int
    seed: int
    layers: int = 1
    steps: int = 1
    zipf_bias: bool = False
    dims: Dims = field(default_factory=Dims)


# The five workloads: small prefill, the 512-token ablation length, 4K prefill,
# batch-1 decode over 40 stacked layers, and skewed routing at 16K tokens.
CONFIGS = {
    "t64": Config("t64", T=64, seed=101),
    "t512": Config("t512", T=512, seed=102),
    "t4096": Config("t4096", T=4096, seed=103),
    "decode": Config("decode", T=1, seed=104, layers=40, steps=256),
    "skew16k": Config("skew16k", T=16384, seed=105, zipf_bias=True),
}


# ---------------------------------------------------------------------- draws

def _cpu_gen(*parts: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(stream_key(*parts) & ((1 << 63) - 1))
    return g


def activations(T: int, H: int, seed: int, step: int = 0) -> torch.Tensor:
    """x ~ N(0, 1) rounded to bfloat16, [T][H], on the CPU."""
    x = torch.randn(T, H, generator=_cpu_gen(seed, 1, step), dtype=torch.float32)
    return x.to(torch.bfloat16)


def gqa_decode_inputs(B: int, Hq: int, Hkv: int, S: int, D: int, seed: int, layer: int = 0, q_std: float = 1.0):
    """One decode step of grouped-query attention on the CPU: q [B][Hq][D] ~ N(0, q_std^2)
    and k, v caches [B][Hkv][S][D] ~ N(0, 1), each rounded to bfloat16."""
    g = _cpu_gen(seed, 9, layer)
    q = (torch.randn(B, Hq, D, generator=g, dtype=torch.float32) * q_std).to(torch.bfloat16)
    k = torch.randn(B, Hkv, S, D, generator=g, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn(B, Hkv, S, D, generator=g, dtype=torch.float32).to(torch.bfloat16)
    return q, k, v


def router_weights(E: int, H: int, seed: int, layer: int = 0) -> torch.Tensor:
    """W_r ~ N(0, 1/H) fp32 [E][H], on the CPU."""
    return torch.randn(E, H, generator=_cpu_gen(seed, 2, layer), dtype=torch.float32) * (1.0 / math.sqrt(H))


def shared_gate_weights(H: int, seed: int, layer: int = 0) -> torch.Tensor:
    """w_sg ~ N(0, 1/H) fp32 [H], on the CPU."""
    return torch.randn(H, generator=_cpu_gen(seed, 3, layer), dtype=torch.float32) * (1.0 / math.sqrt(H))


def zipf_router_bias(E: int, seed: int, s: float = 1.2, layer: int = 0) -> torch.Tensor:
    """b[e] = -s * ln(1 + pi(e)) for a seeded permutation pi of 0..E-1 (fp32 [E])."""
    pi = torch.randperm(E, generator=_cpu_gen(seed, 4, layer))
    return (-s * torch.log1p(pi.to(torch.float64))).to(torch.float32)


_MATRIX_IDS = {"gate_up": 0, "down": 1, "sh_gate_up": 2, "sh_down": 3}


def q4_matrix(n_exp: int, N: int, K: int, G: int, seed: int, layer: int, matrix: str,
              device="cpu"):
    """Affine int4 weights of n_exp experts in the canonical layout.

    Returns (codes uint8 [n_exp][N][K/2], scales int16 [n_exp][N][K/G],
    biases int16 [n_exp][N][K/G]); scales and biases hold fp16 bit patterns.
    """
    assert K % G == 0 and (N * K // 2) % 8 == 0
    mid = _MATRIX_IDS[matrix]
    dev = torch.device(device)
    code_keys = torch.tensor([_s64(stream_key(seed, layer, mid, e, 0)) for e in range(n_exp)],
                             dtype=torch.int64, device=dev)
    scale_keys = torch.tensor([_s64(stream_key(seed, layer, mid, e, 1)) for e in range(n_exp)],
                              dtype=torch.int64, device=dev)
    words = N * K // 16  # 8 bytes (16 codes) per draw
    codes = torch.empty((n_exp, words), dtype=torch.int64, device=dev)
    chunk = max(1, (1 << 24) // max(words, 1))
    idx = torch.arange(words, dtype=torch.int64, device=dev)
    for e0 in range(0, n_exp, chunk):
        e1 = min(n_exp, e0 + chunk)
        codes[e0:e1] = splitmix64(code_keys[e0:e1, None], idx[None, :])
    codes = codes.view(torch.uint8).reshape(n_exp, N, K // 2)
    ng = N * (K // G)
    sidx = torch.arange(ng, dtype=torch.int64, device=dev)
    h = splitmix64(scale_keys[:, None], sidx[None, :])
    j = 1311 + torch.remainder(_lsr(h, 1), 3932)          # grid points of [0.005, 0.02) at 2^-18
    s32 = j.to(torch.float32) * (2.0 ** -18)               # exact in fp32
    s16 = s32.to(torch.float16)                             # nearest-even fp16
    b16 = s16 * -8.0                                        # exact in fp16
    scales = s16.view(torch.int16).reshape(n_exp, N, K // G)
    biases = b16.view(torch.int16).reshape(n_exp, N, K // G)
    return codes, scales, biases


@dataclass
class Layer:
    """One layer's weights as torch tensors (canonical layout)."""
    gate_up: tuple
    down: tuple
    sh_gate_up: tuple
    sh_down: tuple
    router_w: torch.Tensor
    shared_gate_w: torch.Tensor
    router_bias: torch.Tensor | None

    def to(self, device) -> "Layer":
        mv = lambda t: None if t is None else t.to(device)
        return Layer(*(tuple(mv(a) for a in m) for m in (self.gate_up, self.down, self.sh_gate_up, self.sh_down)),
                     mv(self.router_w), mv(self.shared_gate_w), mv(self.router_bias))


def make_layer(d: Dims, seed: int, layer: int = 0, zipf_bias: bool = False, device="cpu",
               dense_device="cpu") -> Layer:
    """All weights of one MoE layer.  int4 matrices are drawn on ``device``
    (identical bytes on CPU and GPU); the fp32 router weights on the CPU, then
    moved to ``dense_device``."""
    H, I, E, G, Is = d.hidden, d.inter, d.n_experts, d.group_size, d.shared_inter
    gu = q4_matrix(E, 2 * I, H, G, seed, layer, "gate_up", device)
    dn = q4_matrix(E, H, I, G, seed, layer, "down", device)
    sgu = q4_matrix(1, 2 * Is, H, G, seed, layer, "sh_gate_up", device)
    sdn = q4_matrix(1, H, Is, G, seed, layer, "sh_down", device)
    rw = router_weights(E, H, seed, layer).to(dense_device)
    sg = shared_gate_weights(H, seed, layer).to(dense_device)
    rb = zipf_router_bias(E, seed, layer=layer).to(dense_device) if zipf_bias else None
    return Layer(gu, dn, sgu, sdn, rw, sg, rb)


def layer_numpy(lay: Layer):
    """The same weights as numpy arrays (codes uint8, scales/biases uint16)."""
    def q(m):
        c, s, b = m
        return (c.cpu().numpy(), s.cpu().view(torch.int16).numpy().view("uint16"),
                b.cpu().view(torch.int16).numpy().view("uint16"))
    return {
        "gate_up": q(lay.gate_up), "down": q(lay.down), "sh_gate_up": q(lay.sh_gate_up),
        "sh_down": q(lay.sh_down), "router_w": lay.router_w.cpu().numpy(),
        "shared_gate_w": lay.shared_gate_w.cpu().numpy(),
        "router_bias": None if lay.router_bias is None else lay.router_bias.cpu().numpy(),
    }


def bf16_bits_numpy(t: torch.Tensor):
    """bfloat16 tensor -> numpy uint16 bit patterns."""
    return t.contiguous().cpu().view(torch.int16).numpy().view("uint16")
