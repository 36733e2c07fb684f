"""Sparse Mixture-of-Experts layer for MI355X (gfx950): Python binding of libmoe.

Thin ctypes marshalling over the C ABI declared in ``include/moe.h``: every
function here has the name of the C entry point it calls, takes torch tensors
for device memory and launches on ``torch.cuda.current_stream()``.  All work
runs in the HIP kernels of ``libmoe.so``; if the library is not built, every
call raises.
"""

from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch  # first: libmoe then binds to the HIP runtime torch already loaded

__all__ = [
    "Dims", "MoeError", "LayerWeights", "lib", "moe_block_m", "moe_max_tiles", "moe_prepack_router",
    "moe_router_logits", "moe_route", "moe_group_workspace_bytes", "moe_group", "moe_grouped_gemm_q4",
    "moe_workspace_bytes", "moe_workspace", "moe_forward", "moe_forward_stages", "moe_packed_q4_bytes",
    "moe_prepack_q4", "moe_host_block_map", "moe_host_routing_bytes", "moe_forward_host_routing",
    "moe_gqa_decode_workspace_bytes", "moe_gqa_decode_attention", "moe_workspace_errors", "moe_fused_residency",
    "moe_forward_noalloc", "NOALLOC_SCRATCH_BYTES",
    "MOE_EPI_SWIGLU_BF16", "MOE_EPI_WEIGHTED_SCATTER_F32", "MOE_DEVERR_HANDOVER_TIMEOUT", "MOE_DEVERR_EXPERT_ID",
    "STAGES", "EXPORTED_SYMBOLS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_EPI_SWIGLU_BF16, MOE_EPI_WEIGHTED_SCATTER_F32 = 0, 1
MOE_DEVERR_HANDOVER_TIMEOUT, MOE_DEVERR_EXPERT_ID = 1, 2
WORKSPACE_HEADER_BYTES = 256   # the device error word is the first int32
NOALLOC_SCRATCH_BYTES = 32 << 20   # MOE_NOALLOC_SCRATCH_BYTES
STAGES = ("router", "topk", "group", "gate_up", "down", "combine")  # MOE_STAGE_* in order
MOE_MAT_GATE_UP, MOE_MAT_DOWN, MOE_MAT_SH_GATE_UP, MOE_MAT_SH_DOWN = 0, 1, 2, 3

EXPORTED_SYMBOLS = (
    "moe_block_m", "moe_max_tiles", "moe_prepack_router", "moe_router_logits", "moe_route",
    "moe_group_workspace_bytes", "moe_group", "moe_grouped_gemm_q4", "moe_workspace_bytes", "moe_forward",
    "moe_forward_stages", "moe_status_str", "moe_last_error_message", "moe_last_hip_error",
    "moe_packed_q4_bytes", "moe_prepack_q4", "moe_host_block_map", "moe_host_routing_bytes",
    "moe_forward_host_routing", "moe_gqa_decode_workspace_bytes", "moe_gqa_decode_attention",
    "moe_workspace_errors", "moe_fused_residency", "moe_forward_noalloc",
)


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


@dataclass(frozen=True)
class Dims:
    hidden: int = 2048
    inter: int = 512
    n_experts: int = 256
    top_k: int = 8
    group_size: int = 64
    shared_inter: int = 512


class _Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("hidden", "inter", "n_experts", "top_k", "group_size", "shared_inter")]


class _Q4(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p),
                ("packed", ctypes.c_void_p)]


class _Layer(ctypes.Structure):
    _fields_ = [("gate_up", _Q4), ("down", _Q4), ("sh_gate_up", _Q4), ("sh_down", _Q4),
                ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("shared_gate_w", ctypes.c_void_p), ("router_w3", ctypes.c_void_p)]


_handle = None
_P, _I32, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t


def lib():
    """The loaded libmoe.so; raises if it has not been built."""
    global _handle
    if _handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        h = ctypes.CDLL(LIB_PATH)
        PD, PL = ctypes.POINTER(_Dims), ctypes.POINTER(_Layer)
        sig = {
            "moe_block_m": ([], _I32),
            "moe_max_tiles": ([_I32, _I32, _I32, _I32], _I32),
            "moe_prepack_router": ([PD, _P, _P, _P], _I32),
            "moe_router_logits": ([PD, PL, _P, _I32, _P, _P, _P], _I32),
            "moe_route": ([PD, _P, _P, _I32, _P, _P, _P, _P], _I32),
            "moe_group_workspace_bytes": ([PD, _I32], _SZ),
            "moe_group": ([PD, _P, _I32, _I32, _P, _P, _P, _P, _P, _I32, _P, _P, _SZ, _P], _I32),
            "moe_grouped_gemm_q4": ([PD, ctypes.POINTER(_Q4), _I32, _P, _I32, _P, _P, _P, _P, _I32, _P, _I32, _I32,
                                     _P, _P], _I32),
            "moe_workspace_bytes": ([PD, _I32], _SZ),
            "moe_forward": ([PD, PL, _P, _I32, _P, _P, _P, _P, _P, _SZ, _P], _I32),
            "moe_forward_stages": ([PD, PL, _P, _I32, _P, _P, _P, _P, _P, _SZ, _I32, _I32, _P], _I32),
            "moe_status_str": ([_I32], ctypes.c_char_p),
            "moe_last_error_message": ([], ctypes.c_char_p),
            "moe_last_hip_error": ([], _I32),
            "moe_packed_q4_bytes": ([PD, _I32, _I32], _SZ),
            "moe_prepack_q4": ([PD, _I32, ctypes.POINTER(_Q4), _I32, _P, _SZ, _P], _I32),
            "moe_host_block_map": ([_P, _I32, _I32, _I32, _P, _P, _P], _I32),
            "moe_host_routing_bytes": ([PD, _I32], _SZ),
            "moe_forward_host_routing": ([PD, PL, _P, _I32, _P, _P, _P, _P, _SZ, _P, _SZ, _P], _I32),
            "moe_gqa_decode_workspace_bytes": ([_I32] * 5, _SZ),
            "moe_gqa_decode_attention": ([_P, _P, _P, _P] + [_I32] * 5 + [ctypes.c_float, _I32, _P, _P, _SZ, _P],
                                         _I32),
            "moe_workspace_errors": ([_P, _SZ, _I32, ctypes.POINTER(_I32), _P], _I32),
            "moe_fused_residency": ([PD, _I32, ctypes.POINTER(_I32), ctypes.POINTER(_I32)], _I32),
            "moe_forward_noalloc": ([PD, PL, _P, _I32, _P, _P, _P, _P, _P], _I32),
        }
        for name, (args, res) in sig.items():
            fn = getattr(h, name)
            fn.argtypes = args
            fn.restype = res
        _handle = h
    return _handle


def _check(status: int):
    if status != MOE_OK:
        L = lib()
        raise MoeError(status, f"{L.moe_status_str(status).decode()}: {L.moe_last_error_message().decode()}")


def _dims(d) -> _Dims:
    return _Dims(d.hidden, d.inter, d.n_experts, d.top_k, d.group_size, d.shared_inter)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _q4(m) -> _Q4:
    """(codes, scales, biases[, packed]) -> moe_q4."""
    c, s, b = m[:3]
    return _Q4(_ptr(c), _ptr(s), _ptr(b), _ptr(m[3]) if len(m) > 3 else None)


class LayerWeights:
    """Device tensors of one layer and the C struct that points at them.

    gate_up/down/sh_gate_up/sh_down: (codes uint8, scales int16, biases int16)
    in the canonical layout of ``include/moe.h``, optionally followed by the
    packed matrix-core layout; with ``pack=True`` (default) missing packed
    copies are made here with moe_prepack_q4 (the T > 1 path needs them).
    """

    def __init__(self, d, gate_up, down, sh_gate_up, sh_down, router_w, shared_gate_w, router_bias=None,
                 router_w3=None, pack: bool = True):
        self.d = d
        if pack:
            gate_up, down, sh_gate_up, sh_down = (
                m if len(m) > 3 else (*m, moe_prepack_q4(d, kind, m))
                for kind, m in ((MOE_MAT_GATE_UP, gate_up), (MOE_MAT_DOWN, down),
                                (MOE_MAT_SH_GATE_UP, sh_gate_up), (MOE_MAT_SH_DOWN, sh_down)))
        self.gate_up, self.down, self.sh_gate_up, self.sh_down = gate_up, down, sh_gate_up, sh_down
        self.router_w, self.shared_gate_w, self.router_bias = router_w, shared_gate_w, router_bias
        self.router_w3 = router_w3 if router_w3 is not None else moe_prepack_router(d, router_w)
        self.c = _Layer(_q4(gate_up), _q4(down), _q4(sh_gate_up), _q4(sh_down), _ptr(router_w), _ptr(router_bias),
                        _ptr(shared_gate_w), _ptr(self.router_w3))


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


# ------------------------------------------------------------------ entry points

def moe_block_m() -> int:
    return int(lib().moe_block_m())


def moe_max_tiles(T: int, top_k: int, n_experts: int, block_m: int) -> int:
    return int(lib().moe_max_tiles(T, top_k, n_experts, block_m))


def moe_prepack_router(d, router_w: torch.Tensor, router_w3: torch.Tensor | None = None) -> torch.Tensor:
    if router_w3 is None:
        router_w3 = _empty((3, d.n_experts, d.hidden), torch.int16, router_w)
    _check(lib().moe_prepack_router(ctypes.byref(_dims(d)), _ptr(router_w), _ptr(router_w3), _stream()))
    return router_w3


def moe_packed_q4_bytes(d, matrix: int, n_exp: int) -> int:
    return int(lib().moe_packed_q4_bytes(ctypes.byref(_dims(d)), matrix, n_exp))


def moe_prepack_q4(d, matrix: int, w, packed: torch.Tensor | None = None) -> torch.Tensor:
    """Packed matrix-core layout of canonical weights w = (codes, scales, biases)."""
    codes = w[0]
    n_exp = codes.shape[0]
    nb = moe_packed_q4_bytes(d, matrix, n_exp)
    if packed is None:
        packed = _empty((max(1, nb),), torch.uint8, codes)
    q = _q4(w[:3])
    _check(lib().moe_prepack_q4(ctypes.byref(_dims(d)), matrix, ctypes.byref(q), n_exp, _ptr(packed),
                                packed.numel(), _stream()))
    return packed


def moe_router_logits(d, layer: LayerWeights, x: torch.Tensor, logits=None, shared_logit=None,
                      want_shared: bool = True):
    T = x.shape[0]
    if logits is None:
        logits = _empty((T, d.n_experts), torch.float32, x)
    if shared_logit is None and want_shared:
        shared_logit = _empty((T,), torch.float32, x)
    _check(lib().moe_router_logits(ctypes.byref(_dims(d)), ctypes.byref(layer.c), _ptr(x), T, _ptr(logits),
                                   _ptr(shared_logit), _stream()))
    return logits, shared_logit


def moe_route(d, logits: torch.Tensor, shared_logit=None, ids=None, weights=None, gate=None):
    T = logits.shape[0]
    if ids is None:
        ids = _empty((T, d.top_k), torch.int32, logits)
    if weights is None:
        weights = _empty((T, d.top_k), torch.float32, logits)
    if shared_logit is not None and gate is None:
        gate = _empty((T,), torch.float32, logits)
    _check(lib().moe_route(ctypes.byref(_dims(d)), _ptr(logits), _ptr(shared_logit), T, _ptr(ids), _ptr(weights),
                           _ptr(gate), _stream()))
    return ids, weights, gate


def moe_group_workspace_bytes(d, T: int) -> int:
    return int(lib().moe_group_workspace_bytes(ctypes.byref(_dims(d)), T))


def moe_group(d, ids: torch.Tensor, block_m: int, max_tiles: int | None = None, out: dict | None = None,
              workspace: torch.Tensor | None = None) -> dict:
    T = ids.shape[0]
    F = T * d.top_k
    mt = moe_max_tiles(T, d.top_k, d.n_experts, block_m) if max_tiles is None else max_tiles
    o = out if out is not None else {
        "counts": _empty((d.n_experts,), torch.int32, ids), "offsets": _empty((d.n_experts + 1,), torch.int32, ids),
        "perm": _empty((F,), torch.int32, ids), "inv_perm": _empty((F,), torch.int32, ids),
        "block_map": _empty((mt, 2), torch.int32, ids), "n_tiles": _empty((1,), torch.int32, ids)}
    if workspace is None:
        workspace = _empty((max(1, moe_group_workspace_bytes(d, T)),), torch.uint8, ids)
    _check(lib().moe_group(ctypes.byref(_dims(d)), _ptr(ids), T, block_m, _ptr(o["counts"]), _ptr(o["offsets"]),
                           _ptr(o["perm"]), _ptr(o["inv_perm"]), _ptr(o["block_map"]), mt, _ptr(o["n_tiles"]),
                           _ptr(workspace), workspace.numel(), _stream()))
    o["max_tiles"] = mt
    return o


def moe_grouped_gemm_q4(d, w, epi: int, a: torch.Tensor, perm, offsets, block_map, n_tiles, max_tiles: int,
                        row_weight, T: int, block_m: int, out: torch.Tensor, a_rows_are_tokens: bool | None = None):
    """a_rows_are_tokens: rows of ``a`` are tokens, gathered through perm (the
    default for SWIGLU), or already in grouped order (the default for SCATTER)."""
    if a_rows_are_tokens is None:
        a_rows_are_tokens = epi == MOE_EPI_SWIGLU_BF16
    q = _q4(w)
    _check(lib().moe_grouped_gemm_q4(ctypes.byref(_dims(d)), ctypes.byref(q), epi, _ptr(a),
                                     1 if a_rows_are_tokens else 0, _ptr(perm), _ptr(offsets), _ptr(block_map),
                                     _ptr(n_tiles), max_tiles, _ptr(row_weight), T, block_m, _ptr(out), _stream()))
    return out


def moe_workspace_bytes(d, T_max: int) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(_dims(d)), T_max))


def moe_workspace_errors(workspace: torch.Tensor, clear: bool = False) -> int:
    """The MOE_DEVERR_* bits of a workspace's device error word (synchronises
    the current stream); clear=True zeroes the word afterwards."""
    flags = ctypes.c_int32(0)
    _check(lib().moe_workspace_errors(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                      1 if clear else 0, ctypes.byref(flags), _stream()))
    return int(flags.value)


def moe_fused_residency(d, T: int):
    """(workgroups the fused layer for T tokens launches, workgroups of it the
    current device holds at once)."""
    n, r = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib().moe_fused_residency(ctypes.byref(_dims(d)), T, ctypes.byref(n), ctypes.byref(r)))
    return int(n.value), int(r.value)


def moe_workspace(d, T_max: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace for moe_forward with up to T_max tokens (the
    fused path for 1-4 tokens keeps counters in it that must start at zero)."""
    return torch.zeros((moe_workspace_bytes(d, T_max),), dtype=torch.uint8, device=device)


def moe_forward(d, layer: LayerWeights, x: torch.Tensor, y=None, logits_out=None, ids_out=None, w_out=None,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
    T = x.shape[0]
    if y is None:
        y = _empty((T, d.hidden), torch.bfloat16, x)
    if workspace is None:
        workspace = moe_workspace(d, T, x.device)
    _check(lib().moe_forward(ctypes.byref(_dims(d)), ctypes.byref(layer.c), _ptr(x), T, _ptr(y), _ptr(logits_out),
                             _ptr(ids_out), _ptr(w_out), _ptr(workspace), workspace.numel(), _stream()))
    return y


def moe_forward_noalloc(d, layer: LayerWeights, x: torch.Tensor, y: torch.Tensor, logits_out=None, ids_out=None,
                        w_out=None) -> torch.Tensor:
    """moe_forward on the library's own device scratch: no workspace, and
    nothing allocated by the call (y and the optional outputs are the
    caller's)."""
    T = x.shape[0]
    _check(lib().moe_forward_noalloc(ctypes.byref(_dims(d)), ctypes.byref(layer.c), _ptr(x), T, _ptr(y),
                                     _ptr(logits_out), _ptr(ids_out), _ptr(w_out), _stream()))
    return y


def moe_host_block_map(counts: torch.Tensor, block_m: int, max_tiles: int):
    """Host offsets, block map and tile count from per-expert counts (CPU
    int32 tensor of length E); returns (offsets [E+1], block_map [max_tiles][2], n_tiles)."""
    if counts.is_cuda or counts.dtype != torch.int32:
        raise ValueError("counts must be a CPU int32 tensor")
    counts = counts.contiguous()
    E = counts.numel()
    offsets = torch.empty(E + 1, dtype=torch.int32)
    block_map = torch.empty((max_tiles, 2), dtype=torch.int32)
    n_tiles = torch.empty(1, dtype=torch.int32)
    _check(lib().moe_host_block_map(counts.data_ptr(), E, block_m, max_tiles, offsets.data_ptr(), block_map.data_ptr(),
                                    n_tiles.data_ptr()))
    return offsets, block_map, int(n_tiles.item())


def moe_host_routing_bytes(d, T: int) -> int:
    return int(lib().moe_host_routing_bytes(ctypes.byref(_dims(d)), T))


def moe_forward_host_routing(d, layer: LayerWeights, x: torch.Tensor, y=None, ids_out=None, w_out=None,
                             workspace: torch.Tensor | None = None, host_buf: torch.Tensor | None = None):
    """moe_forward with the routing counts taken through the host (blocks the
    calling thread).  host_buf: a CPU uint8 tensor of moe_host_routing_bytes
    bytes, pinned for asynchronous copies."""
    T = x.shape[0]
    if y is None:
        y = _empty((T, d.hidden), torch.bfloat16, x)
    if workspace is None:
        workspace = moe_workspace(d, T, x.device)
    if host_buf is None:
        host_buf = torch.empty(moe_host_routing_bytes(d, T), dtype=torch.uint8, pin_memory=True)
    if host_buf.is_cuda:
        raise ValueError("host_buf must be host memory")
    _check(lib().moe_forward_host_routing(ctypes.byref(_dims(d)), ctypes.byref(layer.c), _ptr(x), T, _ptr(y),
                                          _ptr(ids_out), _ptr(w_out), _ptr(workspace), workspace.numel(),
                                          host_buf.data_ptr(), host_buf.numel(), _stream()))
    return y


def moe_forward_stages(d, layer: LayerWeights, x: torch.Tensor, y: torch.Tensor, workspace: torch.Tensor,
                       first: int, last: int, logits_out=None, ids_out=None, w_out=None) -> torch.Tensor:
    """Stages first..last (indices into STAGES) of moe_forward on a workspace
    filled by an earlier call with the same arguments."""
    T = x.shape[0]
    _check(lib().moe_forward_stages(ctypes.byref(_dims(d)), ctypes.byref(layer.c), _ptr(x), T, _ptr(y),
                                    _ptr(logits_out), _ptr(ids_out), _ptr(w_out), _ptr(workspace), workspace.numel(),
                                    first, last, _stream()))
    return y


# ------------------------------------------------------------------ grouped-query decode attention

def moe_gqa_decode_workspace_bytes(B: int, Hq: int, Hkv: int, D: int, S: int) -> int:
    return lib().moe_gqa_decode_workspace_bytes(B, Hq, Hkv, D, S)


def moe_gqa_decode_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, seq_lens: torch.Tensor,
                             scale: float | None = None, pack_heads: bool = True, out=None, workspace=None):
    """One decode step of grouped-query attention.  q [B][Hq][D] bf16, k_cache /
    v_cache [B][Hkv][S][D] bf16, seq_lens [B] int32 (device).  Returns out
    [B][Hq][D] bf16.  scale defaults to 1/sqrt(D)."""
    B, Hq, D = q.shape
    Bk, Hkv, S, Dk = k_cache.shape
    if (Bk, Dk) != (B, D) or v_cache.shape != k_cache.shape or tuple(seq_lens.shape) != (B,):
        raise ValueError("shapes: q [B][Hq][D], caches [B][Hkv][S][D], seq_lens [B]")
    for t, dt in ((q, torch.bfloat16), (k_cache, torch.bfloat16), (v_cache, torch.bfloat16), (seq_lens, torch.int32)):
        if t.dtype != dt or not t.is_contiguous():
            raise ValueError("q and caches must be contiguous bf16, seq_lens contiguous int32")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = _empty((B, Hq, D), torch.bfloat16, q)
    if workspace is None:
        need = moe_gqa_decode_workspace_bytes(B, Hq, Hkv, D, S)
        workspace = _empty((max(need, 1),), torch.uint8, q)
    _check(lib().moe_gqa_decode_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), B, Hq, Hkv, D, S,
                                          float(scale), 1 if pack_heads else 0, _ptr(out), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(), _stream()))
    return out
