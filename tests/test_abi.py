"""The C-ABI library: it loads, exports every symbol include/moe.h declares,
and rejects bad arguments on the host before any launch (CPU only: no
compute call is made)."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def m():
    import sparse_moe_softmax_amd
    return sparse_moe_softmax_amd


def test_every_declared_symbol_is_exported(m):
    names = _declared()
    assert len(names) >= 13
    lib = ctypes.CDLL(m.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(m.EXPORTED_SYMBOLS) == names


def test_small_helpers(m):
    bm = m.moe_block_m()
    assert bm % 16 == 0 and 16 <= bm <= 256
    assert m.moe_max_tiles(4096, 8, 256, 128) == 256 + 256
    assert m.moe_max_tiles(1, 8, 256, 128) == 1 + 256
    L = m.lib()
    for s, name in [(0, "MOE_OK"), (-1, "MOE_ERR_INVALID_ARG"), (-2, "MOE_ERR_UNSUPPORTED"),
                    (-3, "MOE_ERR_WORKSPACE"), (-4, "MOE_ERR_HIP")]:
        assert L.moe_status_str(s).decode() == name


def _d(m, **kw):
    return ctypes.byref(m._dims(m.Dims(**kw)))


FAKE = ctypes.c_void_p(4096)  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("kw,status", [
    ({"group_size": 32}, -2), ({"hidden": 96}, -2), ({"inter": 48}, -2), ({"inter": 96}, -2),
    ({"shared_inter": 160}, -2), ({"n_experts": 512}, -2),
    ({"n_experts": 24}, -2), ({"top_k": 17}, -2), ({"top_k": 0}, -1), ({"hidden": -64}, -1)])
def test_bad_dims_rejected(m, kw, status):
    L = m.lib()
    assert L.moe_route(_d(m, **kw), FAKE, None, 4, FAKE, FAKE, None, None) == status
    assert L.moe_forward(_d(m, **kw), None, FAKE, 4, FAKE, None, None, None, FAKE, 1 << 30, None) == status
    assert L.moe_workspace_bytes(_d(m, **kw), 4) == 0


def test_bad_arguments_rejected(m):
    L = m.lib()
    d = _d(m)
    assert L.moe_route(d, FAKE, None, 0, FAKE, FAKE, None, None) == -1          # T = 0
    assert L.moe_route(d, FAKE, None, 70000, FAKE, FAKE, None, None) == -1      # T too large
    assert L.moe_route(d, None, None, 4, FAKE, FAKE, None, None) == -1          # NULL logits
    assert L.moe_route(d, FAKE, FAKE, 4, FAKE, FAKE, None, None) == -1          # gate without output
    assert L.moe_forward(d, None, FAKE, 4, FAKE, None, None, None, FAKE, 1 << 30, None) == -1   # NULL layer
    # group: block map too small, bad block_m, workspace too small
    need = L.moe_group_workspace_bytes(d, 100)
    assert need > 0
    mt = L.moe_max_tiles(100, 8, 256, 64)
    args = lambda bm, mtiles, ws: (d, FAKE, 100, bm, FAKE, FAKE, FAKE, FAKE, FAKE, mtiles, FAKE, FAKE, ws, None)
    assert L.moe_group(*args(64, mt - 1, need)) == -1
    assert L.moe_group(*args(0, mt, need)) == -1
    assert L.moe_group(*args(64, mt, need - 1)) == -3
    # grouped gemm: block_m above the kernel tile, scatter without weights, unknown epilogue
    q = m._Q4(FAKE, FAKE, FAKE, FAKE)
    g = lambda epi, bm, rw, tok=1: L.moe_grouped_gemm_q4(d, ctypes.byref(q), epi, FAKE, tok, FAKE, FAKE, FAKE, FAKE,
                                                         10, rw, 100, bm, FAKE, None)
    assert g(0, m.moe_block_m() + 1, None) == -1
    assert g(1, 64, None) == -1
    assert g(7, 64, FAKE) == -1
    assert "epilogue" in L.moe_last_error_message().decode()
    assert g(0, 64, None, tok=2) == -1
    assert "a_rows_are_tokens" in L.moe_last_error_message().decode()
    assert L.moe_grouped_gemm_q4(d, ctypes.byref(m._Q4(FAKE, FAKE, FAKE, None)), 0, FAKE, 1, FAKE, FAKE, FAKE, FAKE,
                                 10, None, 100, 64, FAKE, None) == -1           # not prepacked
    assert "moe_prepack_q4" in L.moe_last_error_message().decode()


def test_workspace_header_and_error_query(m):
    """Both workspaces start with the 256-byte header that holds the device
    error word; the query refuses a missing or short workspace and a NULL
    output before touching the device."""
    L = m.lib()
    d = _d(m)
    assert m.WORKSPACE_HEADER_BYTES == 256
    ntile = -(-100 // 16)
    assert L.moe_group_workspace_bytes(d, 100) == 256 + 2 * (-(-ntile * 256 * 4 // 256) * 256)
    flags = ctypes.c_int32(7)
    assert L.moe_workspace_errors(None, 1 << 20, 0, ctypes.byref(flags), None) == -3
    assert L.moe_workspace_errors(FAKE, 255, 0, ctypes.byref(flags), None) == -3
    assert L.moe_workspace_errors(FAKE, 256, 0, None, None) == -1
    assert flags.value == 7
    assert (m.MOE_DEVERR_HANDOVER_TIMEOUT, m.MOE_DEVERR_EXPERT_ID) == (1, 2)


def test_fused_residency_checks(m):
    """The residency query: only the fused sizes, outputs required; without a
    device it reports a HIP error instead of guessing (the forward path then
    refuses to launch the fused layer)."""
    L = m.lib()
    n, r = ctypes.c_int32(-1), ctypes.c_int32(-1)
    assert L.moe_fused_residency(_d(m), 5, ctypes.byref(n), ctypes.byref(r)) == -2      # grouped path
    assert L.moe_fused_residency(_d(m, hidden=4096), 2, ctypes.byref(n), ctypes.byref(r)) == -2
    assert L.moe_fused_residency(_d(m), 1, None, ctypes.byref(r)) == -1
    assert L.moe_fused_residency(_d(m, group_size=32), 1, ctypes.byref(n), ctypes.byref(r)) == -2
    import torch
    if not torch.cuda.is_available():
        assert L.moe_fused_residency(_d(m), 1, ctypes.byref(n), ctypes.byref(r)) == -4
        assert (n.value, r.value) == (0, 0)


def test_forward_workspace_checked(m):
    L = m.lib()
    d = _d(m)
    need = L.moe_workspace_bytes(d, 4096)
    assert need > L.moe_workspace_bytes(d, 64) > 0
    q = m._Q4(FAKE, FAKE, FAKE, FAKE)
    layer = m._Layer(q, q, q, q, FAKE, None, FAKE, FAKE)
    assert L.moe_forward(d, ctypes.byref(layer), FAKE, 4096, FAKE, None, None, None, FAKE, need - 1, None) == -3
    assert L.moe_forward(d, ctypes.byref(layer), FAKE, 4096, FAKE, None, None, None, None, need, None) == -3
    nolayer = m._Layer(q, q, q, q, FAKE, None, None, FAKE)
    assert L.moe_forward(d, ctypes.byref(nolayer), FAKE, 4, FAKE, None, None, None, FAKE, need, None) == -1
    # the grouped path (T > 4) needs the bf16 router planes; the fused path (T <= 4) the fp32 router
    nor3 = m._Layer(q, q, q, q, FAKE, None, FAKE, None)
    assert L.moe_forward(d, ctypes.byref(nor3), FAKE, 64, FAKE, None, None, None, FAKE, need, None) == -1
    assert "router_w3" in L.moe_last_error_message().decode()
    norw = m._Layer(q, q, q, q, None, None, FAKE, FAKE)
    for T in (1, 4):
        assert L.moe_forward(d, ctypes.byref(norw), FAKE, T, FAKE, None, None, None, FAKE, need, None) == -1
        assert "router_w is NULL" in L.moe_last_error_message().decode()
    # the grouped GEMMs (T > 4) read the packed weights
    unpacked = m._Q4(FAKE, FAKE, FAKE, None)
    nopack = m._Layer(unpacked, q, q, q, FAKE, None, FAKE, FAKE)
    assert L.moe_forward(d, ctypes.byref(nopack), FAKE, 64, FAKE, None, None, None, FAKE, need, None) == -1
    assert "moe_prepack_q4" in L.moe_last_error_message().decode()
    # the fused path (1 <= T <= 4) reads only the canonical arrays
    nocanon = m._Layer(m._Q4(None, None, None, FAKE), q, q, q, FAKE, None, FAKE, FAKE)
    for T in (1, 4):
        assert L.moe_forward(d, ctypes.byref(nocanon), FAKE, T, FAKE, None, None, None, FAKE, need, None) == -1
        assert "NULL weight pointer" in L.moe_last_error_message().decode()


def test_packed_sizes_and_checks(m):
    L = m.lib()
    d = _d(m)
    # 256-column slices x 64-wide K blocks x 9216 B: the canonical byte count for these dims
    canon = lambda N, K: N * K // 2 + 2 * N * (K // 64) * 2
    assert L.moe_packed_q4_bytes(d, m.MOE_MAT_GATE_UP, 256) == 256 * canon(1024, 2048)
    assert L.moe_packed_q4_bytes(d, m.MOE_MAT_DOWN, 256) == 256 * canon(2048, 512)
    assert L.moe_packed_q4_bytes(d, m.MOE_MAT_SH_GATE_UP, 1) == canon(1024, 2048)
    assert L.moe_packed_q4_bytes(_d(m, shared_inter=192), m.MOE_MAT_SH_GATE_UP, 1) == 2 * 32 * 9216  # padded slice
    assert L.moe_packed_q4_bytes(d, 4, 1) == 0 and L.moe_packed_q4_bytes(d, 0, 0) == 0
    q = m._Q4(FAKE, FAKE, FAKE, None)
    need = L.moe_packed_q4_bytes(d, 0, 2)
    assert L.moe_prepack_q4(d, 0, ctypes.byref(q), 2, FAKE, need - 1, None) == -1
    assert L.moe_prepack_q4(d, 5, ctypes.byref(q), 2, FAKE, need, None) == -1
    assert L.moe_prepack_q4(d, 0, ctypes.byref(m._Q4(None, FAKE, FAKE, None)), 2, FAKE, need, None) == -1
    assert L.moe_prepack_q4(_d(m, inter=96), 0, ctypes.byref(q), 2, FAKE, need, None) == -2


def test_binding_refuses_host_tensors(m):
    import torch
    with pytest.raises(ValueError):
        m.moe_route(m.Dims(), torch.zeros(4, 256))


# ------------------------------------------------------------------ host-routed variant (host logic only)

def _ids_for(T, E, k, mode, seed):
    import numpy as np
    rng = np.random.default_rng(seed)
    if mode == "one_hot":
        return np.tile(np.arange(k, dtype=np.int32) + 3, (T, 1))
    p = None
    if mode == "zipf":
        p = 1.0 / np.arange(1, E + 1) ** 1.2
        p = p[rng.permutation(E)]
        p /= p.sum()
    return np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,E,k,bm,mode", [(512, 256, 8, 192, "uniform"), (300, 64, 6, 7, "zipf"),
                                           (40, 16, 4, 1, "one_hot"), (4096, 256, 8, 192, "zipf")])
def test_host_block_map_matches_oracle(m, T, E, k, bm, mode):
    """The host builder of the routing round-trip variant gives the oracle's
    offsets, block map and tile count."""
    import numpy as np
    import torch
    import oracle
    ids = _ids_for(T, E, k, mode, T + bm)
    counts = torch.from_numpy(np.bincount(ids.reshape(-1), minlength=E).astype(np.int32))
    mt = m.moe_max_tiles(T, k, E, bm)
    offsets, bmap, nt = m.moe_host_block_map(counts, bm, mt)
    ref = oracle.group(ids, E, bm, n_max_tiles=mt)
    assert np.array_equal(offsets.numpy(), ref.offsets)
    assert np.array_equal(bmap.numpy(), ref.block_map)
    assert nt == ref.n_tiles


def test_host_routing_checks(m):
    L = m.lib()
    E = 16
    vp = lambda a: ctypes.cast(a, ctypes.c_void_p)
    off = (ctypes.c_int32 * (E + 1))()
    bmap = (ctypes.c_int32 * 8)()
    nt = (ctypes.c_int32 * 1)()
    bad = (ctypes.c_int32 * E)(*([1] * (E - 1) + [-1]))
    assert L.moe_host_block_map(vp(bad), E, 4, 4, vp(off), vp(bmap), vp(nt)) == -1      # negative count
    many = (ctypes.c_int32 * E)(*([5] * E))
    assert L.moe_host_block_map(vp(many), E, 4, 4, vp(off), vp(bmap), vp(nt)) == -1     # max_tiles too small
    assert L.moe_host_block_map(None, E, 4, 4, vp(off), vp(bmap), vp(nt)) == -1
    d = _d(m)
    need = L.moe_host_routing_bytes(d, 512)
    assert need == 4 * (256 + 257 + 2 * m.moe_max_tiles(512, 8, 256, m.moe_block_m()) + 1)
    hb = (ctypes.c_uint8 * need)()
    q = m._Q4(FAKE, FAKE, FAKE, FAKE)
    layer = m._Layer(q, q, q, q, FAKE, None, FAKE, FAKE)
    # the fused sizes (1 <= T <= 4 here) are not covered; a short host buffer is refused before any launch
    for T in (1, 3, 4):
        assert L.moe_forward_host_routing(d, ctypes.byref(layer), FAKE, T, FAKE, None, None, FAKE, 1 << 30, vp(hb),
                                          need, None) == -2
    assert L.moe_forward_host_routing(d, ctypes.byref(layer), FAKE, 512, FAKE, None, None, FAKE, 1 << 30, vp(hb),
                                      need - 4, None) == -1


# ------------------------------------------------------------------ grouped-query decode attention (host checks)

def test_gqa_workspace_and_checks(m):
    L = m.lib()
    # 32768 positions, 2 key/value heads: 256 blocks of 128 positions (a
    # 16-position stage per wave of 8) per head -> 1 block per range, 256
    # workgroups, 128 ranges per head
    assert L.moe_gqa_decode_workspace_bytes(1, 16, 2, 256, 32768) == 16 * 128 * (256 + 2) * 4
    assert L.moe_gqa_decode_workspace_bytes(1, 16, 2, 96, 100) == 0          # head_dim
    assert L.moe_gqa_decode_workspace_bytes(1, 18, 2, 128, 100) == 0         # 9 query heads per group
    need = L.moe_gqa_decode_workspace_bytes(2, 16, 2, 128, 1000)
    assert need > 0
    call = lambda Hq, Hkv, D, ws, nbytes, pack=1, k=FAKE: L.moe_gqa_decode_attention(
        FAKE, k, FAKE, FAKE, 2, Hq, Hkv, D, 1000, 0.1, pack, FAKE, ws, nbytes, None)
    assert call(16, 2, 96, FAKE, need) == -2
    assert call(16, 3, 128, FAKE, need) == -1
    assert call(18, 2, 128, FAKE, need) == -2
    assert call(16, 2, 128, FAKE, need - 1) == -3
    assert call(16, 2, 128, None, need) == -3
    assert call(16, 2, 128, FAKE, need, pack=2) == -1
    assert call(16, 2, 128, FAKE, need, k=ctypes.c_void_p(4100)) == -1       # cache not 16-byte aligned
    assert L.moe_gqa_decode_attention(FAKE, FAKE, FAKE, None, 2, 16, 2, 128, 1000, 0.1, 1, FAKE, FAKE, need,
                                      None) == -1


def test_noalloc_limits(m):
    """The no-allocation entry point refuses, before touching the device, a
    T whose workspace exceeds its fixed scratch, and bad arguments."""
    L = m.lib()
    d = _d(m)
    q = m._Q4(FAKE, FAKE, FAKE, FAKE)
    layer = m._Layer(q, q, q, q, FAKE, None, FAKE, FAKE)
    assert m.NOALLOC_SCRATCH_BYTES == 32 << 20
    assert L.moe_workspace_bytes(d, 512) <= m.NOALLOC_SCRATCH_BYTES < L.moe_workspace_bytes(d, 1024)
    assert L.moe_forward_noalloc(d, ctypes.byref(layer), FAKE, 1024, FAKE, None, None, None, None) == -3
    assert "moe_forward_noalloc holds" in L.moe_last_error_message().decode()
    assert L.moe_forward_noalloc(d, ctypes.byref(layer), FAKE, 0, FAKE, None, None, None, None) == -1
    assert L.moe_forward_noalloc(_d(m, group_size=32), ctypes.byref(layer), FAKE, 4, FAKE, None, None, None,
                                 None) == -2
