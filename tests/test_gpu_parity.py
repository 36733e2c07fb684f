"""GPU parity of every step of the MoE layer against the CPU oracle.

Each test calls the HIP library through its C ABI (via the ctypes binding) on
seeded synthetic inputs and compares with the oracle element by element:
bit-exact for routing ids, counts, offsets, permutations, block maps and tile
counts; within the stated tolerances for floating point.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

TINY = synth.Dims(hidden=128, inter=64, n_experts=16, top_k=4, group_size=64, shared_inter=64)
MODEL = synth.MODEL_DIMS


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ generator / prepack

def test_generator_cpu_gpu_identical():
    say("generator cpu vs gpu")
    for m, (N, K) in {"gate_up": (1024, 2048), "down": (2048, 512)}.items():
        c1, s1, b1 = synth.q4_matrix(3, N, K, 64, seed=7, layer=5, matrix=m, device="cpu")
        c2, s2, b2 = synth.q4_matrix(3, N, K, 64, seed=7, layer=5, matrix=m, device="cuda")
        assert torch.equal(c1, c2.cpu()) and torch.equal(s1, s2.cpu()) and torch.equal(b1, b2.cpu())


def test_prepack_router_is_exact_split():
    say("prepack router")
    m = gu.moe()
    W = synth.router_weights(256, 2048, seed=3)
    W[0, :4] = torch.tensor([0.0, -0.0, 1e-20, -3.5e-25])
    w3 = m.moe_prepack_router(gu.to_dims(MODEL), W.cuda())
    torch.cuda.synchronize()
    planes = w3.cpu().view(torch.bfloat16).to(torch.float64)
    assert torch.equal(planes.sum(0), W.to(torch.float64))


def _pack_reference(codes, scales, biases, swiglu, Iw, N, K):
    """The packed layout written out with numpy loops over blocks: per expert,
    slice of 256 columns and K block of 64, 256 rows x 32 code bytes (the two
    16-byte halves of row i swapped when bit 0 of (i >> 2) ^ (i >> 3) is set),
    then 256 (scale, bias) fp16 pairs; gate/up slices hold, per 64 rows, 32 gate
    rows and the 32 up rows of the same intermediate columns; missing rows zero."""
    n_exp = codes.shape[0]
    kg = K // 64
    slices = -(-Iw // 128) if swiglu else -(-N // 256)
    out = np.zeros((n_exp, slices, kg, 9216), dtype=np.uint8)
    i = np.arange(256)
    if swiglu:
        hcol = (i >> 6) * 32 + (i & 31)
        up = (i & 63) >= 32
    for sl in range(slices):
        if swiglu:
            hc = sl * 128 + hcol
            rows = np.where(hc < Iw, np.where(up, Iw + hc, hc), -1)
        else:
            rows = sl * 256 + i
            rows = np.where(rows < N, rows, -1)
        ok = rows >= 0
        swap = (((i >> 2) ^ (i >> 3)) & 1).astype(bool)
        for kb in range(kg):
            blk = np.zeros((n_exp, 256, 32), dtype=np.uint8)
            blk[:, ok] = codes[:, rows[ok], kb * 32:(kb + 1) * 32]
            blk[:, swap] = np.concatenate([blk[:, swap, 16:], blk[:, swap, :16]], axis=2)
            sb = np.zeros((n_exp, 256, 2), dtype=np.uint16)
            sb[:, ok, 0] = scales[:, rows[ok], kb]
            sb[:, ok, 1] = biases[:, rows[ok], kb]
            out[:, sl, kb, :8192] = blk.reshape(n_exp, -1)
            out[:, sl, kb, 8192:] = sb.reshape(n_exp, -1).view(np.uint8)
    return out.reshape(n_exp, -1)


@pytest.mark.parametrize("kind", [0, 1, 2, 3])
def test_prepack_q4_layout(kind):
    say("prepack q4 kind", kind)
    m = gu.moe()
    d = synth.Dims(hidden=512, inter=192, n_experts=16, top_k=4, group_size=64, shared_inter=320)
    Iw = d.shared_inter if kind >= 2 else d.inter
    swiglu = kind in (0, 2)
    N, K = (2 * Iw, d.hidden) if swiglu else (d.hidden, Iw)
    n_exp = 3 if kind < 2 else 1
    w = synth.q4_matrix(n_exp, N, K, 64, seed=11, layer=kind, matrix="gate_up" if swiglu else "down", device="cuda")
    packed = m.moe_prepack_q4(gu.to_dims(d), kind, w)
    torch.cuda.synchronize()
    c, sc, bi = (a.cpu().numpy() for a in w)
    ref = _pack_reference(c, sc.view(np.uint16), bi.view(np.uint16), swiglu, Iw, N, K)
    got = packed.cpu().numpy().reshape(n_exp, -1)
    assert got.shape == ref.shape
    assert np.array_equal(got, ref)


# ------------------------------------------------------------------ router logits

@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 300])
def test_router_logits(T):
    say("router logits T", T)
    m = gu.moe()
    lay = synth.make_layer(MODEL, 31, zipf_bias=(T == 65))
    dl = gu.device_layer(lay, MODEL)
    x = synth.activations(T, MODEL.hidden, 31)
    logits, s = m.moe_router_logits(gu.to_dims(MODEL), dl, x.cuda())
    torch.cuda.synchronize()
    ow = gu.oracle_layer(lay)
    ol, os_ = oracle.router(synth.bf16_bits_numpy(x), ow.router_w, ow.router_bias, ow.shared_gate_w)
    assert np.abs(logits.cpu().numpy() - ol).max() <= gu.LOGIT_ATOL
    assert np.abs(s.cpu().numpy() - os_).max() <= gu.LOGIT_ATOL


# ------------------------------------------------------------------ top-k

def _tie_logits(T, E, k, seed):
    rng = np.random.default_rng(seed)
    l = rng.standard_normal((T, E)).astype(np.float32)
    for t in range(0, T, 2):
        o = np.argsort(-l[t], kind="stable")
        l[t, o[k]] = l[t, o[k - 1]]          # tie across the cut
        l[t, o[2]] = l[t, o[1]]              # tie among the kept
    if T > 3:
        l[1, :] = 0.0
        l[1, ::3] = -0.0                     # +0 / -0 ties
        l[3, :] = np.float32(2.5)            # all equal
    return l


@pytest.mark.parametrize("T,E,k", [(1, 256, 8), (100, 256, 8), (513, 256, 8), (40, 16, 4), (33, 64, 16)])
def test_route_bit_exact(T, E, k):
    say("route T E k", T, E, k)
    m = gu.moe()
    d = synth.Dims(hidden=2048, inter=512, n_experts=E, top_k=k, group_size=64, shared_inter=512)
    l = _tie_logits(T, E, k, T + E)
    s = np.random.default_rng(1).standard_normal(T).astype(np.float32) * 3
    ids, w, g = m.moe_route(gu.to_dims(d), torch.from_numpy(l).cuda(), torch.from_numpy(s).cuda())
    torch.cuda.synchronize()
    oids, ow = oracle.topk(l, k)
    assert np.array_equal(ids.cpu().numpy(), oids)
    assert np.abs(w.cpu().numpy() - ow).max() <= gu.WEIGHT_ATOL
    assert np.abs(g.cpu().numpy() - oracle.sigmoid(s)).max() <= gu.WEIGHT_ATOL


# ------------------------------------------------------------------ grouping

def _ids(T, E, k, mode, seed):
    rng = np.random.default_rng(seed)
    if mode == "one_hot":
        ids = np.tile(np.arange(k, dtype=np.int32)[::-1] + 5, (T, 1))
        return ids
    p = None
    if mode == "zipf":
        p = 1.0 / np.arange(1, E + 1) ** 1.2
        p = p[rng.permutation(E)]
        p /= p.sum()
    return np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,E,k,bm,mode", [
    (1, 256, 8, 128, "uniform"), (64, 256, 8, 128, "uniform"), (65, 256, 8, 16, "uniform"),
    (512, 256, 8, 128, "uniform"), (4096, 256, 8, 128, "uniform"), (16384, 256, 8, 128, "zipf"),
    (200, 16, 4, 7, "one_hot"), (1000, 256, 8, 1, "zipf"), (129, 64, 16, 64, "uniform"),
    (1024, 256, 8, 128, "zipf"), (1040, 256, 8, 128, "zipf"),   # the last one-launch size and the next
    (2000, 256, 8, 4096, "zipf"), (300, 32, 8, 4096, "uniform")])   # the largest tile height moe_group takes
def test_group_bit_exact(T, E, k, bm, mode):
    say("group T E k bm mode", T, E, k, bm, mode)
    m = gu.moe()
    d = synth.Dims(hidden=2048, inter=512, n_experts=E, top_k=k, group_size=64, shared_inter=512)
    ids = _ids(T, E, k, mode, T * 3 + bm)
    out = m.moe_group(gu.to_dims(d), torch.from_numpy(ids).cuda(), bm)
    torch.cuda.synchronize()
    ref = oracle.group(ids, E, bm, n_max_tiles=out["max_tiles"])
    assert np.array_equal(out["counts"].cpu().numpy(), ref.counts)
    assert np.array_equal(out["offsets"].cpu().numpy(), ref.offsets)
    assert np.array_equal(out["perm"].cpu().numpy(), ref.perm)
    assert np.array_equal(out["inv_perm"].cpu().numpy(), ref.inv_perm)
    assert np.array_equal(out["block_map"].cpu().numpy(), ref.block_map)
    assert int(out["n_tiles"].item()) == ref.n_tiles


def test_group_is_deterministic():
    say("group determinism")
    m = gu.moe()
    ids = torch.from_numpy(_ids(4096, 256, 8, "zipf", 5)).cuda()
    a = m.moe_group(gu.to_dims(MODEL), ids, 128)
    b = m.moe_group(gu.to_dims(MODEL), ids, 128)
    torch.cuda.synchronize()
    for key in ("counts", "offsets", "perm", "inv_perm", "block_map", "n_tiles"):
        assert torch.equal(a[key], b[key])


# ------------------------------------------------------------------ grouped GEMMs

def _grouped_case(d, T, seed, mode="uniform", block_m=128):
    lay = synth.make_layer(d, seed)
    x = synth.activations(T, d.hidden, seed)
    ids = _ids(T, d.n_experts, d.top_k, mode, seed)
    gr = oracle.group(ids, d.n_experts, block_m)
    return lay, x, ids, gr


def _h_compare(h_gpu_bits, h_ref_bits):
    g = oracle.bf16_to_double(h_gpu_bits)
    r = oracle.bf16_to_double(h_ref_bits)
    diff = g != r
    # fp32 accumulation vs double: the bf16 rounding of h may differ by one ulp on a few elements
    assert diff.mean() < 0.01, f"{diff.mean():.4f} of h differ"
    # where a dot product nearly cancels, fp32 accumulation differs from double by a
    # small absolute amount that can exceed one ulp of the (tiny) result
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(r), 1e-30))) - 7)
    allowed = np.maximum(ulp * 1.01, 1e-5 * np.abs(r).max())
    assert np.all(np.abs(g - r) <= allowed)


@pytest.mark.parametrize("dname,T,mode,bm,tokens", [("tiny", 24, "uniform", 128, True),
                                                    ("tiny", 300, "one_hot", 128, True),
                                                    ("model", 64, "uniform", 128, True),
                                                    ("model", 700, "zipf", 128, True),
                                                    ("model", 200, "uniform", 37, True),
                                                    ("model", 200, "uniform", 37, False),
                                                    ("tiny", 300, "zipf", 128, False)])
def test_grouped_gemm_swiglu(dname, T, mode, bm, tokens):
    """a_rows_are_tokens = 1: token rows of x gathered through perm; 0: the
    same rows handed over already in grouped order (a[p] = x[perm[p] / k])."""
    say("grouped gemm swiglu", dname, T, mode, bm, tokens)
    m = gu.moe()
    d = TINY if dname == "tiny" else MODEL
    lay, x, ids, gr = _grouped_case(d, T, 41 + T, mode, bm)
    dl = gu.device_layer(lay, d)
    perm = torch.from_numpy(gr.perm).cuda()
    a = x if tokens else x[torch.from_numpy(gr.perm // d.top_k).long()].contiguous()
    h = torch.empty((T * d.top_k, d.inter), dtype=torch.int16, device="cuda")
    m.moe_grouped_gemm_q4(gu.to_dims(d), dl.gate_up, m.MOE_EPI_SWIGLU_BF16, a.cuda(), perm,
                          torch.from_numpy(gr.offsets).cuda(), torch.from_numpy(gr.block_map).cuda(),
                          torch.tensor([gr.n_tiles], dtype=torch.int32, device="cuda"), gr.block_map.shape[0], None,
                          T, bm, h, a_rows_are_tokens=tokens)
    torch.cuda.synchronize()
    ow = gu.oracle_layer(lay)
    href = oracle.grouped_swiglu(synth.bf16_bits_numpy(x), True, d.top_k, gr.perm, gr.offsets, ow.gate_up, d.hidden,
                                 d.inter, d.group_size)
    _h_compare(gu.bits(h), href)


@pytest.mark.parametrize("dname,T,mode,bm,tokens", [("tiny", 24, "uniform", 128, False),
                                                    ("model", 64, "uniform", 128, False),
                                                    ("model", 700, "zipf", 128, False),
                                                    ("model", 130, "uniform", 5, False),
                                                    ("model", 130, "uniform", 5, True),
                                                    ("tiny", 300, "zipf", 128, True)])
def test_grouped_gemm_scatter(dname, T, mode, bm, tokens):
    """a_rows_are_tokens = 0: rows of h in grouped order (the layer's case);
    1: rows of a [T][I] gathered per token, a[perm[p] / k]."""
    say("grouped gemm scatter", dname, T, mode, bm, tokens)
    m = gu.moe()
    d = TINY if dname == "tiny" else MODEL
    lay, x, ids, gr = _grouped_case(d, T, 51 + T, mode, bm)
    dl = gu.device_layer(lay, d)
    ow = gu.oracle_layer(lay)
    if tokens:
        # token-major bf16 rows (any values); the oracle reads them in grouped order
        a_tok = synth.activations(T, d.inter, 51 + T)
        a_bits = synth.bf16_bits_numpy(a_tok)
        href = np.ascontiguousarray(a_bits[gr.perm // d.top_k])
        a_dev = a_tok.cuda()
    else:
        # the oracle's own h as the input of both sides
        href = oracle.grouped_swiglu(synth.bf16_bits_numpy(x), True, d.top_k, gr.perm, gr.offsets, ow.gate_up,
                                     d.hidden, d.inter, d.group_size)
        a_dev = torch.from_numpy(href.view(np.int16)).cuda()
    rw = np.random.default_rng(T).uniform(0.01, 1.0, T * d.top_k).astype(np.float32)
    y = torch.zeros((T, d.hidden), dtype=torch.float32, device="cuda")
    m.moe_grouped_gemm_q4(gu.to_dims(d), dl.down, m.MOE_EPI_WEIGHTED_SCATTER_F32, a_dev,
                          torch.from_numpy(gr.perm).cuda(), torch.from_numpy(gr.offsets).cuda(),
                          torch.from_numpy(gr.block_map).cuda(),
                          torch.tensor([gr.n_tiles], dtype=torch.int32, device="cuda"), gr.block_map.shape[0],
                          torch.from_numpy(rw).cuda(), T, bm, y, a_rows_are_tokens=tokens)
    torch.cuda.synchronize()
    o = oracle.grouped_down(href, gr.offsets, ow.down, d.hidden, d.inter, d.group_size)
    yref = np.zeros((T, d.hidden))
    inv = gr.inv_perm.reshape(T, d.top_k)
    for j in range(d.top_k):
        yref += rw.reshape(T, d.top_k)[:, j:j + 1].astype(np.float64) * o[inv[:, j]]
    yg = y.cpu().numpy().astype(np.float64)
    assert np.abs(yg - yref).max() <= 1e-5 * np.abs(yref).max()


# ------------------------------------------------------------------ the whole layer

@pytest.mark.parametrize("dname,T", [("tiny", 1), ("tiny", 2), ("tiny", 37), ("tiny", 129), ("model", 1),
                                     ("model", 2), ("model", 3), ("model", 4), ("model", 8), ("model", 16),
                                     ("model", 64), ("model", 127), ("model", 512)])
def test_forward_parity_full(dname, T):
    say("forward", dname, T)
    d = TINY if dname == "tiny" else MODEL
    lay = synth.make_layer(d, 61 + T)
    x = synth.activations(T, d.hidden, 61 + T)
    r = gu.forward_and_check(d, lay, x)
    say("errors", r["errs"])


# hidden 512 / inter 256 / shared 384: the fewest K blocks the one-workgroup-per-CU
# GEMM takes (4), a shared expert wider than the routed ones (routed gate/up
# slices past the routed width are skipped) and more than one tile per
# workgroup; hidden 320 takes the one-tile-per-workgroup GEMM (odd K blocks).
# 16 experts at T = 16384 and 128 experts at T = 8192: expert counts below and
# between the router's 64-expert tiles, 65536 routed slots each.  k = 16 and
# k = 1 over 256 experts: the general top-k and the combine with k known only
# at run time
@pytest.mark.parametrize("hidden,inter,shared,E,k,T", [(512, 256, 384, 64, 6, 300), (512, 256, 384, 64, 6, 2000),
                                                         (320, 256, 128, 32, 4, 500), (256, 128, 128, 16, 4, 16384),
                                                         (512, 128, 128, 128, 8, 8192), (512, 256, 256, 256, 16, 200),
                                                         (512, 256, 256, 256, 1, 300)])
def test_forward_parity_gemm_forms(hidden, inter, shared, E, k, T):
    d = synth.Dims(hidden=hidden, inter=inter, n_experts=E, top_k=k, group_size=64, shared_inter=shared)
    say("forward gemm forms", d, T)
    lay = synth.make_layer(d, 5 + T)
    x = synth.activations(T, d.hidden, 5 + T)
    r = gu.forward_and_check(d, lay, x)
    say("errors", r["errs"])


@pytest.mark.parametrize("cfg", ["t4096", "skew16k"])
def test_forward_parity_full_size(cfg):
    """The 4096-token layer and the skewed 16384-token layer, every output
    element against the oracle (the oracle runs on all host threads)."""
    c = synth.CONFIGS[cfg]
    say("forward full size", cfg, c.T)
    lay = synth.make_layer(c.dims, c.seed, zipf_bias=c.zipf_bias)
    x = synth.activations(c.T, c.dims.hidden, c.seed)
    r = gu.forward_and_check(c.dims, lay, x)
    if c.zipf_bias:
        counts = np.bincount(r["ids"].reshape(-1), minlength=256)
        assert counts.max() > 10 * counts.mean() and (counts == 0).any()
    say("errors", r["errs"])


@pytest.mark.parametrize("T,scale", [(1, 64.0), (3, 64.0), (8, 64.0), (512, 64.0), (300, 512.0),
                                     (3, 2.0 ** -12), (300, 2.0 ** -12)])
def test_forward_parity_activation_scale(T, scale):
    """Activations scaled by powers of two (exact in bf16).  By 64 and 512 the
    expert outputs go far past fp16's 65504; by 2^-12 they fall to ~2^-24,
    fp16's subnormal range.  The down GEMM's fp16 slot values cover both only
    through their per-chunk exponents.  Logits scale with x, so their check
    against the oracle scales with it (routing is still bit-exact: the
    protocol shares the GPU logits)."""
    d = MODEL
    say("forward activation scale T", T, "scale", scale)
    lay = synth.make_layer(d, 401 + T)
    x = (synth.activations(T, d.hidden, 401 + T).float() * scale).to(torch.bfloat16)
    r = gu.forward_and_check(d, lay, x, logit_atol=gu.LOGIT_ATOL * scale)
    ref = oracle.bf16_to_double(r["ref_bits"])
    if T >= 8 and scale > 1:
        assert np.abs(ref).max() > 2 * 65504.0   # some slot output exceeds fp16's range
    if scale < 1:
        assert np.abs(ref).max() < 2.0 ** -14    # every output is below fp16's normal range
    say("errors", r["errs"], "max |y|", float(np.abs(ref).max()))


def test_forward_parity_max_tokens():
    """The largest batch the API accepts (65536 tokens, the model's dims):
    logits and routing of every token against the oracle (ids bit for bit),
    the layer output on 48 sampled tokens including the first and the last."""
    d, T, seed = MODEL, 65536, 107
    say("forward max tokens", T)
    lay = synth.make_layer(d, seed)
    x = synth.activations(T, d.hidden, seed)
    rng = np.random.default_rng(seed)
    tokens = np.sort(rng.choice(T, 48, replace=False)).astype(np.int32)
    tokens[0], tokens[-1] = 0, T - 1
    r = gu.forward_and_check(d, lay, x, tokens=tokens)
    say("errors", r["errs"])


@pytest.mark.parametrize("cfg", ["t64", "t512"])
def test_forward_parity_configs(cfg):
    c = synth.CONFIGS[cfg]
    say("forward config", cfg)
    lay = synth.make_layer(c.dims, c.seed)
    x = synth.activations(c.T, c.dims.hidden, c.seed)
    r = gu.forward_and_check(c.dims, lay, x)
    say("errors", r["errs"])


def test_decode_layers():
    c = synth.CONFIGS["decode"]
    for layer in (0, 1, 39):
        say("decode layer", layer)
        lay = synth.make_layer(c.dims, c.seed, layer=layer)
        for step in (0, 255):
            x = synth.activations(1, c.dims.hidden, c.seed, step=step)
            gu.forward_and_check(c.dims, lay, x)


# every register form of the fused T == 1 layer: hidden past 2048, inter past
# 512, k past 8, and a ragged one (hidden 192: most lanes hold no K; 48
# experts: the last top-k wave holds 16 real experts and 16 absent ones)
@pytest.mark.parametrize("hidden,inter,shared,E,k", [(4096, 1024, 1024, 32, 12), (2048, 1024, 512, 64, 4),
                                                     (4096, 256, 512, 16, 8), (1024, 512, 512, 256, 16),
                                                     (192, 128, 64, 48, 5)])
def test_decode_forms(hidden, inter, shared, E, k):
    d = synth.Dims(hidden=hidden, inter=inter, n_experts=E, top_k=k, group_size=64, shared_inter=shared)
    say("decode form", d)
    lay = synth.make_layer(d, 7 + hidden + E)
    for step in (0, 1):
        x = synth.activations(1, d.hidden, 7 + hidden + E, step=step)
        r = gu.forward_and_check(d, lay, x)
        say("errors", r["errs"])


def test_decode_handover_words():
    """The fused layer passes logits and h between its workgroups in tagged
    words at the start of the workspace: after n calls (one-token and
    three-token calls alternating) every block has recorded n completed calls,
    no wait timed out, and repeated calls on one workspace give identical
    outputs."""
    say("decode hand-over words")
    m = gu.moe()
    c = synth.CONFIGS["decode"]
    md = gu.to_dims(c.dims)
    dl = gu.device_layer(synth.make_layer(c.dims, c.seed, layer=3), c.dims)
    outs = []
    ws = m.moe_workspace(md, 4)
    for step in range(6):
        # one token and three tokens (the multi-token form) alternate on one workspace
        T = 1 if step % 2 == 0 else 3
        x = synth.activations(T, c.dims.hidden, c.seed, step=step % 4).cuda()
        outs.append(m.moe_forward(md, dl, x, workspace=ws).clone())
        torch.cuda.synchronize()
        words = ws[:256 + 1024].view(torch.int32).cpu()
        assert torch.all(words[64:64 + 256] == step + 1)   # calls completed, per block, after the header
        assert int(words[0]) == 0                          # error word: no hand-over timed out
        assert m.moe_workspace_errors(ws) == 0
    assert torch.equal(outs[0], outs[4]) and torch.equal(outs[1], outs[5])


@pytest.mark.parametrize("T", [1, 3, 5, 300])
def test_forward_router_ties(T):
    """Duplicated router rows give bitwise-equal logits: for token 0 the top
    expert's row is copied to a lower and a higher expert index (a three-way tie
    for first place, which pushes the old 6th expert to 8th place) and that
    expert's row to two others (a three-way tie across the cut).  The GPU ids must be the oracle's top-k of the GPU logits: lower expert
    index first among equal logits, on the fused (T = 1, 3) and grouped (T = 5,
    300) paths."""
    say("forward router ties T", T)
    d = MODEL
    lay = synth.make_layer(d, 501 + T)
    x = synth.activations(T, d.hidden, 501 + T)
    ow = gu.oracle_layer(lay)
    ol, _ = oracle.router(synth.bf16_bits_numpy(x)[:1], ow.router_w, ow.router_bias, ow.shared_gate_w)
    order = [int(e) for e in np.argsort(-ol[0], kind="stable")]
    top, eighth = order[0], order[5]
    spare = [e for e in range(d.n_experts) if e not in order[:10]]
    lo_t = min(spare)
    hi_t = max(spare)
    mid = [e for e in spare if e not in (lo_t, hi_t)]
    a8, b8 = mid[0], mid[-1]
    W = lay.router_w.clone()
    W[lo_t] = W[top]
    W[hi_t] = W[top]
    W[a8] = W[eighth]
    W[b8] = W[eighth]
    lay = synth.Layer(lay.gate_up, lay.down, lay.sh_gate_up, lay.sh_down, W, lay.shared_gate_w, lay.router_bias)
    r = gu.forward_and_check(d, lay, x)
    gl = r["logits"][0]
    assert gl[lo_t] == gl[top] == gl[hi_t] and gl[a8] == gl[eighth] == gl[b8]
    first = sorted([lo_t, top, hi_t])
    assert list(r["ids"][0][:3]) == first
    say("ids of token 0", list(r["ids"][0]), "ties", first, sorted([a8, eighth, b8]))


@pytest.mark.parametrize("T,cfg", [(5, None), (512, "t512"), (700, None), (4096, "skew16k")])
def test_forward_host_routing_parity(T, cfg):
    """The variant that takes the expert counts through the host against the
    oracle (same protocol as moe_forward)."""
    say("forward host routing vs oracle T", T, cfg)
    c = synth.CONFIGS[cfg] if cfg else None
    lay = synth.make_layer(MODEL, 191 + T, zipf_bias=bool(c and c.zipf_bias))
    x = synth.activations(T, MODEL.hidden, 191 + T)
    r = gu.forward_and_check(MODEL, lay, x, host_routing=True)
    say("errors", r["errs"])


@pytest.mark.parametrize("T,cfg", [(5, None), (512, "t512"), (700, None), (4096, "skew16k")])
def test_forward_host_routing_equals_forward(T, cfg):
    """The variant that takes the expert counts through the host builds the same
    offsets and block map there (pinned against the oracle on the CPU), so every
    output is bitwise that of moe_forward."""
    say("forward host routing T", T, cfg)
    m = gu.moe()
    d = MODEL
    c = synth.CONFIGS[cfg] if cfg else None
    lay = synth.make_layer(d, 91 + T, zipf_bias=bool(c and c.zipf_bias))
    dl = gu.device_layer(lay, d)
    md = gu.to_dims(d)
    x = synth.activations(T, d.hidden, 91 + T).cuda()
    ws_a, ws_b = m.moe_workspace(md, T), m.moe_workspace(md, T)
    ids_a = torch.empty((T, d.top_k), dtype=torch.int32, device="cuda")
    ids_b = torch.empty_like(ids_a)
    w_a = torch.empty((T, d.top_k), dtype=torch.float32, device="cuda")
    w_b = torch.empty_like(w_a)
    y_a = m.moe_forward(md, dl, x, ids_out=ids_a, w_out=w_a, workspace=ws_a)
    y_b = m.moe_forward_host_routing(md, dl, x, ids_out=ids_b, w_out=w_b, workspace=ws_b)
    torch.cuda.synchronize()
    assert torch.equal(ids_a, ids_b) and torch.equal(w_a, w_b) and torch.equal(y_a, y_b)


def test_forward_repeatable():
    say("forward repeatable")
    m = gu.moe()
    d = MODEL
    lay = synth.make_layer(d, 77)
    dl = gu.device_layer(lay, d)
    x = synth.activations(333, d.hidden, 77).cuda()
    outs = []
    for _ in range(3):
        ids = torch.empty((333, d.top_k), dtype=torch.int32, device="cuda")
        y = m.moe_forward(gu.to_dims(d), dl, x, ids_out=ids)
        outs.append((ids, y))
    torch.cuda.synchronize()
    for ids, y in outs[1:]:
        assert torch.equal(ids, outs[0][0])
        assert torch.equal(y, outs[0][1])      # fixed-order combine: bitwise reproducible


@pytest.mark.parametrize("T", [1, 3, 300, 2048])
def test_forward_stages_compose(T):
    """moe_forward_stages run one stage at a time, in order, on a fresh
    workspace gives moe_forward's outputs bit for bit (the per-stage timing of
    the bench relies on it); the fused forms run whole in the router stage."""
    say("forward stages compose T", T)
    m = gu.moe()
    d = MODEL
    lay = synth.make_layer(d, 91 + T)
    dl = gu.device_layer(lay, d)
    md = gu.to_dims(d)
    x = synth.activations(T, d.hidden, 91 + T).cuda()
    ref_ids = torch.empty((T, d.top_k), dtype=torch.int32, device="cuda")
    ref = m.moe_forward(md, dl, x, ids_out=ref_ids)
    ws = m.moe_workspace(md, T)
    y = torch.empty((T, d.hidden), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((T, d.top_k), dtype=torch.int32, device="cuda")
    for st in range(len(m.STAGES)):
        m.moe_forward_stages(md, dl, x, y, ws, st, st, ids_out=ids)
    torch.cuda.synchronize()
    assert m.moe_workspace_errors(ws) == 0
    assert torch.equal(ids, ref_ids)
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("T", [1, 300, 2048])
def test_graph_capture_replays(T):
    """The layer makes no host round trip: it captures into a HIP graph, and
    every replay (with unrelated eager work and synchronisations between
    replays) reproduces the eager result.  T = 1: the fused layer; 300: the
    one-launch grouping; 2048: the two-launch grouping (more than 64 routing
    tiles)."""
    say("graph capture T", T)
    m = gu.moe()
    d = MODEL
    lay = synth.make_layer(d, 88 + T)
    dl = gu.device_layer(lay, d)
    md = gu.to_dims(d)
    x = synth.activations(T, d.hidden, 88 + T).cuda()
    ws = m.moe_workspace(md, T)
    ids_e = torch.empty((T, d.top_k), dtype=torch.int32, device="cuda")
    y_e = m.moe_forward(md, dl, x, ids_out=ids_e, workspace=ws).clone()
    ids_g = torch.empty_like(ids_e)
    y_g = torch.empty_like(y_e)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        m.moe_forward(md, dl, x, y=y_g, ids_out=ids_g, workspace=ws)
    a = torch.randn(512, 512, device="cuda")
    for rep in range(4):
        y_g.zero_()
        ids_g.fill_(-1)
        b = a @ a                      # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ids_g, ids_e), rep
        assert torch.equal(y_g, y_e), rep
        del b


# ------------------------------------------------------------------ device error word, residency

def test_group_flags_out_of_range_ids():
    """Caller-supplied ids outside [0, E) are skipped and flagged in the
    workspace's error word; the in-range slots are grouped as the oracle groups
    them on their own (counts, and the stable order of the remaining slots)."""
    say("group out-of-range ids")
    m = gu.moe()
    d = MODEL
    T, bm = 300, 128
    ids = _ids(T, d.n_experts, d.top_k, "uniform", 9)
    bad = ids.copy()
    bad[3, 2], bad[100, 0], bad[299, 7] = -1, d.n_experts, 1 << 20
    ws = torch.zeros(m.moe_group_workspace_bytes(gu.to_dims(d), T), dtype=torch.uint8, device="cuda")
    out = m.moe_group(gu.to_dims(d), torch.from_numpy(bad).cuda(), bm, workspace=ws)
    torch.cuda.synchronize()
    assert m.moe_workspace_errors(ws, clear=True) == m.MOE_DEVERR_EXPERT_ID
    assert m.moe_workspace_errors(ws) == 0
    ok = (bad >= 0) & (bad < d.n_experts)
    assert np.array_equal(out["counts"].cpu().numpy(), np.bincount(bad[ok], minlength=d.n_experts))
    inv = out["inv_perm"].cpu().numpy().reshape(T, d.top_k)
    assert np.all(inv[~ok] == -1)
    flat = np.flatnonzero(ok.reshape(-1))
    order = flat[np.argsort(bad.reshape(-1)[flat], kind="stable")]   # expert-major, ascending slot
    assert np.array_equal(out["perm"].cpu().numpy()[:order.size], order)
    # a clean call on the same workspace leaves the word clear
    m.moe_group(gu.to_dims(d), torch.from_numpy(ids).cuda(), bm, workspace=ws)
    assert m.moe_workspace_errors(ws) == 0


def test_fused_residency():
    """The fused layer's workgroups all fit on the device at once."""
    m = gu.moe()
    for T in (1, 2, 4):
        needed, resident = m.moe_fused_residency(gu.to_dims(MODEL), T)
        say("fused residency T", T, needed, resident)
        assert needed == 256 and resident >= needed
    with pytest.raises(m.MoeError):
        m.moe_fused_residency(gu.to_dims(MODEL), 5)
