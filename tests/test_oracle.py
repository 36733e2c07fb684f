"""Pins of the CPU oracle against things other than itself (CPU only).

Each test checks one step of the layer against a library routine, exact
rational arithmetic, a brute-force enumeration, a closed form or an invariant,
chosen so that a plausible slip in the oracle (a swapped nibble, a wrong tie
rule, a dropped term, an unstable permutation, a transposed matrix) fails.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import refs

TINY = oracle.Dims(hidden=128, inter=64, n_experts=16, top_k=4, group_size=64, shared_inter=64)


# ------------------------------------------------------------------ number formats

def test_half_decode_matches_numpy_all_patterns(oracle_lib):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.half_to_double(pats)
    ref = pats.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_decode_matches_torch_all_patterns(oracle_lib):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_to_double(pats)
    ref = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def _float_cases(rng):
    # random magnitudes over the whole float range, exact ties between bf16
    # neighbours, subnormals and values near the largest bf16.
    r = rng.standard_normal(20000) * np.exp2(rng.integers(-140, 120, 20000))
    bf = torch.from_numpy(rng.standard_normal(5000).astype(np.float32)).to(torch.bfloat16)
    bf_bits = bf.view(torch.int16).numpy().view(np.uint16).astype(np.uint32)
    ties = ((bf_bits << 16) | 0x8000).astype(np.uint32).view(np.float32)        # exactly half-way
    near = ((bf_bits << 16) | 0x7FFF).astype(np.uint32).view(np.float32)
    sub = (rng.integers(1, 1 << 23, 2000).astype(np.uint32)).view(np.float32)   # float32 subnormals
    big = np.float32([3.38e38, 3.389e38, -3.39e38, 1.0, -1.0, 0.0, -0.0])
    return np.concatenate([r.astype(np.float32), ties, near, sub, big])


def test_round_bf16_matches_torch_on_floats(oracle_lib):
    rng = np.random.default_rng(1)
    f = _float_cases(rng)
    got_bits = oracle.bf16_bits(f.astype(np.float64))
    ref_bits = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got_bits, ref_bits)


def test_round_bf16_single_rounding_of_doubles(oracle_lib):
    # doubles that are not floats: compare against exact rational rounding
    rng = np.random.default_rng(2)
    v = rng.standard_normal(3000) * np.exp2(rng.integers(-130, 100, 3000))
    # plus doubles just above/below a bf16 tie (where float double-rounding would go wrong)
    bf = torch.from_numpy(rng.standard_normal(500).astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    ulp = np.exp2(np.floor(np.log2(np.abs(bf))) - 7)
    v = np.concatenate([v, bf + ulp / 2 + ulp * 2.0 ** -30, bf + ulp / 2 - ulp * 2.0 ** -30, bf + ulp / 2])
    got = oracle.round_bf16(v)
    ref = np.array([float(refs.bf16_rn_fraction(float(a))) for a in v])
    assert np.array_equal(got, ref)
    # the round-to-odd + torch route used by the other tests agrees too
    assert np.array_equal(refs.bf16_rn(v), ref)


# ------------------------------------------------------------------ dequantisation

def test_dequant_exhaustive_codes_over_scale_range(oracle_lib):
    # every code against every fp16 scale in [2^-9, 2^-5) with bias = -8*scale
    s16 = np.arange(0x1800, 0x2800, dtype=np.uint16)          # fp16 values 2^-9 .. 2^-5
    b16 = (s16.view(np.float16) * np.float16(-8)).view(np.uint16)
    N, K, G = s16.size, 64, 64
    codes = np.zeros((N, 32), np.uint8)
    codes[:, :8] = np.array([0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE], np.uint8)  # k -> code k (k < 16)
    got = oracle.dequant(codes, s16[:, None], b16[:, None], N, K, G)
    s = s16.view(np.float16).astype(np.float64)
    exact = (np.arange(16)[None, :] - 8.0) * s[:, None]           # exact in float64 and float32
    ref = refs.bf16_rn_f32(exact.astype(np.float32))
    assert np.array_equal(got[:, :16], ref)
    assert np.all(got[:, 8] == 0.0)                                # code 8 is zero
    assert np.array_equal(got[:, 15], refs.bf16_rn_f32((7.0 * s).astype(np.float32)))
    assert np.array_equal(got[:, 16:], np.broadcast_to(got[:, :1], (N, 48)))  # code 0 elsewhere


def test_dequant_general_affine_and_nibble_order(oracle_lib):
    rng = np.random.default_rng(3)
    N, K, G = 8, 256, 64
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = np.float16(rng.uniform(0.001, 0.5, (N, K // G))).view(np.uint16)
    biases = np.float16(rng.uniform(-2, 2, (N, K // G))).view(np.uint16)
    got = oracle.dequant(codes, scales, biases, N, K, G)
    ref = refs.dequant_ref(codes, scales, biases, G)
    assert np.array_equal(got, ref)
    # swapping nibbles would change a row whose bytes are not palindromic
    swapped = ((codes & 0x0F) << 4) | (codes >> 4)
    assert not np.array_equal(oracle.dequant(swapped, scales, biases, N, K, G), got)


def test_dequant_power_of_two_scaling(oracle_lib):
    rng = np.random.default_rng(4)
    N, K, G = 4, 128, 64
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    s = np.float16(rng.uniform(0.005, 0.02, (N, K // G)))
    w1 = oracle.dequant(codes, s.view(np.uint16), (s * np.float16(-8)).view(np.uint16), N, K, G)
    s2 = s * np.float16(2)
    w2 = oracle.dequant(codes, s2.view(np.uint16), (s2 * np.float16(-8)).view(np.uint16), N, K, G)
    assert np.array_equal(w2, 2 * w1)


# ------------------------------------------------------------------ router

def test_router_matches_float64_matmul(oracle_lib):
    rng = np.random.default_rng(5)
    T, H, E = 9, 2048, 256
    x = synth.bf16_bits_numpy(synth.activations(T, H, seed=5))
    W = synth.router_weights(E, H, seed=5).numpy()
    wsg = synth.shared_gate_weights(H, seed=5).numpy()
    logits, s = oracle.router(x, W, None, wsg)
    xd = refs.bf16_rn_f32(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float().numpy())
    ref = (xd @ W.astype(np.float64).T)
    # different summation order in double: the fp32 results agree to within one ulp
    assert np.all(np.abs(logits - ref) <= np.spacing(np.abs(ref).astype(np.float32)))
    assert np.all(np.abs(s - xd @ wsg.astype(np.float64)) <= np.spacing(np.abs(s)))
    # the bias is one float32 add after rounding the dot product
    b = rng.standard_normal(E).astype(np.float32)
    lb, _ = oracle.router(x, W, b, wsg)
    assert np.array_equal(lb, (logits + b).astype(np.float32))


# ------------------------------------------------------------------ top-k

def test_topk_brute_force_with_ties(oracle_lib):
    rng = np.random.default_rng(6)
    T, E, k = 200, 256, 8
    logits = rng.standard_normal((T, E)).astype(np.float32)
    # inject exact ties at the k-th / (k+1)-th boundary and among the winners
    for t in range(0, T, 3):
        order = np.argsort(-logits[t], kind="stable")
        logits[t, order[k]] = logits[t, order[k - 1]]
        if t % 2 == 0:
            logits[t, order[1]] = logits[t, order[0]]
    logits[5, :] = 0.0
    logits[5, 7] = -0.0            # -0 and +0 tie
    logits[6, :] = np.float32(1.5)
    ids, w = oracle.topk(logits, k)
    rids, rw = refs.topk_ref(logits, k)
    assert np.array_equal(ids, rids)
    assert np.allclose(w, rw, rtol=2e-7, atol=0)
    assert np.array_equal(ids[5], np.arange(8)) and np.array_equal(ids[6], np.arange(8))


def test_topk_closed_forms(oracle_lib):
    E, k = 256, 8
    eq = np.zeros((1, E), np.float32)
    ids, w = oracle.topk(eq, k)
    assert np.array_equal(ids[0], np.arange(k)) and np.all(w == np.float32(1 / 8))
    lin = -np.arange(E, dtype=np.float32)[None, :]
    ids, w = oracle.topk(lin, k)
    ref = np.exp(-np.arange(k)) / np.exp(-np.arange(k)).sum()
    assert np.array_equal(ids[0], np.arange(k))
    assert np.allclose(w[0], ref, rtol=1e-7, atol=0)
    # shifting every logit by a constant changes nothing; relabelling experts relabels ids
    rng = np.random.default_rng(7)
    l = rng.standard_normal((50, E)).astype(np.float32)
    ids1, w1 = oracle.topk(l, k)
    pi = rng.permutation(E)
    ids2, w2 = oracle.topk(l[:, np.argsort(pi)], k)   # expert pi[e] now holds old expert e's logit
    assert np.array_equal(ids2, pi[ids1])
    assert np.allclose(w2, w1, rtol=1e-7)
    assert np.allclose(w1.astype(np.float64).sum(1), 1.0, atol=1e-6)


def test_sigmoid_gate(oracle_lib):
    from scipy.special import expit
    s = np.concatenate([[0.0], np.random.default_rng(8).standard_normal(1000) * 4]).astype(np.float32)
    g = oracle.sigmoid(s)
    assert g[0] == np.float32(0.5)
    assert np.array_equal(g, expit(s.astype(np.float64)).astype(np.float32))


# ------------------------------------------------------------------ grouping

def _group_ref(ids, E, BM):
    flat = ids.reshape(-1)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size, dtype=np.int32)
    tiles = [(e, offsets[e] + m * BM) for e in range(E) for m in range(-(-counts[e] // BM))]
    return counts, offsets, perm, inv, tiles


@pytest.mark.parametrize("T,k,E,BM,mode", [
    (1, 8, 256, 64, "uniform"), (37, 8, 256, 16, "uniform"), (512, 8, 256, 128, "uniform"),
    (64, 4, 16, 32, "one_expert"), (100, 8, 256, 64, "zipf"), (33, 2, 8, 1, "uniform")])
def test_group_against_stable_sort(oracle_lib, T, k, E, BM, mode):
    rng = np.random.default_rng(T * 7 + E)
    if mode == "one_expert":
        ids = np.zeros((T, k), np.int32)
        ids[:, 0] = 3
        ids[:, 1:] = np.arange(k - 1) + 4
    else:
        p = None
        if mode == "zipf":
            p = 1.0 / (np.arange(1, E + 1) ** 1.2)
            p /= p.sum()
        ids = np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    gr = oracle.group(ids, E, BM)
    counts, offsets, perm, inv, tiles = _group_ref(ids, E, BM)
    assert np.array_equal(gr.counts, counts) and gr.counts.sum() == T * k
    assert np.array_equal(gr.offsets, offsets)
    assert np.array_equal(gr.perm, perm) and np.array_equal(gr.inv_perm, inv)
    assert np.array_equal(np.sort(gr.perm), np.arange(T * k))           # bijection
    assert np.array_equal(gr.perm[gr.inv_perm], np.arange(T * k))
    assert gr.n_tiles == len(tiles)
    assert [tuple(r) for r in gr.block_map[:gr.n_tiles]] == [tuple(map(int, t)) for t in tiles]
    assert np.all(gr.block_map[gr.n_tiles:] == -1)
    # every segment is covered exactly once by tiles of at most BM rows
    cover = np.zeros(T * k, np.int32)
    for e, start in gr.block_map[:gr.n_tiles]:
        end = min(start + BM, gr.offsets[e + 1])
        assert 0 < end - start <= BM
        cover[start:end] += 1
        assert np.all(ids.reshape(-1)[gr.perm[start:end]] == e)
        assert np.all(np.diff(gr.perm[start:end]) > 0)                   # stable
    assert np.all(cover == 1)


def test_group_rejects_small_block_map(oracle_lib):
    ids = np.arange(16, dtype=np.int32).reshape(4, 4)
    with pytest.raises(ValueError):
        oracle.group(ids, 16, 1, n_max_tiles=15)


# ------------------------------------------------------------------ experts and the layer

def _tiny_layer(seed, d=TINY, T=24, zipf=False):
    lay = synth.make_layer(synth.Dims(**d.__dict__), seed, zipf_bias=zipf)
    ln = synth.layer_numpy(lay)
    lw = oracle.LayerWeights(ln["gate_up"], ln["down"], ln["sh_gate_up"], ln["sh_down"], ln["router_w"],
                             ln["shared_gate_w"], ln["router_bias"])
    x = synth.bf16_bits_numpy(synth.activations(T, d.hidden, seed))
    return lw, x


def _dense_weights(lw, d):
    H, I, E, G, Is = d.hidden, d.inter, d.n_experts, d.group_size, d.shared_inter
    dq = lambda m, e, N, K: refs.dequant_ref(m[0][e], m[1][e], m[2][e], G)
    return {"gu": np.stack([dq(lw.gate_up, e, 2 * I, H) for e in range(E)]),
            "dn": np.stack([dq(lw.down, e, H, I) for e in range(E)]),
            "sgu": dq(lw.sh_gate_up, 0, 2 * Is, H), "sdn": dq(lw.sh_down, 0, H, Is)}


# shared expert wider and narrower than the routed ones: an exchange of the two
# intermediate widths anywhere in the oracle fails these
UNEQUAL = [TINY, oracle.Dims(hidden=128, inter=64, n_experts=16, top_k=4, group_size=64, shared_inter=192),
           oracle.Dims(hidden=192, inter=128, n_experts=8, top_k=3, group_size=64, shared_inter=64)]


@pytest.mark.parametrize("d", UNEQUAL, ids=lambda d: f"I{d.inter}_Is{d.shared_inter}")
def test_layer_matches_dense_numpy_reference(oracle_lib, d):
    lw, x = _tiny_layer(11, d=d)
    res = oracle.layer(d, x, lw)
    rids, rw = refs.topk_ref(res["logits"], d.top_k)
    assert np.array_equal(res["ids"], rids)
    out_ref, y_ref = refs.layer_ref(x, res["ids"], res["w"], res["g"], _dense_weights(lw, d), d)
    out, y, _, _ = oracle.moe_tokens(d, x, res["ids"], res["w"], res["g"], lw, want_y=True)
    assert np.allclose(y, y_ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(oracle.bf16_to_double(out), out_ref)


@pytest.mark.parametrize("d", UNEQUAL, ids=lambda d: f"I{d.inter}_Is{d.shared_inter}")
def test_grouped_form_equals_token_loop_bitwise(oracle_lib, d):
    lw, x = _tiny_layer(12, d=d, T=40)
    res = oracle.layer(d, x, lw)
    ids, w, g = res["ids"], res["w"], res["g"]
    gr = oracle.group(ids, d.n_experts, 16)
    out, y, h_tok, hs = oracle.moe_tokens(d, x, ids, w, g, lw, want_y=True, want_h=True)
    h = oracle.grouped_swiglu(x, True, d.top_k, gr.perm, gr.offsets, lw.gate_up, d.hidden, d.inter, d.group_size)
    T, k = ids.shape
    assert np.array_equal(h[gr.inv_perm].reshape(T, k, d.inter), h_tok)
    o = oracle.grouped_down(h, gr.offsets, lw.down, d.hidden, d.inter, d.group_size)
    # the shared expert as a one-expert group over all tokens
    sh_off = np.array([0, T], np.int32)
    hs2 = oracle.grouped_swiglu(x, False, 1, np.arange(T, dtype=np.int32), sh_off, lw.sh_gate_up, d.hidden,
                                d.shared_inter, d.group_size)
    assert np.array_equal(hs2, hs)
    osh = oracle.grouped_down(hs2, sh_off, lw.sh_down, d.hidden, d.shared_inter, d.group_size)
    yy = np.zeros((T, d.hidden))
    for j in range(k):
        yy += w[:, j:j + 1].astype(np.float64) * o[gr.inv_perm.reshape(T, k)[:, j]]
    yy += g[:, None].astype(np.float64) * osh
    assert np.array_equal(yy, y)


def test_layer_invariants(oracle_lib):
    d = TINY
    lw, x = _tiny_layer(13, T=16)
    res = oracle.layer(d, x, lw)
    ids, w, g = res["ids"], res["w"], res["g"]
    out, y, _, _ = oracle.moe_tokens(d, x, ids, w, g, lw, want_y=True)
    # zero input -> zero output
    z = np.zeros_like(x)
    zo, _, _, _ = oracle.moe_tokens(d, z, ids, w, g, lw)
    assert np.all(oracle.bf16_to_double(zo) == 0)
    # doubling every down-projection scale and bias doubles the output exactly
    dbl = lambda m: (m[0], (m[1].view(np.float16) * np.float16(2)).view(np.uint16),
                     (m[2].view(np.float16) * np.float16(2)).view(np.uint16))
    lw2 = oracle.LayerWeights(lw.gate_up, dbl(lw.down), lw.sh_gate_up, dbl(lw.sh_down), lw.router_w,
                              lw.shared_gate_w)
    o2, y2, _, _ = oracle.moe_tokens(d, x, ids, w, g, lw2, want_y=True)
    assert np.array_equal(y2, 2 * y)
    assert np.array_equal(oracle.bf16_to_double(o2), 2 * oracle.bf16_to_double(out))
    # routed experts with every code 8 contribute nothing: out = bf16(g * shared)
    c8 = lambda m: (np.full_like(m[0], 0x88), m[1], m[2])
    lw3 = oracle.LayerWeights(c8(lw.gate_up), c8(lw.down), lw.sh_gate_up, lw.sh_down, lw.router_w,
                              lw.shared_gate_w)
    o3, y3, _, _ = oracle.moe_tokens(d, x, ids, w, g, lw3, want_y=True)
    lw4 = oracle.LayerWeights(lw.gate_up, lw.down, lw.sh_gate_up, lw.sh_down, lw.router_w, lw.shared_gate_w)
    zero_w = np.zeros_like(w)
    o4, y4, _, _ = oracle.moe_tokens(d, x, ids, zero_w, g, lw4, want_y=True)
    assert np.array_equal(y3, y4)
    # permuting tokens permutes outputs
    pi = np.random.default_rng(0).permutation(x.shape[0])
    op, _, _, _ = oracle.moe_tokens(d, x[pi], ids[pi], w[pi], g[pi], lw)
    assert np.array_equal(op, out[pi])
    # a subset of tokens gives the same rows as the full run
    sub = np.array([3, 0, 11], np.int32)
    os_, _, _, _ = oracle.moe_tokens(d, x, ids, w, g, lw, tokens=sub)
    assert np.array_equal(os_, out[sub])


def test_layer_full_dims_few_tokens(oracle_lib):
    # model dims, a handful of tokens: dense numpy reference on the experts used
    d = oracle.Dims()
    lay = synth.make_layer(synth.MODEL_DIMS, 21)
    ln = synth.layer_numpy(lay)
    lw = oracle.LayerWeights(ln["gate_up"], ln["down"], ln["sh_gate_up"], ln["sh_down"], ln["router_w"],
                             ln["shared_gate_w"])
    x = synth.bf16_bits_numpy(synth.activations(3, d.hidden, 21))
    res = oracle.layer(d, x, lw)
    used = sorted(set(res["ids"].reshape(-1).tolist()))
    G = d.group_size
    W = {"gu": {}, "dn": {}}
    for e in used:
        W["gu"][e] = refs.dequant_ref(ln["gate_up"][0][e], ln["gate_up"][1][e], ln["gate_up"][2][e], G)
        W["dn"][e] = refs.dequant_ref(ln["down"][0][e], ln["down"][1][e], ln["down"][2][e], G)
    W["sgu"] = refs.dequant_ref(*(a[0] for a in ln["sh_gate_up"]), G)
    W["sdn"] = refs.dequant_ref(*(a[0] for a in ln["sh_down"]), G)
    out_ref, _ = refs.layer_ref(x, res["ids"], res["w"], res["g"], W, d)
    assert np.array_equal(oracle.bf16_to_double(res["out"]), out_ref)
    assert np.allclose(res["w"].sum(1), 1.0, atol=1e-6)


# ------------------------------------------------------------------ grouped-query decode attention

def _bf16_bits_of(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)


def _attn_case(B, Hq, Hkv, S, D, seed):
    g = np.random.default_rng(seed)
    q = _bf16_bits_of(g.standard_normal((B, Hq, D)))
    k = _bf16_bits_of(g.standard_normal((B, Hkv, S, D)))
    v = _bf16_bits_of(g.standard_normal((B, Hkv, S, D)))
    return q, k, v


def test_gqa_single_position_returns_its_value_row(oracle_lib):
    """One cached position: its softmax weight is 1, so every query head of the
    group returns that value row exactly."""
    q, k, v = _attn_case(2, 16, 2, 5, 64, 1)
    out = oracle.gqa_decode(q, k, v, np.array([1, 1], np.int32), 0.125)
    vd = oracle.bf16_to_double(v)
    for h in range(16):
        assert np.array_equal(out[:, h], vd[:, h // 8, 0])


def test_gqa_equal_keys_average_the_values(oracle_lib):
    """All keys equal: every score is equal, so the output is the plain mean of
    the value rows in use."""
    q, k, v = _attn_case(1, 8, 2, 37, 128, 2)
    k[:] = k[:, :, :1, :]
    L = 29
    out = oracle.gqa_decode(q, k, v, np.array([L], np.int32), 0.0883883)
    mean = oracle.bf16_to_double(v)[0, :, :L].mean(axis=1)          # [Hkv][D]
    for h in range(8):
        assert np.allclose(out[0, h], mean[h // 4], rtol=0, atol=1e-13)


@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (8, 4), (4, 4)])
def test_gqa_head_mapping_contiguous_groups(oracle_lib, Hq, Hkv):
    """Value rows of key/value head j are the constant (j + 1) / 4: query head h
    must return h // (Hq / Hkv) + 1 over 4 (a mapping h % Hkv fails for Hkv > 1
    and Hq > Hkv)."""
    q, k, v = _attn_case(1, Hq, Hkv, 19, 64, 3)
    for j in range(Hkv):
        v[0, j] = _bf16_bits_of(np.full((19, 64), (j + 1) / 4.0))
    out = oracle.gqa_decode(q, k, v, np.array([19], np.int32), 0.125)
    for h in range(Hq):
        assert np.allclose(out[0, h], (h // (Hq // Hkv) + 1) / 4.0, rtol=0, atol=1e-14)


def test_gqa_two_positions_logistic_closed_form(oracle_lib):
    """Two positions: out = v0 + sigmoid(scale * q.(k1 - k0)) * (v1 - v0), the dot
    products summed exactly with math.fsum."""
    q, k, v = _attn_case(1, 2, 1, 2, 64, 4)
    scale = 0.3
    out = oracle.gqa_decode(q, k, v, np.array([2], np.int32), scale)
    qd, kd, vd = oracle.bf16_to_double(q)[0], oracle.bf16_to_double(k)[0, 0], oracle.bf16_to_double(v)[0, 0]
    for h in range(2):
        delta = scale * (math.fsum(qd[h] * kd[1]) - math.fsum(qd[h] * kd[0]))
        sig = 1.0 / (1.0 + math.exp(-delta))
        assert np.allclose(out[0, h], vd[0] + sig * (vd[1] - vd[0]), rtol=0, atol=1e-13)


def test_gqa_dominant_key_selects_its_row(oracle_lib):
    """A key equal to 64 times the query outscores every other position by
    hundreds: the output is that position's value row to double precision."""
    q, k, v = _attn_case(1, 1, 1, 50, 64, 5)
    k = _bf16_bits_of(oracle.bf16_to_double(k) * 0.01)
    k[0, 0, 31] = _bf16_bits_of(64.0 * oracle.bf16_to_double(q)[0, 0])
    out = oracle.gqa_decode(q, k, v, np.array([50], np.int32), 1.0)
    assert np.allclose(out[0, 0], oracle.bf16_to_double(v)[0, 0, 31], rtol=1e-12, atol=0)


def test_gqa_reads_only_positions_in_use(oracle_lib):
    """Positions at or past a sequence's length hold NaN: the output stays finite
    and equals the result on the cache cut to that length; length 0 gives zeros."""
    q, k, v = _attn_case(3, 4, 2, 40, 64, 6)
    lens = np.array([40, 13, 0], np.int32)
    for b in range(3):
        k[b, :, lens[b]:] = 0x7FC0
        v[b, :, lens[b]:] = 0x7FC0
    out = oracle.gqa_decode(q, k, v, lens, 0.125)
    assert np.all(np.isfinite(out))
    assert np.array_equal(out[2], np.zeros((4, 64)))
    cut = oracle.gqa_decode(q[1:2], k[1:2, :, :13].copy(), v[1:2, :, :13].copy(), np.array([13], np.int32), 0.125)
    assert np.array_equal(out[1], cut[0])


def test_gqa_matches_torch_sdpa_float64(oracle_lib):
    """torch's scaled_dot_product_attention in float64 with enable_gqa (query
    heads grouped onto key/value heads by h // (Hq / Hkv)), ragged lengths."""
    import torch.nn.functional as F
    B, Hq, Hkv, S, D = 3, 16, 2, 70, 128
    q, k, v = _attn_case(B, Hq, Hkv, S, D, 7)
    lens = np.array([70, 1, 33], np.int32)
    scale = 1.0 / math.sqrt(D)
    out = oracle.gqa_decode(q, k, v, lens, scale)
    qd, kd, vd = (torch.from_numpy(oracle.bf16_to_double(a)) for a in (q, k, v))
    for b in range(B):
        L = int(lens[b])
        ref = F.scaled_dot_product_attention(qd[b:b + 1, :, None, :], kd[b:b + 1, :, :L], vd[b:b + 1, :, :L],
                                             scale=scale, enable_gqa=True)[0, :, 0]
        assert np.allclose(out[b], ref.numpy(), rtol=1e-12, atol=1e-14)
