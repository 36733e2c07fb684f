"""Pins of the seeded input generator (CPU only)."""

import json
import os

import numpy as np
import torch

import synth


def test_splitmix64_published_vectors():
    # splitmix64 seeded with 1234567: first outputs of the reference generator
    # (Vigna's splitmix64.c / Java's SplittableRandom use the same stream).
    expect = [6457827717110365317, 3203168211198807973, 9817491932198370423,
              4593380528125082431, 16408922859458223821]
    assert [synth.splitmix64_int(1234567, i) for i in range(5)] == expect
    keys = torch.tensor([1234567], dtype=torch.int64)
    got = synth.splitmix64(keys[:, None], torch.arange(5)[None, :])[0]
    assert [v & ((1 << 64) - 1) for v in got.tolist()] == expect


def test_q4_draws_are_well_formed():
    codes, scales, biases = synth.q4_matrix(3, 64, 256, 64, seed=9, layer=2, matrix="down")
    assert codes.shape == (3, 64, 128) and scales.shape == (3, 64, 4)
    nib = torch.cat([codes & 15, codes >> 4]).flatten().numpy()
    hist = np.bincount(nib, minlength=16)
    expected = nib.size / 16
    chi2 = ((hist - expected) ** 2 / expected).sum()
    assert chi2 < 50          # 15 dof; p ~ 1e-5
    s = scales.view(torch.float16).float()
    b = biases.view(torch.float16).float()
    assert float(s.min()) >= 0.005 - 1e-6 and float(s.max()) < 0.02
    assert torch.equal(b, -8 * s)
    # different matrices / layers / experts draw different bytes
    c2, _, _ = synth.q4_matrix(3, 64, 256, 64, seed=9, layer=3, matrix="down")
    assert not torch.equal(codes, c2)
    assert not torch.equal(codes[0], codes[1])
    # drawing a subset of experts reproduces the same bytes
    c3, _, _ = synth.q4_matrix(2, 64, 256, 64, seed=9, layer=2, matrix="down")
    assert torch.equal(codes[:2], c3)


def test_zipf_bias_skews_load():
    b = synth.zipf_router_bias(256, seed=105)
    got = np.sort(-b.numpy().astype(np.float64) / 1.2)
    assert np.allclose(got, np.log1p(np.arange(256)), rtol=1e-6, atol=1e-6)


def test_format_matches_pages_checkpoint_size():
    facts = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))
    d = synth.MODEL_DIMS
    assert facts["routed_experts"]["value"] == d.n_experts
    assert facts["experts_per_token"]["value"] == d.top_k
    # int4 codes plus an fp16 scale and an fp16 bias per 64 weights = 4.5 bits per weight
    bytes_per_expert = 2 * d.inter * d.hidden // 2 + d.hidden * d.inter // 2 + 2 * 2 * (3 * d.inter * d.hidden // 64)
    bits = 8 * bytes_per_expert / (3 * d.inter * d.hidden)
    assert bits == 4.5
    params = facts["total_params_billion"]["value"] * 1e9
    gb_4bit = params * bits / 8 / 1e9
    assert abs(gb_4bit - facts["checkpoint_4bit_gb"]["value"]) / facts["checkpoint_4bit_gb"]["value"] < 0.03
    assert abs(params * 2 / 1e9 - facts["checkpoint_bf16_gb"]["value"]) < 1
