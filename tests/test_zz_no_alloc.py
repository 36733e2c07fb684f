"""moe_forward_noalloc (the library's own device scratch, no workspace)
against moe_forward on the same inputs through the C ABI: the same kernels
on the same data, so every output must be bitwise equal.  Calls in a row share
the scratch, each later one with fewer tokens than the one before, across the
grouped and the fused path."""

from __future__ import annotations

import sys

import pytest
import torch

import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def test_noalloc_equals_forward():
    m = gu.moe()
    d = synth.MODEL_DIMS
    md = gu.to_dims(d)
    lay = synth.make_layer(d, 601)
    dl = gu.device_layer(lay, d)
    for T in (512, 300, 37, 4, 3, 1):      # each call smaller than the one before
        print("[case] noalloc T", T, file=sys.stderr, flush=True)
        x = synth.activations(T, d.hidden, 601 + T).cuda()
        outs = []
        for noalloc in (True, False):
            logits = torch.empty((T, d.n_experts), dtype=torch.float32, device="cuda")
            ids = torch.empty((T, d.top_k), dtype=torch.int32, device="cuda")
            w = torch.empty((T, d.top_k), dtype=torch.float32, device="cuda")
            y = torch.empty((T, d.hidden), dtype=torch.bfloat16, device="cuda")
            if noalloc:
                m.moe_forward_noalloc(md, dl, x, y, logits_out=logits, ids_out=ids, w_out=w)
            else:
                m.moe_forward(md, dl, x, y=y, logits_out=logits, ids_out=ids, w_out=w)
            outs.append((y, logits, ids, w))
        torch.cuda.synchronize()
        for a, b in zip(*outs):
            assert torch.equal(a, b), T


def test_noalloc_parity_against_oracle():
    """The no-allocation call on its own, checked against the oracle (logits,
    routing bit for bit, layer output within the parity bar)."""
    m = gu.moe()
    d = synth.MODEL_DIMS
    md = gu.to_dims(d)
    for T in (200, 2):
        print("[case] noalloc vs oracle T", T, file=sys.stderr, flush=True)
        lay = synth.make_layer(d, 611 + T)
        dl = gu.device_layer(lay, d)
        x = synth.activations(T, d.hidden, 611 + T)
        y = torch.empty((T, d.hidden), dtype=torch.bfloat16, device="cuda")
        logits = torch.empty((T, d.n_experts), dtype=torch.float32, device="cuda")
        ids = torch.empty((T, d.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, d.top_k), dtype=torch.float32, device="cuda")
        m.moe_forward_noalloc(md, dl, x.cuda(), y, logits_out=logits, ids_out=ids, w_out=w)
        torch.cuda.synchronize()
        gu.check_outputs(d, lay, x, y, logits, ids, w)
