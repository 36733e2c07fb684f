"""Helpers shared by the GPU parity tests: device copies of synthetic layers,
the oracle's view of the same bytes, and the error metrics of the parity bar."""

from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

# Parity bar for the layer output (bf16): max|gpu-oracle| / max|oracle| and
# sum|gpu-oracle| / sum|oracle|.
MAX_REL_TOL = 1e-2
L1_REL_TOL = 2e-3
LOGIT_ATOL = 1e-4      # router logits (fp32 accumulate vs double)
WEIGHT_ATOL = 2e-6     # routing weights and shared gate


def moe():
    import sparse_moe_softmax_amd
    return sparse_moe_softmax_amd


def to_dims(d):
    return moe().Dims(d.hidden, d.inter, d.n_experts, d.top_k, d.group_size, d.shared_inter)


def device_layer(lay: synth.Layer, d):
    t = lambda a: None if a is None else a.to("cuda").contiguous()
    q = lambda m: tuple(t(a) for a in m)
    return moe().LayerWeights(to_dims(d), q(lay.gate_up), q(lay.down), q(lay.sh_gate_up), q(lay.sh_down),
                              t(lay.router_w), t(lay.shared_gate_w), t(lay.router_bias))


def oracle_layer(lay: synth.Layer) -> oracle.LayerWeights:
    ln = synth.layer_numpy(lay)
    return oracle.LayerWeights(ln["gate_up"], ln["down"], ln["sh_gate_up"], ln["sh_down"], ln["router_w"],
                               ln["shared_gate_w"], ln["router_bias"])


def odims(d) -> oracle.Dims:
    return oracle.Dims(d.hidden, d.inter, d.n_experts, d.top_k, d.group_size, d.shared_inter)


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 / int16 tensor -> numpy uint16 bit patterns."""
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def out_errors(gpu_bits: np.ndarray, ref_bits: np.ndarray):
    g = oracle.bf16_to_double(gpu_bits)
    r = oracle.bf16_to_double(ref_bits)
    diff = np.abs(g - r)
    max_rel = float(diff.max() / max(np.abs(r).max(), 1e-30))
    l1_rel = float(diff.sum() / max(np.abs(r).sum(), 1e-30))
    return max_rel, l1_rel


def assert_layer_close(gpu_bits, ref_bits, what=""):
    max_rel, l1_rel = out_errors(gpu_bits, ref_bits)
    assert np.all(np.isfinite(oracle.bf16_to_double(gpu_bits))), f"{what}: non-finite output"
    assert max_rel <= MAX_REL_TOL, f"{what}: max rel {max_rel:.3e}"
    assert l1_rel <= L1_REL_TOL, f"{what}: L1 rel {l1_rel:.3e}"
    return max_rel, l1_rel


def forward_and_check(d, lay: synth.Layer, x_cpu: torch.Tensor, tokens=None, threads: int = 0, dl=None,
                      host_routing: bool = False, logit_atol: float = LOGIT_ATOL):
    """Run moe_forward on the GPU and check it against the oracle with the
    shared-logits protocol: logits within logit_atol; the oracle's top-k of
    the GPU logits equals the GPU ids bit for bit and its weights are within
    WEIGHT_ATOL; the oracle layer output from those ids meets the parity bar
    on ``tokens`` (all tokens if None).

    host_routing: run moe_forward_host_routing instead (grouped path only).
    It has no logits output; its router and top-k are moe_forward's stages, so
    the logits come from those stages run alone on a second workspace."""
    m = moe()
    dl = dl or device_layer(lay, d)
    T = x_cpu.shape[0]
    x = x_cpu.to("cuda")
    md = to_dims(d)
    logits = torch.empty((T, d.n_experts), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, d.top_k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, d.top_k), dtype=torch.float32, device="cuda")
    ws = m.moe_workspace(md, T)
    if host_routing:
        y = m.moe_forward_host_routing(md, dl, x, ids_out=ids, w_out=wts, workspace=ws)
        ws2 = m.moe_workspace(md, T)
        scratch = torch.empty((T, d.hidden), dtype=torch.bfloat16, device="cuda")
        m.moe_forward_stages(md, dl, x, scratch, ws2, 0, 1, logits_out=logits)
    else:
        y = m.moe_forward(md, dl, x, logits_out=logits, ids_out=ids, w_out=wts, workspace=ws)
    torch.cuda.synchronize()
    assert m.moe_workspace_errors(ws) == 0
    return check_outputs(d, lay, x_cpu, y, logits, ids, wts, tokens=tokens, threads=threads, logit_atol=logit_atol)


def check_outputs(d, lay: synth.Layer, x_cpu: torch.Tensor, y, logits, ids, wts, tokens=None, threads: int = 0,
                  logit_atol: float = LOGIT_ATOL):
    """The shared-logits parity protocol on outputs the GPU produced (see
    forward_and_check)."""
    T = x_cpu.shape[0]
    ow = oracle_layer(lay)
    xb = synth.bf16_bits_numpy(x_cpu)
    o_logits, o_s = oracle.router(xb, ow.router_w, ow.router_bias, ow.shared_gate_w, threads)
    g_logits = logits.cpu().numpy()
    assert np.abs(g_logits - o_logits).max() <= logit_atol
    o_ids, o_w = oracle.topk(g_logits, d.top_k)
    g_ids = ids.cpu().numpy()
    assert np.array_equal(g_ids, o_ids)
    assert np.abs(wts.cpu().numpy() - o_w).max() <= WEIGHT_ATOL
    o_g = oracle.sigmoid(o_s)
    tok = np.arange(T, dtype=np.int32) if tokens is None else np.asarray(tokens, np.int32)
    o_out, _, _, _ = oracle.moe_tokens(odims(d), xb, o_ids, o_w, o_g, ow, tokens=tok, threads=threads)
    g_out = bits(y)[tok]
    errs = assert_layer_close(g_out, o_out, f"T={T}")
    return {"y": y, "ids": g_ids, "logits": g_logits, "errs": errs, "ref_bits": o_out}
