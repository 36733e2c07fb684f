"""The benchmark's work figures (CPU only): the flop and byte counts that turn
measured times into roofline fractions, checked against values computed here
from the layer's shape, and the rule that the committed HBM-traffic figure is
reported only for the GEMM source it was measured on."""

import importlib.util
import os

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_flops_per_token(bench):
    d = synth.MODEL_DIMS   # hidden 2048, inter 512, 256 experts, top-8, shared inter 512
    # 8 routed + 1 shared expert, three H x I matrices each, 2 flops per multiply-add
    assert bench.layer_flops_per_token(d) == 9 * 3 * 2 * 2048 * 512 == 56_623_104
    # gate/up only: (8 + 1) experts x 2I rows x H, per token
    assert bench.gate_up_flops(d, 4096) == 2 * 4096 * 9 * 1024 * 2048 == 154_618_822_656
    assert bench.gate_up_flops(d, 4096) / (4096 * bench.layer_flops_per_token(d)) == pytest.approx(2 / 3)


def test_expert_and_decode_bytes(bench):
    d = synth.MODEL_DIMS
    # int4 codes (half a byte per weight) plus an fp16 scale and an fp16 bias per 64 weights
    weights = 3 * 2048 * 512
    assert bench.expert_bytes(d) == weights // 2 + 2 * 2 * weights // 64 == 1_769_472
    # one decode layer: 8 routed experts + the shared one, the fp32 router [E][H]
    # and shared-gate row [H], the bf16 token in and out
    assert bench.decode_bytes_per_layer(d) == 9 * 1_769_472 + 256 * 2048 * 4 + 2048 * 4 + 2 * 2048 * 2
    assert bench.decode_bytes_per_layer(d) == 18_038_784


def test_traffic_reported_only_for_the_measured_source(bench, tmp_path, monkeypatch):
    prof = tmp_path / "traffic.md"
    prof.write_text("- hbm_bytes_per_launch: `123456`\n- gemm_source_sha256_16: `" + bench.gemm_source_hash() + "`\n")
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(prof))
    assert bench.measured_traffic() == 123456
    prof.write_text("- hbm_bytes_per_launch: `123456`\n- gemm_source_sha256_16: `0000000000000000`\n")
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(tmp_path / "absent.md"))
    assert bench.measured_traffic() is None


def test_committed_traffic_profile_parses(bench):
    """The committed profile carries both keys the bench reads, and its byte
    count exceeds the launch's algorithmic bytes (re-reads only add)."""
    vals = {}
    for line in open(os.path.join(ROOT, bench.TRAFFIC_PROFILE)):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    assert len(vals["gemm_source_sha256_16"]) == 16
    assert int(vals["hbm_bytes_per_launch"]) > int(vals["algorithmic_bytes_per_launch"]) > 0
