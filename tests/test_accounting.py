"""Byte accounting pinned to the figures the pages print (tests/golden/page_byte_figures.json)."""
import json
import os

from persistent_megakernel_mk_amd import accounting as A

G = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "page_byte_figures.json")))


def test_expert_byte_formulas_reproduce_page_figures():
    e = A.kimi_expert_bytes()
    assert e["mxfp4"] == G["mxfp4_expert_bytes"]
    assert e["fp8_gate_up_mxfp4_down"] == G["fp8_gate_up_expert_bytes"]
    assert round(G["experts_per_token"] * e["mxfp4"] / 1e9, 2) == G["expert_gb_mxfp4"]
    assert round(G["experts_per_token"] * e["fp8_gate_up_mxfp4_down"] / 1e9, 2) == G["expert_gb_fp8"]


def test_bandwidth_floor_arithmetic():
    per_tok = G["trunk_gb"] * 1e9 + G["experts_per_token"] * G["fp8_gate_up_expert_bytes"]
    assert round(per_tok / 1e9, 2) == G["tpu_bytes_per_token_gb"]
    assert 16 * 7380 == G["tpu_aggregate_gbs"]
    ms = A.roofline_floor_ms(per_tok, 16, 7380)
    assert round(ms, 2) == G["tpu_floor_ms"]
    assert round(1e3 / ms) == G["tpu_ceiling_tok_s"]
    gb = G["trunk_gb"] * 1e9 + G["experts_per_token"] * G["mxfp4_expert_bytes"]
    assert round(gb / 1e9, 2) == G["gb200_bytes_per_token_gb"]
    ms2 = A.roofline_floor_ms(gb, 16, 8000)
    assert round(ms2, 2) == G["gb200_floor_ms"] and round(1e3 / ms2) == G["gb200_ceiling_tok_s"]


def test_step_bytes_hybrid_27b():
    from persistent_megakernel_mk_amd import synth

    cfg = synth.CONFIGS["c1"]
    b1 = A.step_bytes(cfg, 1, cfg.ctx)
    # weights touched: every matrix once except the embedding table (one row gathered)
    assert 40.9e9 < b1["weights"] < 41.1e9
    assert b1["lin_state"] == 48 * 2 * 16 * 128 * 128 * 4
    assert b1["kv"] == 16 * (2 * 4096 * 4 * 128 * 2 + 2 * 4 * 128 * 2)
    assert 41.1e9 < b1["total"] < 41.4e9
    b8 = A.step_bytes(cfg, 8, cfg.ctx)
    assert b8["weights"] == b1["weights"] and b8["kv"] > 7 * b1["kv"]


def test_expected_union_closed_forms():
    assert abs(A.expected_union(384, 8, 1) - 8.0) < 1e-9  # one token selects exactly k experts
    assert abs(A.expected_union(16, 16, 5) - 16.0) < 1e-12  # top-k = E touches every expert
    assert round(A.expected_union(384, 8, 8), 1) == 59.5
    assert round(A.expected_union(256, 8, 8), 1) == 57.4


def test_step_bytes_expert_latent_and_verify_configs():
    from persistent_megakernel_mk_amd import synth

    c3 = synth.CONFIGS["c3"]
    b = A.step_bytes(c3, 8, c3.ctx)
    # latent cache: 4096 rows of (512 + 64) bf16 read per sequence, one row appended per token
    assert b["kv"] == 8 * (4096 * 576 * 2 + 576 * 2)
    assert b["lin_state"] == 3 * 8 * 2 * 32 * 128 * 128 * 4
    assert 22.6e9 < b["total"] < 22.8e9
    # a routed expert enters once per layer however many rows select it
    one = A.step_bytes(c3, 8, c3.ctx, union=[1.0] * 4)
    two = A.step_bytes(c3, 8, c3.ctx, union=[2.0] * 4)
    assert two["weights"] - one["weights"] == 4 * 3 * 2048 * 7168 * 2
    c4 = synth.CONFIGS["c4"]
    n = 2048 * 6144
    e = A.step_bytes(c4, 1, c4.ctx, union=[8.0] * 8)
    f = A.step_bytes(c4, 1, c4.ctx, union=[9.0] * 8)
    assert f["weights"] - e["weights"] == 8 * 3 * (n // 2 + n // 16 + 4)  # NVFP4: 0.5625 B per weight
    assert 3.0e9 < A.step_bytes(c4, 1, c4.ctx)["total"] < 3.1e9
    assert 11.8e9 < A.step_bytes(c4, 8, c4.ctx)["total"] < 12.0e9
    c2 = synth.CONFIGS["c2"]
    v = A.step_bytes(c2, 1, c2.ctx, rows=8)
    st = 16 * 128 * 128 * 4
    assert v["lin_state"] == 48 * (st + 8 * st)  # live state read once, eight snapshots written
    assert v["out"] == 8 * 151936 * 4
