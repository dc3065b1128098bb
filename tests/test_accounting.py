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
