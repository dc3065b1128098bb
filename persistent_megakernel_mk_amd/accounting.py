"""Byte accounting of a decode step: the algorithmic bytes the step must move, and the byte formulas
the pages use for the Kimi K3 expert formats.

A decode step at small batch streams every weight it touches about once, at roughly one FLOP per byte
(page "Kimi K3's TPU megakernel: 92 layers in one Pallas call, and what 709 tokens a second measures",
section "Why one user at a time is a bandwidth problem"); its floor is bytes over bandwidth (same page,
section "The bandwidth arithmetic"). Algorithmic bytes count each touched weight once, the K/V (or
latent) cache rows read and the new rows written, the linear-attention state read and written, the
embedding rows gathered and the logits (or hidden states) written. Over-fetch, padding and reductions
are not counted.
"""
from __future__ import annotations

import re
from typing import Dict

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth


def mxfp4_bytes(n_params: int) -> float:
    """MXFP4: 4-bit E2M1 values plus one 8-bit E8M0 scale per 32 values = 4.25 bits per value."""
    return n_params * 4.25 / 8


def fp8_rowscaled_bytes(rows: int, cols: int, rows_per_scale: int = 256) -> float:
    """FP8 E4M3 values with one bf16 scale per `rows_per_scale` rows of each column."""
    return rows * cols * (1 + 2 / rows_per_scale)


def kimi_expert_bytes(hidden: int = 7168, expert_ffn: int = 1536) -> Dict[str, float]:
    """One routed expert (gate, up, down of hidden x expert_ffn), stored as the pages describe:
    all three projections in MXFP4, or gate/up re-encoded to FP8 with a bf16 scale per 256 rows and down
    kept in MXFP4 (page "Kimi K3's TPU megakernel ...", section "How it maps onto a TPU v7")."""
    n = hidden * expert_ffn
    return {"mxfp4": mxfp4_bytes(3 * n),
            "fp8_gate_up_mxfp4_down": 2 * fp8_rowscaled_bytes(hidden, expert_ffn) + mxfp4_bytes(n)}


def roofline_floor_ms(bytes_per_token: float, devices: int, gbs_per_device: float) -> float:
    return bytes_per_token / (devices * gbs_per_device * 1e9) * 1e3


def expected_union(n_experts: int, top_k: int, tokens: int) -> float:
    """Expected number of distinct experts selected by `tokens` independent uniform top-k draws."""
    if n_experts <= 0:
        return 0.0
    return n_experts * (1.0 - (1.0 - top_k / n_experts) ** tokens)


def _matrix_bytes(spec) -> float:
    if spec.kind == "bf16":
        return spec.numel * 2
    if spec.kind == "nvfp4":  # E2M1 codes (half a byte) + one E4M3 scale per 16 values + the tensor scale
        return spec.numel // 2 + spec.numel // 16 + 4
    if spec.kind == "mxfp4":  # gate/up re-encoded to FP8 with a bf16 scale per 256; down kept in MXFP4
        if spec.name.endswith(".wd"):
            return mxfp4_bytes(spec.numel)
        return fp8_rowscaled_bytes(spec.numel, 1)
    return 0


def step_bytes(cfg, batch: int, position: int, rows: int = 1, union=None) -> Dict[str, float]:
    """Algorithmic bytes of one decode step (rows = 1) or verify block (rows = 8, batch = 1).
    `position` is the position of the (first) new token, so position cached rows are read per sequence
    and kv head (or latent rows per sequence). Mixture-of-experts layers count the router, the shared
    experts and each routed expert in the batch's union once: `union` gives the union size per MoE layer
    (counted from the step's routing), else its expectation under uniform routing is used."""
    from persistent_megakernel_mk_amd import synth

    seqs = batch
    toks = batch * rows
    moe_layers = [l for l in range(cfg.n_layers) if cfg.ffns[l] == "moe"]
    if union is None:
        union = [expected_union(cfg.n_experts, cfg.top_k, toks)] * len(moe_layers)
    union_of = dict(zip(moe_layers, union))
    w = 0.0
    for s in synth.weight_specs(cfg):
        if s.name == "embed":
            continue  # only the gathered rows are read
        m = re.match(r"l(\d+)\.e(\d+)\.", s.name)
        if m:  # routed expert: counted through the union below
            if int(m.group(2)) == 0:
                w += union_of[int(m.group(1))] * _matrix_bytes(s)
            continue
        w += _matrix_bytes(s)
    emb = toks * cfg.hidden * 2 if cfg.vocab else toks * cfg.hidden * 4
    kv = lin = 0
    for l in range(cfg.n_layers):
        m = cfg.mixers[l]
        if m == "gqa":
            row = cfg.n_kv_heads * cfg.head_dim * 2  # one position of K (or V), bf16
            kv += seqs * 2 * (position * row) + toks * 2 * row
        elif m == "mla":
            row = (cfg.kv_rank + cfg.rope_dim) * 2  # one latent row, bf16
            kv += seqs * position * row + toks * row
        elif m in ("gdn", "kda"):
            st = cfg.lin_heads * cfg.d_v * cfg.d_k * 4
            if rows > 1:  # verify: the live state is read, one snapshot per row is written, and the
                lin += seqs * st + rows * st  # commit selects a snapshot slot (nothing copied back)
            else:
                lin += seqs * 2 * st
    out = toks * cfg.vocab * 4 if cfg.vocab else toks * cfg.hidden * 4
    total = w + emb + kv + lin + out
    return {"weights": w, "embed": emb, "kv": kv, "lin_state": lin, "out": out, "total": total}
