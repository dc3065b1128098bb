"""The C ABI library without a GPU: it loads, exports every entry point include/mk.h declares, validates
configurations, and builds the step schedule (host-only contexts, hip_device = -1)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "mk.h")).read()
    return sorted(set(re.findall(r"^\s*(?:mk_status|void|const char \*|int)\s*\*?\s*(mk_[a-z_]+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def mkmod():
    from persistent_megakernel_mk_amd import mk

    return mk


def test_library_exports_every_declared_symbol(mkmod):
    lib = mkmod.load()
    names = declared_functions()
    assert "mk_decode_step" in names and "mk_verify_step" in names and "mk_load_weights" in names
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layouts_match_header(mkmod):
    # sizes implied by the header's field lists (LP64)
    assert ctypes.sizeof(mkmod.Config) == 4 * (3 + 2 * 128 + 1 + 3 + 3 + 5 + 5 + 2) + 8
    assert ctypes.sizeof(mkmod.WeightDesc) == 16 + 16 + 16 + 8
    assert ctypes.sizeof(mkmod.StepIO) == 8 * 8
    assert ctypes.sizeof(mkmod.Buffers) == 8 * (2 + 4 * 128)


def test_invalid_configs_are_rejected(mkmod, synth):
    from dataclasses import replace

    cfg = synth.CONFIGS["c1s"]
    for bad, status in [(replace(cfg, hidden=1000), 3), (replace(cfg, n_layers=0, mixers=(), ffns=()), 1),
                        (replace(cfg, head_dim=96), 3), (replace(cfg, n_kv_heads=4), 1)]:
        with pytest.raises(mkmod.MKError) as ei:
            mkmod.HostContext(bad)
        assert ei.value.status == status
    with pytest.raises(mkmod.MKError):
        mkmod.HostContext(cfg, max_batch=17)
    mkmod.HostContext(cfg, max_batch=16)  # dense stacks take up to 16 rows
    with pytest.raises(mkmod.MKError) as ei:  # mixture-of-experts layers at most 8
        mkmod.HostContext(synth.CONFIGS["c4s"], max_batch=9)
    assert ei.value.status == 3


def test_schedule_layer_pattern_and_phase_counts(mkmod, synth):
    cfg = synth.CONFIGS["c1"]
    h = mkmod.HostContext(cfg, max_batch=8)
    ph = h.phases(1)
    types = [p[0] for p in ph]
    # embed; per GDN layer: product, delta rule, product, product, product; per GQA layer one more
    # (attention partials + merge); LM head; final
    n_gqa = sum(1 for m in cfg.mixers if m == "gqa")
    assert n_gqa == 16 and cfg.mixers[3] == "gqa" and cfg.mixers[0] == "gdn"
    assert len(ph) == 1 + 5 * 64 + n_gqa + 2 == h.sizes.n_phases
    assert types[0] == 1 and types[-1] == 6 and types[-2] == 2
    assert types.count(3) == 48 and types.count(4) == 16 and types.count(5) == 16
    # the 4th layer (index 3) uses attention: embed + 3 * 5 phases precede it
    assert types[16] == 2 and types[17] == 4 and types[18] == 5


def test_split_choice_respects_lds_and_waves(mkmod, synth):
    cfg = synth.CONFIGS["c1"]
    h = mkmod.HostContext(cfg, max_batch=16)
    for rows in range(1, 17):
        cols = 2 * rows if rows <= 8 else 32  # bf16 high and low halves: 16 columns per group of 8 rows
        for p in h.phases(rows):
            if p[0] != 2:
                continue
            N, K, T, KF, S, nf = p[2], p[3], p[4], p[5], p[6], p[7]
            assert T * 16 == N and KF * 32 == K
            # four streaming waves split a k-split (evenly up to 8 rows; above, runs one fragment apart)
            assert S >= 1 and KF == S * nf and (nf % 4 == 0 if rows <= 8 else nf >= 4)
            assert 256 % S == 0  # a power-of-two split count: each workgroup works inside one k-split
            assert nf * 64 * cols <= (96 if rows <= 8 else 112) * 1024  # activation fragments of one split fit


def test_sizes(mkmod, synth):
    cfg = synth.CONFIGS["c1"]
    h = mkmod.HostContext(cfg, max_batch=1)
    s = h.sizes
    assert s.kv_cache_per_layer == 1 * 4 * cfg.max_ctx * 128 * 2
    assert s.lin_state_per_layer == 16 * 128 * 128 * 4
    # packed weights hold every matrix once (plus 256-byte alignment and the fused a/b row padding)
    params = sum(sp.numel for sp in synth.weight_specs(cfg))
    assert params * 2 <= s.packed_weights <= params * 2 + 64 * 64 * 1024


def test_moe_schedule(mkmod, synth):
    """MoE layers: router product, expert gate/up product and expert down product (the last two are
    segmented by expert); NVFP4 expert products stream four fragments per item (nf a multiple of 16)."""
    for name in ("c4s", "c4s_bf16", "c4"):
        cfg = synth.CONFIGS[name]
        h = mkmod.HostContext(cfg, max_batch=8)
        for rows in (1, 4, 8):
            ph = h.phases(rows)
            types = [p[0] for p in ph]
            # slice configs: embed; per GQA layer q/k/v product, attention, merge, o product; router, expert
            # gate/up, expert down; hidden out
            assert types.count(2) == cfg.n_layers * 5
            assert len(ph) == 1 + cfg.n_layers * 7 + 1
            for l in range(cfg.n_layers):
                r, gu, dn = ph[1 + l * 7 + 4], ph[1 + l * 7 + 5], ph[1 + l * 7 + 6]
                assert r[2] == (cfg.n_experts + 15) // 16 * 16 and r[3] == cfg.hidden
                assert gu[3] == cfg.hidden and dn[3] == cfg.expert_ffn and dn[9] == 1  # down adds into the residual
                for p in (gu, dn):
                    S, nf = p[6], p[7]
                    assert S >= 1 and nf * S == p[3] // 32
                    assert nf % (16 if cfg.expert_format == "nvfp4" else 4) == 0


def test_expert_weight_validation(mkmod, synth):
    """Expert tensors must name a MoE layer, an existing expert and the configured format."""
    import ctypes

    cfg = synth.CONFIGS["c4s"]
    h = mkmod.HostContext(cfg, max_batch=1)
    # a host-only context rejects loads before looking at them; the resolution rules are exercised on
    # the GPU; here only the shared-expert naming of the binding is checked
    assert mkmod.weight_target("l1.s0.wg") == (1, mkmod.W_GATE, -2)
    assert mkmod.weight_target("l0.e5.wd") == (0, mkmod.W_DOWN, 5)
    assert mkmod.weight_target("l0.router") == (0, mkmod.W_ROUTER, -1)
    d = mkmod.WeightDesc()
    assert h.lib.mk_load_weights(h.ctx, ctypes.byref(d), 1, None) == 3  # MK_E_UNSUPPORTED: host-only


def test_mla_schedule(mkmod, synth):
    """Latent attention layers: fused q / latent / rotary-key product, absorbed-query product (one segment
    per head), split-KV latent attention, merge, value up-projection (one segment per head), output
    product; the chunking covers the cache and gives at most one unit per workgroup at batch 8 (C3)."""
    cfg = synth.CONFIGS["c3"]
    h = mkmod.HostContext(cfg, max_batch=8)
    ph = h.phases(8)
    l = cfg.mixers.index("mla")
    first = 1 + l * 6  # embed, then 6 phases per KDA+MoE layer before it
    types = [p[0] for p in ph[first:first + 6]]
    assert types == [2, 2, 8, 9, 2, 2]
    qkv, ak, att, mg, av, o = ph[first:first + 6]
    hq, rank = cfg.mla_heads, cfg.kv_rank
    assert qkv[2] >= hq * (cfg.nope_dim + cfg.rope_dim) + rank + cfg.rope_dim
    assert ak[2] == hq * rank and ak[3] == cfg.nope_dim and ak[6] == 1  # complete absorbed queries
    assert av[2] == hq * cfg.v_dim and av[3] == rank
    assert o[2] == cfg.hidden and o[3] == hq * cfg.v_dim and o[9] == 1
    n_chunks, chunk = att[12], att[13]
    assert chunk % 64 == 0 and n_chunks * chunk >= cfg.max_ctx > (n_chunks - 1) * chunk
    assert 8 * n_chunks * (hq // 8) <= h.sizes.n_workgroups


def test_mx_expert_configs_schedule(mkmod, synth):
    """MXFP4-shipped experts: the schedules build at both sizes, and the packed expert bytes follow the
    formats (gate|up: one byte per weight plus a bf16 per 256; down: half a byte plus one per 32)."""
    for name in ("c3ms", "c3m"):
        cfg = synth.CONFIGS[name]
        h = mkmod.HostContext(cfg, max_batch=8)
        bf = mkmod.HostContext(synth.CONFIGS[name.replace("m", "", 1) if name == "c3m" else "c3s"], max_batch=8)
        E = (cfg.n_experts + cfg.n_shared) * cfg.n_layers
        F, Hd = cfg.expert_ffn, cfg.hidden
        per_mx = 2 * F * Hd * (1 + 2 / 256) + F * Hd * (0.5 + 1 / 32)
        per_bf = 3 * F * Hd * 2
        diff = bf.sizes.packed_weights - h.sizes.packed_weights
        assert abs(diff - E * (per_bf - per_mx)) <= E * 3 * 256 + 4096, (name, diff, E * (per_bf - per_mx))


def test_delta_rule_units(mkmod, synth):
    """Gated delta rule: each unit is a block of one head's state rows; the block is the smallest of
    8, 16, 32 and 64 rows that leaves at most one unit per workgroup (a workgroup's units run one after
    another), else 64."""
    G = 256
    for name, rows, want in (("c1", 1, 8), ("c1", 4, 32), ("c1", 8, 64), ("c3", 8, 64)):
        cfg = synth.CONFIGS[name]
        h = mkmod.HostContext(cfg, max_batch=8)
        assert h.sizes.n_workgroups == G
        delta = [p for p in h.phases(rows) if p[0] == 3]
        assert len(delta) == sum(m in ("gdn", "kda") for m in cfg.mixers)
        for p in delta:
            assert p[13] == want, (name, rows, p[13])
            units = rows * cfg.lin_heads * (cfg.d_v // p[13])
            assert units <= G or p[13] == 64
