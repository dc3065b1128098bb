"""GPU parity at the full dimensions of the hybrid 27B-class stack (hidden 5120, SwiGLU 17408, vocab
151936, 4096-token KV cache, 16 GDN heads, 24/4 GQA heads) in the launch configuration the benchmark
times, on the first four layers (one 3 GDN : 1 GQA group: every phase kind and every matrix shape of
the 64-layer stack). The weights and caches are generated in device memory by the device generator and
on the host by the host generator (bit-identical definitions)."""
import os
import sys
from dataclasses import replace

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import harness as H  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch


def _trunc(cfg, layers=4):
    return replace(cfg, n_layers=layers, mixers=cfg.mixers[:layers], ffns=cfg.ffns[:layers])


def _gpu_from_device_generator(torch_gpu, cfg, max_batch):
    from persistent_megakernel_mk_amd import mk, synth

    m = mk.Megakernel(cfg, device=0, max_batch=max_batch)
    for spec in synth.weight_specs(cfg):
        t = synth.generate_gpu(spec, cfg.seed)
        layer, kind, expert = mk.weight_target(spec.name)
        d = mk.WeightDesc()
        d.layer, d.kind, d.expert, d.dtype = layer, kind, expert, 0
        d.rows, d.cols = (1, spec.shape[0]) if len(spec.shape) == 1 else spec.shape
        d.data = t.data_ptr()
        mk.check(m.lib.mk_load_weights(m.ctx, (mk.WeightDesc * 1)(d), 1, torch_gpu.cuda.current_stream().cuda_stream))
        torch_gpu.cuda.synchronize()
    return m


def test_device_generator_matches_host_generator(torch_gpu, synth):
    cfg = synth.CONFIGS["c1s"]
    for spec in synth.weight_specs(cfg)[:6] + synth.state_specs(cfg):
        g = synth.generate_gpu(spec, cfg.seed)
        h = synth.generate(spec, cfg.seed)
        gn = g.view(torch_gpu.int16).cpu().numpy().view(np.uint16) if spec.kind == "bf16" else g.cpu().numpy()
        assert np.array_equal(gn, h), spec.name


@pytest.mark.timeout(600)
@pytest.mark.parametrize("batch", [1, 8])
def test_full_dims_decode_matches_oracle(torch_gpu, oracle, synth, batch):
    cfg = _trunc(synth.CONFIGS["c1"]).with_batch(batch)
    m = _gpu_from_device_generator(torch_gpu, cfg, batch)
    S = synth.make_states(cfg)
    m.set_states(S)
    inp = synth.make_inputs(cfg)
    out = m.decode([cfg.ctx] * batch, tokens=torch_gpu.from_numpy(inp["tokens"]).cuda())
    torch_gpu.cuda.synchronize()
    assert m.device_status() == (0, -1)
    W = synth.LazyWeights(cfg)
    ref = oracle.decode_step(cfg, W, S, inp, cfg.ctx)
    e = H.rel_err(out["logits"].cpu().numpy(), ref["logits"])
    print(f"full dims B={batch}: logits rel err {e:.2e}")
    assert e < H.REL_TOL
    H.argmax_parity(out["argmax"].cpu().numpy(), ref, W, f"full dims B={batch}")
    H.compare_states(m.get_states(batch), S, new_positions=[cfg.ctx])


@pytest.mark.timeout(600)
def test_full_dims_verify_matches_oracle(torch_gpu, oracle, synth):
    cfg = _trunc(synth.CONFIGS["c2"])
    m = _gpu_from_device_generator(torch_gpu, cfg, 1)
    S = synth.make_states(cfg)
    m.set_states(S)
    rng = np.random.default_rng(3)
    toks = rng.integers(0, cfg.vocab, 8).astype(np.int32)
    out = m.verify(cfg.ctx, torch_gpu.from_numpy(toks).cuda())
    torch_gpu.cuda.synchronize()
    assert m.device_status() == (0, -1)
    W = synth.LazyWeights(cfg)
    ref = oracle.verify_step(cfg, W, S, toks, cfg.ctx)
    e = H.rel_err(out["logits"].cpu().numpy(), ref["logits"])
    print(f"full dims verify: logits rel err {e:.2e}")
    assert e < H.REL_TOL
    ab = out["accepted_bonus"].cpu().numpy()
    assert int(ab[0]) == ref["accepted"] and int(ab[1]) == ref["bonus"]
    H.compare_states(m.get_states(1), S, new_positions=range(cfg.ctx, cfg.ctx + 8))
