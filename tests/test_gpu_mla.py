"""GPU parity of absorbed multi-head latent attention (with its latent cache append), and of the full
C3-shaped slice (Kimi delta attention, latent attention, mixture of experts), through the C ABI against
the CPU oracle on identical seeded inputs."""
import os
import sys

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


@pytest.mark.parametrize("batch", [1, 3])
def test_mla_decode_matches_oracle(torch_gpu, oracle, synth, batch):
    cfg = synth.CONFIGS["c1s_mla"].with_batch(batch)
    W = synth.LazyWeights(cfg)
    S = synth.make_states(cfg)
    inp = synth.make_inputs(cfg)
    m = H.make_gpu(cfg, W, S, max_batch=batch)
    print(f"c1s_mla B={batch}: step", flush=True)
    out = m.decode([cfg.ctx] * batch, tokens=torch_gpu.from_numpy(inp["tokens"]).cuda())
    torch_gpu.cuda.synchronize()
    assert m.device_status() == (0, -1)
    ref = oracle.decode_step(cfg, W, S, inp, cfg.ctx)
    e = H.rel_err(out["logits"].cpu().numpy(), ref["logits"])
    print(f"c1s_mla B={batch}: logits rel err {e:.2e}")
    assert e < H.REL_TOL
    H.argmax_parity(out["argmax"].cpu().numpy(), ref, W, f"c1s_mla B={batch}")
    H.compare_states(m.get_states(batch), S, new_positions=[cfg.ctx])


def test_mla_verify_matches_oracle(torch_gpu, oracle, synth):
    from dataclasses import replace

    cfg = replace(synth.CONFIGS["c1s_mla"], verify_rows=8)
    W = synth.LazyWeights(cfg)
    S = synth.make_states(cfg)
    toks = np.array([(int(synth.make_inputs(cfg)["tokens"][0]) + 53 * j) % cfg.vocab for j in range(8)], np.int32)
    m = H.make_gpu(cfg, W, S, max_batch=1)
    print("c1s_mla verify: step", flush=True)
    out = m.verify(cfg.ctx, torch_gpu.from_numpy(toks).cuda())
    torch_gpu.cuda.synchronize()
    assert m.device_status() == (0, -1)
    ref = oracle.verify_step(cfg, W, S, toks, cfg.ctx)
    e = H.rel_err(out["logits"].cpu().numpy(), ref["logits"])
    print(f"mla verify: logits rel err {e:.2e}, accepted {ref['accepted']}")
    assert e < H.REL_TOL
    ab = out["accepted_bonus"].cpu().numpy()
    assert int(ab[0]) == ref["accepted"] and int(ab[1]) == ref["bonus"]
    H.compare_states(m.get_states(1), S, new_positions=range(cfg.ctx, cfg.ctx + 8))


@pytest.mark.parametrize("batch", [8, 2])
def test_c3_slice_matches_oracle(torch_gpu, oracle, synth, batch):
    cfg = synth.CONFIGS["c3s"].with_batch(batch)
    W = synth.LazyWeights(cfg)
    S = synth.make_states(cfg)
    inp = synth.make_inputs(cfg)
    m = H.make_gpu(cfg, W, S, max_batch=batch)
    route = m.route_outputs(batch)
    print(f"c3s B={batch}: step", flush=True)
    out = m.decode([cfg.ctx] * batch, hidden_in=torch_gpu.from_numpy(inp["hidden_in"]).cuda(), route=route)
    torch_gpu.cuda.synchronize()
    assert m.device_status() == (0, -1)
    ref = oracle.decode_step(cfg, W, S, inp, cfg.ctx)
    e = H.rel_err(out["hidden_out"].cpu().numpy(), ref["hidden_out"])
    idx, w = (t.cpu().numpy() for t in route)
    H.routes_parity(idx, w, ref, cfg, W, f"c3s B={batch}")
    print(f"c3s B={batch}: hidden rel err {e:.2e}")
    assert e < H.REL_TOL
    H.compare_states(m.get_states(batch), S, new_positions=[cfg.ctx])
