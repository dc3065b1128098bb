"""GPU parity of the mixture-of-experts FFN (router top-k, shared + routed experts, bf16 and NVFP4
weights) and of Kimi delta attention, through the C ABI against the CPU oracle on identical seeded
inputs. The slice configurations take hidden states in and give hidden states and routing out."""
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


def _slice_pair(torch_gpu, oracle, synth, name, batch, perop=False, step=0):
    cfg = synth.CONFIGS[name].with_batch(batch)
    W = synth.LazyWeights(cfg)
    S = synth.make_states(cfg)
    inp = synth.make_inputs(cfg, step=step)
    m = H.make_gpu(cfg, W, S, max_batch=batch)
    route = m.route_outputs(batch)
    print(f"{name} B={batch} perop={perop}: step", flush=True)
    out = m.decode([cfg.ctx] * batch, hidden_in=torch_gpu.from_numpy(inp["hidden_in"]).cuda(), route=route, perop=perop)
    torch_gpu.cuda.synchronize()
    assert m.device_status() == (0, -1)
    ref = oracle.decode_step(cfg, W, S, inp, cfg.ctx)
    return cfg, m, out, ref, S


def _moe_layers(cfg):
    return [l for l in range(cfg.n_layers) if cfg.ffns[l] == "moe"]


@pytest.mark.parametrize("name,batch", [("c4s_bf16", 1), ("c4s_bf16", 4), ("c4s", 1), ("c4s", 4), ("c4s", 8)])
def test_moe_slice_matches_oracle(torch_gpu, oracle, synth, name, batch):
    cfg, m, out, ref, S_ref = _slice_pair(torch_gpu, oracle, synth, name, batch)
    h = out["hidden_out"].cpu().numpy()
    e = H.rel_err(h, ref["hidden_out"])
    idx, w = (t.cpu().numpy() for t in out["route"])
    H.routes_parity(idx, w, ref, cfg, synth.LazyWeights(cfg), f"{name} B={batch}")
    print(f"{name} B={batch}: hidden rel err {e:.2e}")
    assert e < H.REL_TOL
    H.compare_states(m.get_states(batch), S_ref, new_positions=[cfg.ctx])


def test_moe_perop_matches_megakernel_bitwise(torch_gpu, oracle, synth):
    _, _, o1, _, _ = _slice_pair(torch_gpu, oracle, synth, "c4s", 4)
    _, _, o2, _, _ = _slice_pair(torch_gpu, oracle, synth, "c4s", 4, perop=True)
    assert torch_gpu.equal(o1["hidden_out"], o2["hidden_out"])
    assert torch_gpu.equal(o1["route"][0], o2["route"][0])


def test_moe_consecutive_steps(torch_gpu, oracle, synth):
    """Two steps in a row on one context: routing tables, counters and caches carry over correctly."""
    cfg = synth.CONFIGS["c4s"].with_batch(2)
    W = synth.LazyWeights(cfg)
    S = synth.make_states(cfg)
    m = H.make_gpu(cfg, W, S, max_batch=2)
    for step in range(2):
        inp = synth.make_inputs(cfg, step=step)
        pos = cfg.ctx + step
        route = m.route_outputs(2)
        out = m.decode([pos, pos], hidden_in=torch_gpu.from_numpy(inp["hidden_in"]).cuda(), route=route)
        ref = oracle.decode_step(cfg, W, S, inp, pos)
        torch_gpu.cuda.synchronize()
        e = H.rel_err(out["hidden_out"].cpu().numpy(), ref["hidden_out"])
        assert e < H.REL_TOL, (step, e)
        idx, w = (t.cpu().numpy() for t in route)
        H.routes_parity(idx, w, ref, cfg, W, f"c4s step {step}")
    H.compare_states(m.get_states(2), S)


@pytest.mark.parametrize("batch", [1, 3])
def test_kda_decode_matches_oracle(torch_gpu, oracle, synth, batch):
    cfg = synth.CONFIGS["c1s_kda"].with_batch(batch)
    W = synth.LazyWeights(cfg)
    S = synth.make_states(cfg)
    inp = synth.make_inputs(cfg)
    m = H.make_gpu(cfg, W, S, max_batch=batch)
    out = m.decode([cfg.ctx] * batch, tokens=torch_gpu.from_numpy(inp["tokens"]).cuda())
    torch_gpu.cuda.synchronize()
    assert m.device_status() == (0, -1)
    ref = oracle.decode_step(cfg, W, S, inp, cfg.ctx)
    e = H.rel_err(out["logits"].cpu().numpy(), ref["logits"])
    print(f"c1s_kda B={batch}: logits rel err {e:.2e}")
    assert e < H.REL_TOL
    H.argmax_parity(out["argmax"].cpu().numpy(), ref, W, f"c1s_kda B={batch}")
    H.compare_states(m.get_states(batch), S, new_positions=[cfg.ctx])


def test_kda_verify_matches_oracle(torch_gpu, oracle, synth):
    from dataclasses import replace

    cfg = replace(synth.CONFIGS["c1s_kda"], verify_rows=8)
    W = synth.LazyWeights(cfg)
    S = synth.make_states(cfg)
    toks = np.array([(int(synth.make_inputs(cfg)["tokens"][0]) + 97 * j) % cfg.vocab for j in range(8)], np.int32)
    m = H.make_gpu(cfg, W, S, max_batch=1)
    out = m.verify(cfg.ctx, torch_gpu.from_numpy(toks).cuda())
    torch_gpu.cuda.synchronize()
    assert m.device_status() == (0, -1)
    ref = oracle.verify_step(cfg, W, S, toks, cfg.ctx)
    e = H.rel_err(out["logits"].cpu().numpy(), ref["logits"])
    print(f"kda verify: logits rel err {e:.2e}, accepted {ref['accepted']}")
    assert e < H.REL_TOL
    ab = out["accepted_bonus"].cpu().numpy()
    assert int(ab[0]) == ref["accepted"] and int(ab[1]) == ref["bonus"]
    H.compare_states(m.get_states(1), S, new_positions=range(cfg.ctx, cfg.ctx + 8))
