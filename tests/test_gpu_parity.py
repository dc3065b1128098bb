"""GPU parity: the HIP megakernel (through the C ABI) against the CPU oracle on identical seeded inputs.

Sizes are ones the oracle finishes in seconds while still spanning many 16-row tiles, several k-splits,
split-KV chunks and ragged tails (the *s configurations), plus the exact tiny dense configuration."""
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


def _decode_pair(torch_gpu, oracle, synth, name, batch, perop=False):
    cfg = synth.CONFIGS[name].with_batch(batch)
    W = synth.LazyWeights(cfg)
    S = synth.make_states(cfg)
    inp = synth.make_inputs(cfg)
    m = H.make_gpu(cfg, W, S, max_batch=batch)
    pos = [cfg.ctx] * batch
    if cfg.vocab:
        out = m.decode(pos, tokens=torch_gpu.from_numpy(inp["tokens"]).cuda(), perop=perop)
    else:
        out = m.decode(pos, hidden_in=torch_gpu.from_numpy(inp["hidden_in"]).cuda(), perop=perop)
    torch_gpu.cuda.synchronize()
    assert m.device_status() == (0, -1)
    ref = oracle.decode_step(cfg, W, S, inp, cfg.ctx)
    return cfg, m, out, ref, S


@pytest.mark.parametrize("name,batch", [("c0", 1), ("c1s", 1), ("c1s", 3), ("c1s", 8)])
def test_decode_matches_oracle(torch_gpu, oracle, synth, name, batch):
    cfg, m, out, ref, S_ref = _decode_pair(torch_gpu, oracle, synth, name, batch)
    logits = out["logits"].cpu().numpy()
    e = H.rel_err(logits, ref["logits"])
    print(f"{name} B={batch}: logits rel err {e:.2e}")
    assert e < H.REL_TOL
    H.argmax_parity(out["argmax"].cpu().numpy(), ref, synth.LazyWeights(cfg), f"{name} B={batch}")
    H.compare_states(m.get_states(batch), S_ref, new_positions=[cfg.ctx])


def test_perop_baseline_matches_megakernel_bitwise(torch_gpu, oracle, synth):
    _, _, out1, _, _ = _decode_pair(torch_gpu, oracle, synth, "c1s", 2)
    _, _, out2, _, _ = _decode_pair(torch_gpu, oracle, synth, "c1s", 2, perop=True)
    assert torch_gpu.equal(out1["logits"], out2["logits"])


def test_repeat_is_deterministic(torch_gpu, synth):
    cfg = synth.CONFIGS["c1s"]
    W = synth.LazyWeights(cfg)
    S = synth.make_states(cfg)
    inp = synth.make_inputs(cfg)
    toks = torch_gpu.from_numpy(inp["tokens"]).cuda()
    outs = []
    for _ in range(2):
        m = H.make_gpu(cfg, W, S)
        outs.append(m.decode([cfg.ctx], tokens=toks)["logits"].clone())
        torch_gpu.cuda.synchronize()
        m.close()
    assert torch_gpu.equal(outs[0], outs[1])


def test_consecutive_steps_track_oracle(torch_gpu, oracle, synth):
    """Three decode steps in a row (positions advance, caches and states carry over)."""
    cfg = synth.CONFIGS["c1s"].with_batch(2)
    W = synth.LazyWeights(cfg)
    S = synth.make_states(cfg)
    m = H.make_gpu(cfg, W, S, max_batch=2)
    for step in range(3):
        inp = synth.make_inputs(cfg, step=step)
        pos = cfg.ctx + step
        out = m.decode([pos, pos], tokens=torch_gpu.from_numpy(inp["tokens"]).cuda())
        ref = oracle.decode_step(cfg, W, S, inp, pos)
        torch_gpu.cuda.synchronize()
        e = H.rel_err(out["logits"].cpu().numpy(), ref["logits"])
        assert e < H.REL_TOL, (step, e)
    H.compare_states(m.get_states(2), S)


def test_verify_matches_oracle(torch_gpu, oracle, synth):
    cfg = synth.CONFIGS["c2s"]
    W = synth.LazyWeights(cfg)
    S = synth.make_states(cfg)
    from dataclasses import replace

    # drafts: greedy continuation (from the oracle) with one wrong token, so 0 < a < 7
    cfg_d = replace(cfg, verify_rows=0)
    Sd = oracle.copy_states(S)
    toks = [int(synth.make_inputs(cfg)["tokens"][0])]
    for j in range(7):
        toks.append(int(oracle.decode_step(cfg_d, W, Sd, {"tokens": np.array(toks[j:j + 1], np.int32)},
                                           cfg.ctx + j)["argmax"][0]))
    toks[5] = (toks[5] + 11) % cfg.vocab
    toks = np.array(toks, np.int32)
    m = H.make_gpu(cfg, W, S, max_batch=1)
    out = m.verify(cfg.ctx, torch_gpu.from_numpy(toks).cuda())
    torch_gpu.cuda.synchronize()
    assert m.device_status() == (0, -1)
    ref = oracle.verify_step(cfg, W, S, toks, cfg.ctx)
    e = H.rel_err(out["logits"].cpu().numpy(), ref["logits"])
    print(f"verify: logits rel err {e:.2e}, accepted {ref['accepted']}")
    assert e < H.REL_TOL
    ab = out["accepted_bonus"].cpu().numpy()
    assert int(ab[0]) == ref["accepted"] == 4
    assert int(ab[1]) == ref["bonus"]
    H.compare_states(m.get_states(1), S, new_positions=range(cfg.ctx, cfg.ctx + 8))
