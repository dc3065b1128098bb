"""The on-device decode loop (mk_decode_loop: n greedy decode steps in one persistent launch, each step's
argmax re-embedded by the kernel) against the oracle run one step at a time with its own argmax fed back,
and against the same steps as separate launches."""
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


@pytest.mark.parametrize("name,batch,n", [("c1s", 2, 4), ("c1s", 1, 8), ("c1s_mla", 2, 3), ("c1s_kda", 3, 3),
                                          ("c0", 1, 8)])
def test_decode_loop_matches_oracle_steps(torch_gpu, oracle, synth, name, batch, n):
    cfg = synth.CONFIGS[name].with_batch(batch)
    W = synth.LazyWeights(cfg)
    S = synth.make_states(cfg)
    inp = synth.make_inputs(cfg)
    m = H.make_gpu(cfg, W, S, max_batch=batch)
    pos = [cfg.ctx] * batch
    print(f"{name} B={batch}: loop of {n} steps", flush=True)
    out = m.decode_loop(pos, torch_gpu.from_numpy(inp["tokens"]).cuda(), n)
    torch_gpu.cuda.synchronize()
    assert m.device_status() == (0, -1)
    emitted = out["tokens"].cpu().numpy()
    toks = inp["tokens"].copy()
    for s in range(n):
        ref = oracle.decode_step(cfg, W, S, {"tokens": toks}, [p + s for p in pos])
        exact, ties = H.argmax_parity(emitted[s], ref, W, f"{name} loop step {s}")
        assert ties == 0, "a tie within rounding would let the sequences diverge"
        toks = ref["argmax"].astype(np.int32)
    e = H.rel_err(out["logits"].cpu().numpy(), ref["logits"])
    print(f"{name} B={batch}: last-step logits rel err {e:.2e}; emitted {emitted.T.tolist()}")
    assert e < H.REL_TOL
    assert np.array_equal(out["argmax"].cpu().numpy(), emitted[-1])
    H.compare_states(m.get_states(batch), S, new_positions=range(cfg.ctx, cfg.ctx + n))


def test_loop_equals_single_step_launches_bitwise(torch_gpu, synth):
    """One context runs loop(3), one ordinary step, loop(2); another runs six ordinary steps, each fed the
    previous step's argmax on the device. Same arithmetic in the same order: identical tokens, logits
    and states (this also checks the grid-barrier accounting across launches of different lengths)."""
    cfg = synth.CONFIGS["c1s"].with_batch(2)
    W = synth.LazyWeights(cfg)
    S = synth.make_states(cfg)
    inp = synth.make_inputs(cfg)
    a = H.make_gpu(cfg, W, S, max_batch=2)
    b = H.make_gpu(cfg, W, S, max_batch=2)
    t0 = torch_gpu.from_numpy(inp["tokens"]).cuda()
    p0 = cfg.ctx
    o1 = a.decode_loop([p0, p0], t0, 3)
    mid = a.decode([p0 + 3, p0 + 3], tokens=o1["tokens"][2].clone())
    o2 = a.decode_loop([p0 + 4, p0 + 4], mid["argmax"].clone(), 2)
    seq_a = torch_gpu.cat([o1["tokens"], mid["argmax"][None], o2["tokens"]]).cpu().numpy()
    toks, seq_b = t0, []
    for s in range(6):
        r = b.decode([p0 + s, p0 + s], tokens=toks)
        toks = r["argmax"].clone()
        seq_b.append(toks.cpu().numpy())
    torch_gpu.cuda.synchronize()
    assert a.device_status() == (0, -1) and b.device_status() == (0, -1)
    print(f"loop/step mix {seq_a.T.tolist()} vs steps {np.array(seq_b).T.tolist()}")
    assert np.array_equal(seq_a, np.array(seq_b))
    assert torch_gpu.equal(o2["logits"], r["logits"])
    sa, sb = a.get_states(2), b.get_states(2)
    for k in sa:
        assert np.array_equal(sa[k], sb[k]), k
