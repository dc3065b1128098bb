"""GPU edge cases against the CPU oracle: exact ties (the lowest index wins, for the LM-head argmax and
for the router's top-k), sequences at different positions in one decode step, a verify block whose
seven drafts are all accepted, and switching between the persistent step and the one-launch-per-phase
baseline on one context."""
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


def _weights(synth, cfg):
    Wl = synth.LazyWeights(cfg)
    return {n: Wl[n] for n in Wl.keys()}


def test_lm_head_exact_tie_takes_lowest_index(torch_gpu, oracle, synth):
    """Row j < a of the LM head is made a copy of the row of the oracle's argmax a: both logits are the
    same sum of the same products, so they are equal, and the first maximum (j) must win on both sides."""
    cfg = synth.CONFIGS["c1s"].with_batch(3)
    W = _weights(synth, cfg)
    S0 = synth.make_states(cfg)
    inp = synth.make_inputs(cfg)
    a = int(oracle.decode_step(cfg, W, oracle.copy_states(S0), inp, cfg.ctx)["argmax"][0])
    j = a // 2 if a >= 32 else a + 37  # another 16-row tile, another workgroup's range
    W["lm_head"] = W["lm_head"].copy()
    W["lm_head"][j] = W["lm_head"][a]
    S = oracle.copy_states(S0)
    m = H.make_gpu(cfg, W, S0, max_batch=3)
    out = m.decode([cfg.ctx] * 3, tokens=torch_gpu.from_numpy(inp["tokens"]).cuda())
    torch_gpu.cuda.synchronize()
    assert m.device_status() == (0, -1)
    ref = oracle.decode_step(cfg, W, S, inp, cfg.ctx)
    logits = out["logits"].cpu().numpy()
    print(f"tie rows {min(a, j)} and {max(a, j)}: gpu logits {logits[0, a]!r} {logits[0, j]!r}")
    assert ref["logits"][0, a] == ref["logits"][0, j]
    assert logits[0, a] == logits[0, j]  # identical rows give identical sums on the GPU too
    assert int(ref["argmax"][0]) == min(a, j)
    assert int(out["argmax"][0]) == min(a, j)
    H.argmax_parity(out["argmax"].cpu().numpy()[1:], {"logits": ref["logits"][1:], "final_y": ref["final_y"][1:]}, W,
                    "c1s tie, other rows")


@pytest.mark.parametrize("name", ["c4s", "c3s"])
def test_router_exact_tie_takes_lowest_index(torch_gpu, oracle, synth, name):
    """In layer 0 a router row is made a copy of the row of the expert the oracle ranks first for token
    0: the two logits are equal, both experts are selected, the lower index first, with equal gates."""
    cfg = synth.CONFIGS[name].with_batch(4)
    W = _weights(synth, cfg)
    S0 = synth.make_states(cfg)
    inp = synth.make_inputs(cfg)
    first = int(oracle.decode_step(cfg, W, oracle.copy_states(S0), inp, cfg.ctx)["routes"][0][0][0, 0])
    E = cfg.n_experts
    twin = (first + E // 2 + 1) % E
    W["l0.router"] = W["l0.router"].copy()
    W["l0.router"][twin] = W["l0.router"][first]
    lo, hi = min(first, twin), max(first, twin)
    m = H.make_gpu(cfg, W, S0, max_batch=4)
    route = m.route_outputs(4)
    out = m.decode([cfg.ctx] * 4, hidden_in=torch_gpu.from_numpy(inp["hidden_in"]).cuda(), route=route)
    torch_gpu.cuda.synchronize()
    assert m.device_status() == (0, -1)
    ref = oracle.decode_step(cfg, W, oracle.copy_states(S0), inp, cfg.ctx)
    idx, gw = (t.cpu().numpy() for t in route)
    ridx, rgw = ref["routes"][0][0], ref["routes"][0][1]
    assert list(ridx[0, :2]) == [lo, hi]
    print(f"{name}: tied experts {lo}, {hi}; gpu token 0 ranks {idx[0, 0].tolist()}")
    for b in range(4):
        for t in range(cfg.top_k):
            if ridx[b, t] in (lo, hi):
                assert idx[0, b, t] == ridx[b, t], (b, t, idx[0, b].tolist(), ridx[b].tolist())
    assert gw[0, 0, 0] == gw[0, 0, 1]
    H.routes_parity(idx, gw, ref, cfg, W, f"{name} tie", max_tie_frac=None)  # the planted tie adds ties


def test_decode_at_unequal_positions(torch_gpu, oracle, synth):
    """Three sequences at positions before, at and after the end of their cached prefix: each appends
    at its own position and attends to its own 0..p."""
    cfg = synth.CONFIGS["c1s"].with_batch(3)
    W = synth.LazyWeights(cfg)
    S = synth.make_states(cfg)
    inp = synth.make_inputs(cfg)
    pos = [cfg.ctx - 117, cfg.ctx, cfg.ctx + 5]
    m = H.make_gpu(cfg, W, S, max_batch=3)
    out = m.decode(pos, tokens=torch_gpu.from_numpy(inp["tokens"]).cuda())
    torch_gpu.cuda.synchronize()
    assert m.device_status() == (0, -1)
    ref = oracle.decode_step(cfg, W, S, inp, pos)
    e = H.rel_err(out["logits"].cpu().numpy(), ref["logits"])
    print(f"unequal positions {pos}: logits rel err {e:.2e}")
    assert e < H.REL_TOL
    H.argmax_parity(out["argmax"].cpu().numpy(), ref, W, "unequal positions")
    G = m.get_states(3)
    H.compare_states(G, S)
    for l in range(cfg.n_layers):  # every row other than a sequence's own new row is unchanged
        if cfg.mixers[l] != "gqa":
            continue
        for name in (f"l{l}.kcache", f"l{l}.vcache"):
            for b, p in enumerate(pos):
                mask = np.ones(G[name].shape[2], bool)
                mask[p] = False
                assert np.array_equal(G[name][b][:, mask], S[name][b][:, mask]), (name, b)


def test_verify_with_all_drafts_accepted(torch_gpu, oracle, synth):
    """Drafts equal to the oracle's greedy continuation: a = 7, the bonus token is the argmax of the
    last row, and every linear state is committed to its value after the last row."""
    cfg_v = synth.CONFIGS["c2s"]
    cfg_d = replace(cfg_v, verify_rows=0)
    W = synth.LazyWeights(cfg_v)
    S0 = synth.make_states(cfg_v)
    pos = cfg_v.ctx
    toks = [int(synth.make_inputs(cfg_v)["tokens"][0])]
    Sd = oracle.copy_states(S0)
    for j in range(7):
        toks.append(int(oracle.decode_step(cfg_d, W, Sd, {"tokens": np.array(toks[j:j + 1], np.int32)},
                                           pos + j)["argmax"][0]))
    toks = np.array(toks, np.int32)
    S = oracle.copy_states(S0)
    ref = oracle.verify_step(cfg_v, W, S, toks, pos)
    assert ref["accepted"] == 7
    m = H.make_gpu(cfg_v, W, S0, max_batch=1)
    out = m.verify(pos, torch_gpu.from_numpy(toks).cuda())
    torch_gpu.cuda.synchronize()
    assert m.device_status() == (0, -1)
    e = H.rel_err(out["logits"].cpu().numpy(), ref["logits"])
    ab = out["accepted_bonus"].cpu().numpy()
    print(f"all-accepted verify: logits rel err {e:.2e}, gpu a = {int(ab[0])}, bonus {int(ab[1])}")
    assert e < H.REL_TOL
    H.argmax_parity(out["argmax"].cpu().numpy(), ref, W, "all-accepted verify")
    assert int(ab[0]) == 7 and int(ab[1]) == ref["bonus"]
    H.compare_states(m.get_states(1), S, new_positions=range(pos, pos + 8))


def test_persistent_and_per_op_steps_interleave_on_one_context(torch_gpu, oracle, synth):
    """Steps 0 and 2 persistent, step 1 one launch per phase, on one context: the barrier counters and
    the count of barriers already passed carry over, so every step equals the all-persistent sequence on a second context bit for
    bit and tracks the oracle."""
    cfg = synth.CONFIGS["c1s"].with_batch(2)
    W = synth.LazyWeights(cfg)
    S = synth.make_states(cfg)
    mixed = H.make_gpu(cfg, W, S, max_batch=2)
    plain = H.make_gpu(cfg, W, S, max_batch=2)
    for step, perop in enumerate((False, True, False)):
        inp = synth.make_inputs(cfg, step=step)
        pos = [cfg.ctx + step] * 2
        t = torch_gpu.from_numpy(inp["tokens"]).cuda()
        a = mixed.decode(pos, tokens=t, perop=perop)
        b = plain.decode(pos, tokens=t)
        ref = oracle.decode_step(cfg, W, S, inp, pos)
        torch_gpu.cuda.synchronize()
        assert mixed.device_status() == (0, -1) and plain.device_status() == (0, -1)
        assert torch_gpu.equal(a["logits"], b["logits"]), step
        e = H.rel_err(a["logits"].cpu().numpy(), ref["logits"])
        print(f"step {step} perop={perop}: logits rel err {e:.2e}")
        assert e < H.REL_TOL
    H.compare_states(mixed.get_states(2), S)


def test_per_op_graph_replays_match_eager_launches(torch_gpu, oracle, synth):
    """The per-op baseline replayed as a HIP graph: three replays of one graph (same position, tokens and
    buffers; the linear states advance each time), with unrelated eager GPU work and synchronisations
    between them, each bit-identical to the eager per-op launches on a second context, and the first
    one within tolerance of the oracle."""
    cfg = synth.CONFIGS["c1s"].with_batch(2)
    W = synth.LazyWeights(cfg)
    S = synth.make_states(cfg)
    eager = H.make_gpu(cfg, W, S, max_batch=2)
    graph = H.make_gpu(cfg, W, S, max_batch=2)
    inp = synth.make_inputs(cfg)
    t = torch_gpu.from_numpy(inp["tokens"]).cuda()
    pos = [cfg.ctx] * 2
    out_e, out_g = eager.outputs(2), graph.outputs(2)
    ref = oracle.decode_step(cfg, W, S, inp, pos)
    junk = torch_gpu.randn(1 << 20, device="cuda")
    for rep in range(3):
        a = eager.decode(pos, tokens=t, out=out_e, perop=True)
        b = graph.decode(pos, tokens=t, out=out_g, perop=True, graph=True)
        junk = (junk * 1.0001 + 1.0).sin()  # eager work between replays
        torch_gpu.cuda.synchronize()
        assert eager.device_status() == (0, -1) and graph.device_status() == (0, -1)
        assert torch_gpu.equal(a["logits"], b["logits"]), rep
        assert torch_gpu.equal(a["argmax"], b["argmax"]), rep
        if rep == 0:
            e = H.rel_err(b["logits"].cpu().numpy(), ref["logits"])
            print(f"graph replay 0: logits rel err {e:.2e}")
            assert e < H.REL_TOL
    sa, sb = eager.get_states(2), graph.get_states(2)
    for k in sa:
        assert np.array_equal(sa[k], sb[k]), k
