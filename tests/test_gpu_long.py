"""Longer contexts: split-KV attention (grouped-query and absorbed latent) over caches far beyond the
4096-position workloads, against the oracle. The chunking adapts to the cache length (more and longer
chunks, one log-sum-exp merge over all of them)."""
import os
import sys
from dataclasses import replace

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


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,ctx,batch", [("c1s", 12000, 2), ("c1s_mla", 12000, 2), ("c1s", 32768, 1)])
def test_long_context_decode_matches_oracle(torch_gpu, oracle, synth, name, ctx, batch):
    cfg = replace(synth.CONFIGS[name], ctx=ctx).with_batch(batch)
    W = synth.LazyWeights(cfg)
    S = synth.make_states(cfg)
    inp = synth.make_inputs(cfg)
    m = H.make_gpu(cfg, W, S, max_batch=batch)
    ph = [p for p in m.phases(batch) if p[0] in (4, 8)]  # attention phases: their split-KV geometry
    print(f"{name} ctx={ctx} B={batch}: split-KV (chunks, chunk length) {sorted({(p[12], p[13]) for p in ph})}", flush=True)
    pos = [ctx - 3] + [ctx] * (batch - 1)
    out = m.decode(pos, tokens=torch_gpu.from_numpy(inp["tokens"]).cuda())
    torch_gpu.cuda.synchronize()
    assert m.device_status() == (0, -1)
    ref = oracle.decode_step(cfg, W, S, inp, pos)
    e = H.rel_err(out["logits"].cpu().numpy(), ref["logits"])
    print(f"{name} ctx={ctx} B={batch}: logits rel err {e:.2e}", flush=True)
    assert e < H.REL_TOL
    H.argmax_parity(out["argmax"].cpu().numpy(), ref, W, f"{name} ctx={ctx}")
    H.compare_states(m.get_states(batch), S)
