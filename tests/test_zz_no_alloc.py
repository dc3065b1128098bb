"""mk_decode_step_noalloc (the decode step on library-held working memory, for callers that cannot
allocate) against mk_decode_step on the same context state: outputs and every state update must be
bit-identical, on two calls in a row, the second with a smaller batch (so the second call reuses the
array the first one left behind)."""
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


# a dense GQA/GDN stack with a vocabulary, latent attention with KDA and bf16 experts, NVFP4 experts
@pytest.mark.parametrize("name", ["c1s", "c3s", "c4s"])
def test_noalloc_matches_decode_step(torch_gpu, synth, name):
    torch = torch_gpu
    cfg = synth.CONFIGS[name].with_batch(8)
    W = synth.LazyWeights(cfg)
    S = synth.make_states(cfg)
    ref = H.make_gpu(cfg, W, S, max_batch=8)
    new = H.make_gpu(cfg, W, S, max_batch=8)
    for step, B in enumerate((8, 3)):
        print(f"noalloc {name} step {step} batch {B}", flush=True)
        inp = synth.make_inputs(cfg.with_batch(B), step=step)
        pos = [cfg.ctx + step] * B
        key = "tokens" if cfg.vocab else "hidden_in"
        x = torch.from_numpy(inp[key]).cuda()
        a = ref.decode(pos, **{key: x})
        b = new.decode(pos, noalloc=True, **{key: x})
        torch.cuda.synchronize()
        assert ref.device_status() == (0, -1)
        assert new.device_status() == (0, -1)
        if cfg.vocab:
            assert torch.equal(a["logits"], b["logits"]), step
            assert torch.equal(a["argmax"], b["argmax"]), step
        else:
            assert torch.equal(a["hidden_out"], b["hidden_out"]), step
    sa, sb = ref.get_states(8), new.get_states(8)
    for k in sa:
        assert np.array_equal(sa[k], sb[k]), k
    ref.close()
    new.close()
