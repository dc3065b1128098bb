"""Experts shipped in MXFP4 (E2M1 with an E8M0 scale per 32): the library re-encodes gate/up into FP8
E4M3 with a bf16 scale per 256 at load time, checking bit for bit that the new encoding decodes to the
same values and refusing the tensor otherwise; down stays MXFP4 (page "Kimi K3's TPU megakernel: 92
layers in one Pallas call, and what 709 tokens a second measures", section "How it maps onto a TPU v7").
Through the C ABI against the oracle, which re-encodes with its own definition."""
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


@pytest.mark.parametrize("batch", [1, 4, 8])
def test_mx_slice_matches_oracle(torch_gpu, oracle, synth, batch):
    cfg = synth.CONFIGS["c3ms"].with_batch(batch)
    W = synth.LazyWeights(cfg)
    S = synth.make_states(cfg)
    inp = synth.make_inputs(cfg)
    m = H.make_gpu(cfg, W, S, max_batch=batch)
    route = m.route_outputs(batch)
    print(f"c3ms B={batch}: step", flush=True)
    out = m.decode([cfg.ctx] * batch, hidden_in=torch_gpu.from_numpy(inp["hidden_in"]).cuda(), route=route)
    torch_gpu.cuda.synchronize()
    assert m.device_status() == (0, -1)
    ref = oracle.decode_step(cfg, W, S, inp, cfg.ctx)
    e = H.rel_err(out["hidden_out"].cpu().numpy(), ref["hidden_out"])
    idx, w = (t.cpu().numpy() for t in route)
    H.routes_parity(idx, w, ref, cfg, W, f"c3ms B={batch}")
    print(f"c3ms B={batch}: hidden rel err {e:.2e}", flush=True)
    assert e < H.REL_TOL
    H.compare_states(m.get_states(batch), S, new_positions=[cfg.ctx])


def test_inexact_reencode_is_refused(torch_gpu, oracle, synth):
    """A gate matrix with a 256-block whose nonzero 32-blocks span 15 E8M0 exponents has no lossless FP8
    encoding: the loader returns MK_E_INEXACT, the step refuses to run until the matrix is loaded again,
    and after a good load the step matches the oracle."""
    from persistent_megakernel_mk_amd import mk

    cfg = synth.CONFIGS["c3ms"].with_batch(2)
    Wl = synth.LazyWeights(cfg)
    W = {n: Wl[n] for n in Wl.keys()}
    S = synth.make_states(cfg)
    good = W["l0.e3.wg"]
    bad = synth.MXFP4Tensor(good.codes.copy(), good.scales.copy())
    bad.scales[5, 0] = 127
    bad.scales[5, 7] = 127 - 15
    bad.codes[5, 0] = (bad.codes[5, 0] & 0xF0) | 7       # 6 * 2^0 in the first 32-block
    bad.codes[5, 7 * 16] = (bad.codes[5, 7 * 16] & 0xF0) | 1  # 0.5 * 2^-15 in the last one
    with pytest.raises(ValueError):
        oracle.fp8_reencode(bad)  # the oracle's own definition refuses it too
    m = mk.Megakernel(cfg, device=0, max_batch=2)
    m.load_weights(W)
    m.set_states(S)
    with pytest.raises(mk.MKError) as ei:
        m.load_weights({"l0.e3.wg": bad})
    assert ei.value.status == 8  # MK_E_INEXACT
    inp = synth.make_inputs(cfg)
    hid = torch_gpu.from_numpy(inp["hidden_in"]).cuda()
    with pytest.raises(mk.MKError) as ei:
        m.decode([cfg.ctx] * 2, hidden_in=hid)
    assert ei.value.status == 7  # MK_E_STATE: that expert's gate is not loaded
    m.load_weights({"l0.e3.wg": good})
    out = m.decode([cfg.ctx] * 2, hidden_in=hid)
    torch_gpu.cuda.synchronize()
    assert m.device_status() == (0, -1)
    ref = oracle.decode_step(cfg, W, S, inp, cfg.ctx)
    assert H.rel_err(out["hidden_out"].cpu().numpy(), ref["hidden_out"]) < H.REL_TOL
