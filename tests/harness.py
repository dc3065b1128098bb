"""Shared test harness: builds an oracle run and a GPU run of the same seeded workload and compares them.

Inputs come from the seeded generator (persistent_megakernel_mk_amd.synth), identical for both sides.
The oracle (oracle/) and the HIP path (libmk.so through persistent_megakernel_mk_amd.mk) share nothing
else."""
from __future__ import annotations

import numpy as np

# Parity bar: per tensor, max |gpu - oracle| / max |oracle|. The contract is 2e-2; both sides
# accumulate in fp32 and the GPU keeps 16 significant bits of every activation entering a matrix
# product (bf16 high + low halves), so the expected difference is ~1e-5 and the tests use 2e-3.
REL_TOL = 2e-3
CONTRACT_TOL = 2e-2


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    den = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(gpu.astype(np.float64) - ref.astype(np.float64)))) / max(den, 1e-30)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def argmax_margin(logits_row: np.ndarray) -> float:
    s = np.sort(logits_row.astype(np.float64))
    return float(s[-1] - s[-2])


def assert_argmax(gpu_am, ref_logits, tol_abs):
    """Identical argmax wherever the oracle's top-1/top-2 margin exceeds the rounding bound; below it the
    decision is a tie within rounding and the GPU's pick must be one of the tied candidates."""
    for b, row in enumerate(ref_logits):
        ref = int(np.argmax(row))
        if argmax_margin(row) > tol_abs:
            assert int(gpu_am[b]) == ref, (b, int(gpu_am[b]), ref)
        else:
            assert row[int(gpu_am[b])] >= row[ref] - tol_abs


def make_gpu(cfg, W, S, max_batch=None, device=0):
    from persistent_megakernel_mk_amd import mk

    m = mk.Megakernel(cfg, device=device, max_batch=max_batch)
    m.load_weights(W)
    m.set_states(S)
    return m


def compare_states(gpu_S, ref_S, new_positions=None):
    """Caches: rows other than this step's new rows bit-identical; new rows (bf16 roundings of fp32
    projections that differ from the oracle's by summation order) within one bf16 ulp plus the
    projection tolerance relative to the row's largest entry. Linear states: fp32, relative tolerance."""
    for name, ref in ref_S.items():
        g = gpu_S[name]
        if name.endswith("lstate"):
            e = rel_err(g, ref)
            assert e < REL_TOL, (name, e)
            continue
        gf, rf = bf16_to_f32(g).astype(np.float64), bf16_to_f32(ref).astype(np.float64)
        rowmax = np.max(np.abs(rf), axis=-1, keepdims=True)
        bound = np.maximum(np.abs(rf), np.abs(gf)) * 2.0 ** -7 + REL_TOL * rowmax
        diff = np.abs(gf - rf)
        assert np.all(diff <= bound), (name, float(diff.max()))
        if new_positions is not None:
            pax = 1 if name.endswith("latent") else 2  # position axis: latent [B][pos][D], K/V [B][heads][pos][d]
            mask = np.ones(g.shape[pax], bool)
            mask[list(new_positions)] = False
            idx = (slice(None),) * pax + (mask,)
            assert np.array_equal(g[idx], ref[idx]), name


def assert_routes(gpu_idx, gpu_w, route_log, moe_layers, tol_rel=REL_TOL):
    """Routing parity per MoE layer and row: the selected experts and their order are identical wherever
    the oracle's logit gaps around them exceed the rounding bound (8 * tol_rel * max |z|); a selection
    inside a gap below the bound is a tie within rounding and only has to pick among the tied experts.
    Gates (normalised sigmoids) agree to tol_rel. Returns the number of decisions checked exactly."""
    exact = 0
    for i, l in enumerate(moe_layers):
        idxs, gws, z = route_log[l]
        tol = 8 * tol_rel * float(np.max(np.abs(z)))
        for b in range(idxs.shape[0]):
            zs = z[b].astype(np.float64)
            order = np.argsort(-zs, kind="stable")
            K = idxs.shape[1]
            for t in range(K):
                gap_above = zs[order[t - 1]] - zs[order[t]] if t > 0 else np.inf
                gap_below = zs[order[t]] - zs[order[t + 1]] if t + 1 < len(zs) else np.inf
                if min(gap_above, gap_below) > tol:
                    assert int(gpu_idx[i, b, t]) == int(idxs[b, t]), (l, b, t, gpu_idx[i, b].tolist(), idxs[b].tolist())
                    exact += 1
                else:
                    assert abs(zs[int(gpu_idx[i, b, t])] - zs[order[t]]) <= tol, (l, b, t)
            if np.array_equal(gpu_idx[i, b], idxs[b]):
                e = float(np.max(np.abs(gpu_w[i, b] - gws[b])) / np.max(np.abs(gws[b])))
                assert e < tol_rel, (l, b, e)
    return exact
