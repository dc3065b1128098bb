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


# Decisions (argmax, router top-k). The pre-registered rule: a decision between outputs i and j must
# be exact wherever the oracle's margin exceeds 4 * gamma_K * max(S_i, S_j), where
# S_i = sum_k |w_ik| |y_k| over the product's K inputs and gamma_K = K u / (1 - K u), u = 2^-24, is the
# worst-case relative error of a K-term fp32 dot product. A decision inside that bound is reported as
# a tie within rounding (not counted as exact); the GPU's pick must then be one of the tied outputs.
U32 = 2.0 ** -24


def gamma(K: int) -> float:
    return K * U32 / (1.0 - K * U32)


def decision_bounds(W_bits: np.ndarray, y: np.ndarray, chunk: int = 16384) -> np.ndarray:
    """4 * gamma_K * sum_k |w_ik| |y_bk| for every row b of y and output i of the bf16 matrix W [N][K]."""
    W_bits = np.ascontiguousarray(W_bits)
    N, K = W_bits.shape
    Y = np.abs(np.asarray(y, np.float32).reshape(-1, K))
    out = np.empty((Y.shape[0], N), np.float64)
    for n0 in range(0, N, chunk):
        A = np.abs(bf16_to_f32(W_bits[n0:n0 + chunk]))
        out[:, n0:n0 + chunk] = Y @ A.T
    return 4.0 * gamma(K) * out


def check_argmax(gpu_am, logits, bounds, label=""):
    """Argmax parity under the decision rule; the oracle's argmax is the first maximum. Returns
    (exact, ties)."""
    exact = ties = 0
    for b, row in enumerate(logits):
        z = row.astype(np.float64)
        order = np.argsort(-z, kind="stable")
        i, j = int(order[0]), int(order[1])
        thr = max(bounds[b, i], bounds[b, j])
        g = int(gpu_am[b])
        if z[i] - z[j] > thr:
            assert g == i, (label, b, g, i)
            exact += 1
        else:
            ties += 1
            print(f"{label} argmax row {b}: tie within rounding (margin {z[i] - z[j]:.3g} <= bound {thr:.3g})")
            assert z[g] >= z[i] - thr, (label, b, g, i)
    return exact, ties


def make_gpu(cfg, W, S, max_batch=None, device=0):
    from persistent_megakernel_mk_amd import mk

    m = mk.Megakernel(cfg, device=device, max_batch=max_batch)
    m.load_weights(W)
    m.set_states(S)
    return m


def compare_states(gpu_S, ref_S, new_positions=None, tol=None):
    """Caches: rows other than this step's new rows bit-identical; new rows (bf16 roundings of fp32
    projections that differ from the oracle's by summation order) within one bf16 ulp plus the
    projection tolerance relative to the row's largest entry. Linear states: fp32, relative tolerance.
    tol replaces REL_TOL (steps whose activations enter products as bf16)."""
    tol = REL_TOL if tol is None else tol
    for name, ref in ref_S.items():
        g = gpu_S[name]
        if name.endswith("lstate"):
            e = rel_err(g, ref)
            assert e < tol, (name, e)
            continue
        gf, rf = bf16_to_f32(g).astype(np.float64), bf16_to_f32(ref).astype(np.float64)
        rowmax = np.max(np.abs(rf), axis=-1, keepdims=True)
        bound = np.maximum(np.abs(rf), np.abs(gf)) * 2.0 ** -7 + tol * rowmax
        diff = np.abs(gf - rf)
        assert np.all(diff <= bound), (name, float(diff.max()))
        if new_positions is not None:
            pax = 1 if name.endswith("latent") else 2  # position axis: latent [B][pos][D], K/V [B][heads][pos][d]
            mask = np.ones(g.shape[pax], bool)
            mask[list(new_positions)] = False
            idx = (slice(None),) * pax + (mask,)
            assert np.array_equal(g[idx], ref[idx]), name


def check_routes(gpu_idx, gpu_w, route_log, moe_layers, W, label=""):
    """Routing parity per MoE layer, row and rank t under the decision rule: the expert at rank t is
    determined when its margins to ranks t-1 and t+1 both exceed their bounds, and must then be the
    oracle's. Gates (normalised sigmoids) of identical selections agree to REL_TOL. Returns
    (exact, ties, ties where the GPU still picked the oracle's expert)."""
    exact = ties = agree = 0
    for li, l in enumerate(moe_layers):
        idxs, gws, z, y = route_log[l]
        bnd = decision_bounds(W[f"l{l}.router"], y)
        E = z.shape[1]
        for b in range(idxs.shape[0]):
            zs = z[b].astype(np.float64)
            order = np.argsort(-zs, kind="stable")
            assert np.array_equal(order[:idxs.shape[1]], idxs[b])  # the oracle's rank order (first max on ties)

            def apart(e1, e2):
                return zs[e1] - zs[e2] > max(bnd[b, e1], bnd[b, e2])

            for t in range(idxs.shape[1]):
                e = int(order[t])
                g = int(gpu_idx[li, b, t])
                ok_above = t == 0 or apart(int(order[t - 1]), e)
                ok_below = t + 1 >= E or apart(e, int(order[t + 1]))
                if ok_above and ok_below:
                    assert g == e, (label, l, b, t, gpu_idx[li, b].tolist(), idxs[b].tolist())
                    exact += 1
                else:
                    ties += 1
                    agree += g == e
                    assert 0 <= g < E and abs(zs[g] - zs[e]) <= 2 * max(bnd[b, g], bnd[b, e]), (label, l, b, t)
            if np.array_equal(gpu_idx[li, b], idxs[b]):
                err = float(np.max(np.abs(gpu_w[li, b] - gws[b])) / np.max(np.abs(gws[b])))
                assert err < REL_TOL, (label, l, b, err)
    return exact, ties, agree


def argmax_parity(gpu_am, ref, W, label=""):
    """check_argmax with the bounds of the LM head on the oracle's final normalised rows."""
    exact, ties = check_argmax(gpu_am, ref["logits"], decision_bounds(W["lm_head"], ref["final_y"]), label)
    print(f"{label}: argmax {exact} exact, {ties} ties within rounding")
    return exact, ties


def routes_parity(gpu_idx, gpu_w, ref, cfg, W, label="", max_tie_frac=0.1):
    """check_routes over every MoE layer. With max_tie_frac, at most that fraction of the decisions may be
    ties within rounding (the small configurations, whose products are short). The worst-case bound
    grows with K, so at full size (K = 6144, 7168) most router decisions fall inside it; there the ties
    are reported together with how many of them still match the oracle's pick."""
    layers = [l for l in range(cfg.n_layers) if cfg.ffns[l] == "moe"]
    exact, ties, agree = check_routes(gpu_idx, gpu_w, ref["routes"], layers, W, label)
    print(f"{label}: routing {exact} exact, {ties} ties within rounding ({agree} of them the oracle's pick)")
    assert exact + ties == len(layers) * gpu_idx.shape[1] * cfg.top_k
    if max_tie_frac is not None:
        assert ties <= int((exact + ties) * max_tie_frac), (label, exact, ties)
    return exact, ties, agree


class FullSizeWeights:
    """name -> host array of a full-size configuration, with the values bench.build_gpu loads: bf16
    tensors from the seeded generator, NVFP4 expert matrices from the per-projection pool
    (bench.pooled_source). Holds only the tensors of the layer in use and the pool, so the oracle can
    run a step whose experts would not fit on the host at once; prints a line as each layer starts."""

    def __init__(self, cfg, expert_pool=8):
        from persistent_megakernel_mk_amd import synth

        self.cfg, self.expert_pool, self.synth = cfg, expert_pool, synth
        self.specs = {s.name: s for s in synth.weight_specs(cfg)}
        self.layer, self.cache, self.pool = None, {}, {}

    def __getitem__(self, name):
        import bench

        spec = self.specs[name]
        prefix = name.split(".")[0]
        if prefix != self.layer:
            self.layer, self.cache = prefix, {}
            print(f"  oracle {self.cfg.name}: {prefix}", flush=True)
        if spec.kind in ("nvfp4", "mxfp4"):
            key, src = bench.pooled_source(self.cfg, spec, self.expert_pool)
            if key not in self.pool:
                self.pool[key] = self.synth.generate(src, self.cfg.seed)
            return self.pool[key]
        if name not in self.cache:
            self.cache[name] = self.synth.generate(spec, self.cfg.seed)
        return self.cache[name]

    def __contains__(self, name):
        return name in self.specs

    def keys(self):
        return self.specs.keys()
