"""Pins for the CPU oracle: each test checks an oracle op against something other than itself — a
library routine, a closed form, a special case, an invariant, or an independent formulation of the same
quantity (the O(T^2) matrix form of the delta rule, the naive form of absorbed latent attention, the
dense form of a mixture of experts with top-k = E, and eight sequential decode steps for a verify block).
A plausible mistake in an op (a dropped term, a wrong sign or index, a transposed operand) fails one of
them. CPU only."""
import math

import numpy as np
import pytest
import torch


def bf16_bits(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_val(bits):
    return torch.tensor(np.asarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).float().numpy()


# ---- conversions -----------------------------------------------------------------------------

def test_bf16_round_matches_torch(oracle):
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(5000).astype(np.float32) * 3,
                        # exact ties between two bf16 neighbours: 1 + 2^-8 -> 1, 1 + 3*2^-8 -> 1 + 2^-6
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0, -0.0, 65504.0], np.float32)])
    ours = oracle.round_bf16(x)
    assert np.array_equal(ours, bf16_bits(x))
    assert np.array_equal(oracle.widen(ours), bf16_val(ours))


def test_e4m3_all_codes_match_torch(oracle):
    L = oracle.lib()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    ours = np.array([L.orc_e4m3_value(c) for c in range(256)], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7e] == 448.0 and ours[1] == 2.0 ** -9


def test_e2m1_codes_match_ocp_table(oracle):
    # OCP microscaling spec, FP4 E2M1 magnitudes for codes 0..7; bit 3 is the sign
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    L = oracle.lib()
    for c in range(16):
        v = L.orc_e2m1_value(c)
        assert v == (-1.0 if c & 8 else 1.0) * mags[c & 7]


def test_nvfp4_dequant_nibble_order_and_scales(oracle):
    L = oracle.lib()
    K = 32
    codes = np.zeros(K // 2, np.uint8)
    codes[0] = 0x71  # element 0 -> code 1 (0.5), element 1 -> code 7 (6.0)
    codes[8] = 0xA3  # element 16 -> code 3 (1.5), element 17 -> code 10 (-1.0)
    scales = np.array([0x38, 0x40], np.uint8)  # e4m3: 1.0 and 2.0
    out = np.zeros(K, np.float32)
    L.orc_nvfp4_dequant_row(codes.ctypes.data, scales.ctypes.data, 0.5, K, out.ctypes.data)
    assert out[0] == 0.5 * 1.0 * 0.5 and out[1] == 6.0 * 0.5
    assert out[16] == 1.5 * 2.0 * 0.5 and out[17] == -1.0 * 2.0 * 0.5
    assert np.count_nonzero(out) == 4


# ---- matrix-vector product ---------------------------------------------------------------------

@pytest.mark.parametrize("N,K,B", [(37, 100, 1), (64, 513, 3), (16, 2048, 8)])
def test_gemv_matches_float64_matmul(oracle, N, K, B):
    rng = np.random.default_rng(N * K + B)
    W = bf16_bits(rng.standard_normal((N, K)) * 0.05)
    X = rng.standard_normal((B, K)).astype(np.float32)
    Y = oracle.gemv(W, X)
    ref = X.astype(np.float64) @ bf16_val(W).astype(np.float64).T
    bound = 2 * K * 2 ** -24 * (np.abs(X).astype(np.float64) @ np.abs(bf16_val(W)).astype(np.float64).T)
    assert np.all(np.abs(Y - ref) <= bound + 1e-30)


def test_gemv_nvfp4_equals_dequantised_gemv(oracle, synth):
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((48, 256)) * 0.02).astype(np.float32)
    t = synth.nvfp4_encode(w)
    X = rng.standard_normal((2, 256)).astype(np.float32)
    Y = oracle.gemv(t, X)
    # dequantise with torch's fp8 decode and the OCP fp4 table, then a float64 product
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    nib = np.stack([t.codes & 15, t.codes >> 4], -1).reshape(48, 256)
    vals = mags[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    sc = torch.tensor(t.scales).view(torch.float8_e4m3fn).double().numpy()
    wd = vals * np.repeat(sc, 16, axis=1) * t.tensor_scale
    ref = X.astype(np.float64) @ wd.T
    assert np.allclose(Y, ref, rtol=1e-5, atol=1e-6)
    # the encoding is a faithful quantiser of the synthetic weights (documented 6*448 scale choice)
    assert np.max(np.abs(wd - w)) <= 0.25 * np.max(np.abs(w))


# ---- norms, rotary embedding, activations ------------------------------------------------------

def test_rmsnorm_constant_vector_closed_form(oracle):
    H, eps = 64, 1e-6
    g = bf16_bits(1.0 + 0.02 * np.random.default_rng(1).standard_normal(H))
    for c in (0.5, -3.0, 1e-3):
        x = np.full((1, H), c, np.float32)
        y = oracle.rmsnorm(x, g, eps)
        ref = bf16_val(g) * math.copysign(1.0, c) / math.sqrt(1.0 + eps / c ** 2)
        assert np.allclose(y[0], ref, rtol=3e-6)


def test_rmsnorm_scale_invariance_and_unit_rms(oracle):
    rng = np.random.default_rng(2)
    H = 5120
    x = rng.standard_normal((2, H)).astype(np.float32)
    ones = bf16_bits(np.ones(H))
    y1 = oracle.rmsnorm(x, ones, 1e-6)
    y2 = oracle.rmsnorm(x * 8.0, ones, 1e-6)
    assert np.allclose(y1, y2, rtol=1e-5, atol=1e-6)
    assert np.allclose(np.sqrt(np.mean(y1.astype(np.float64) ** 2, axis=1)), 1.0, rtol=1e-5)


def test_rope_identity_norm_and_relative_position(oracle):
    rng = np.random.default_rng(3)
    d, theta = 128, 1e6
    q = rng.standard_normal(d).astype(np.float32)
    k = rng.standard_normal(d).astype(np.float32)
    assert np.array_equal(oracle.rope(q, 1, d, 0, d, 0, theta), q)  # position 0: identity
    r = oracle.rope(q, 1, d, 0, d, 4096, theta)
    assert abs(np.linalg.norm(r) - np.linalg.norm(q)) < 1e-4  # a rotation keeps the norm
    # <R_m q, R_n k> depends only on m - n
    a = np.dot(oracle.rope(q, 1, d, 0, d, 700, theta).astype(np.float64), oracle.rope(k, 1, d, 0, d, 300, theta))
    b = np.dot(oracle.rope(q, 1, d, 0, d, 400, theta).astype(np.float64), k)
    assert abs(a - b) < 1e-4 * (1 + abs(b))
    # a single pair rotates the plane (i, i + d/2) at frequency theta^(-2i/d)
    e = np.zeros(d, np.float32)
    e[5] = 1.0
    r = oracle.rope(e, 1, d, 0, d, 9, theta)
    w = 9 * theta ** (-2 * 5 / d)
    assert abs(r[5] - math.cos(w)) < 1e-6 and abs(r[5 + d // 2] - math.sin(w)) < 1e-6
    assert np.count_nonzero(np.abs(r) > 1e-12) == 2


def test_rope_partial_offset_leaves_other_entries(oracle):
    rng = np.random.default_rng(4)
    v = rng.standard_normal((2, 192)).astype(np.float32)
    r = oracle.rope(v, 2, 192, 128, 64, 77, 1e6)
    assert np.array_equal(r[:, :128], v[:, :128])
    assert not np.allclose(r[:, 128:], v[:, 128:])


def test_silu_values_and_gates(oracle):
    g = np.array([0.0, 1.0, 30.0, -30.0, -1.0], np.float32)
    h = oracle.silu_mul(g, np.ones_like(g))
    assert h[0] == 0.0
    assert abs(h[1] - 0.7310585786300049) < 1e-7  # 1 / (1 + e^-1)
    assert abs(h[2] - 30.0) < 1e-5 and abs(h[3]) < 1e-10
    assert abs(h[4] + 0.2689414213699951) < 1e-7
    a = np.linspace(-30, 30, 121).astype(np.float32)
    al = oracle.decay_gates(a)
    # exp(-softplus(a)) = sigmoid(-a): a decay in (0, 1)
    assert np.allclose(al, 1 / (1 + np.exp(a.astype(np.float64))), rtol=2e-6, atol=1e-12)
    assert np.all(al > 0) and np.all(al <= 1)  # (0, 1) up to fp32 rounding at the ends
    assert np.allclose(oracle.sigmoid(a), 1 / (1 + np.exp(-a.astype(np.float64))), rtol=2e-6, atol=1e-12)


def test_argmax_and_topk_ties_take_lowest_index(oracle):
    assert oracle.argmax(np.array([1, 3, 3, 2], np.float32)) == 1
    z = np.array([0.5, 2.0, 2.0, -1.0, 2.0, 0.1], np.float32)
    idx, g = oracle.topk(z, 4)
    assert list(idx) == [1, 2, 4, 0]
    s = 1 / (1 + np.exp(-z[idx].astype(np.float64)))
    assert np.allclose(g, s / s.sum(), rtol=1e-6)
    assert abs(float(g.sum()) - 1.0) < 1e-6
    idx, g = oracle.topk(z, 6)  # k = E: every expert, in descending order, stable on ties
    assert list(idx) == [1, 2, 4, 0, 5, 3]


# ---- attention -----------------------------------------------------------------------------------

def _cache(rng, nkv, cap, d):
    return bf16_bits(rng.standard_normal((nkv, cap, d)))


def test_attention_single_key_returns_value(oracle):
    rng = np.random.default_rng(6)
    kc, vc = _cache(rng, 2, 8, 64), _cache(rng, 2, 8, 64)
    q = rng.standard_normal(4 * 64).astype(np.float32)
    o = oracle.attention(q, 4, 64, kc, vc, 1).reshape(4, 64)
    for h in range(4):
        assert np.array_equal(o[h], bf16_val(vc[h // 2, 0]))


def test_attention_uniform_and_grouping(oracle):
    rng = np.random.default_rng(7)
    nq, nkv, d, L = 6, 2, 32, 50
    kc = _cache(rng, nkv, 64, d)
    vc = _cache(rng, nkv, 64, d)
    o = oracle.attention(np.zeros(nq * d, np.float32), nq, d, kc, vc, L).reshape(nq, d)  # q = 0: uniform weights
    for h in range(nq):
        ref = bf16_val(vc[h // 3, :L]).astype(np.float64).mean(axis=0)  # query head h reads kv head h // 3
        assert np.allclose(o[h], ref, atol=2e-6)
    # a key far better aligned than the rest takes all the weight
    kc2 = kc.copy()
    q = np.zeros(nq * d, np.float32)
    q[:d] = 40.0
    kc2[0, 17] = bf16_bits(np.full(d, 4.0))
    o2 = oracle.attention(q, nq, d, kc2, vc, L).reshape(nq, d)
    assert np.allclose(o2[0], bf16_val(vc[0, 17]), atol=1e-5)


# ---- gated delta rule ---------------------------------------------------------------------------

def _delta_matrix_form(S0, Q, K, V, A, beta):
    """O(T^2) closed form of o_t for S_t = S_{t-1} Diag(a_t)(I - b_t k_t k_t^T) + b_t v_t k_t^T,
    o_t = S_t q_t, in float64 (rows of Q, K, V are time steps; A[t] holds the d_k decays)."""
    T, dk = K.shape
    cum = np.cumprod(A, axis=0)  # cum[t] = a_1 * ... * a_t (0-based t)

    def D(i, j):  # diag of a_{j+1} ... a_i, for j <= i (j = -1 means from the start)
        num = cum[i]
        den = cum[j] if j >= 0 else np.ones(dk)
        return num / den

    M = np.zeros((T, T))
    P = np.zeros((T, T))
    for i in range(T):
        for j in range(i + 1):
            dij = D(i, j)
            if j < i:
                M[i, j] = beta[i] * np.dot(K[j] * dij, K[i])
            P[i, j] = np.dot(K[j] * dij, Q[i])
    W0 = np.stack([S0 @ (D(i, -1) * K[i]) for i in range(T)])
    U = np.linalg.solve(np.eye(T) + M, beta[:, None] * (V - W0))
    return P @ U + np.stack([S0 @ (D(i, -1) * Q[i]) for i in range(T)])


def _delta_backward_form(S0, Q, K, V, A, beta):
    """Second independent form: o_t = sum over i <= t of b_i v_i (k_i . w_i) + S0 w_0 with
    w <- Diag(a_i)(w - b_i k_i (k_i . w)) walking i from t down to 1."""
    T = K.shape[0]
    out = []
    for t in range(T):
        w = Q[t].copy()
        o = np.zeros(S0.shape[0])
        for i in range(t, -1, -1):
            kw = np.dot(K[i], w)
            o += beta[i] * V[i] * kw
            w = A[i] * (w - beta[i] * K[i] * kw)
        out.append(o + S0 @ w)
    return np.stack(out)


@pytest.mark.parametrize("per_channel", [False, True])
def test_delta_rule_equals_matrix_and_backward_forms(oracle, per_channel):
    rng = np.random.default_rng(9 + per_channel)
    T, dk, dv = 7, 16, 12
    S0 = (rng.standard_normal((dv, dk)) * 0.1).astype(np.float32)
    Q = rng.standard_normal((T, dk)); Q /= np.linalg.norm(Q, axis=1, keepdims=True)
    K = rng.standard_normal((T, dk)); K /= np.linalg.norm(K, axis=1, keepdims=True)
    V = rng.standard_normal((T, dv))
    if per_channel:
        A = rng.uniform(0.5, 1.0, (T, dk))
    else:
        A = np.repeat(rng.uniform(0.5, 1.0, (T, 1)), dk, axis=1)
    beta = rng.uniform(0.1, 1.0, T)
    Q, K, V, A = (a.astype(np.float32) for a in (Q, K, V, A))
    beta = beta.astype(np.float32)
    S = S0.copy()
    O = np.stack([oracle.delta_step(S, Q[t], K[t], V[t], A[t], float(beta[t])) for t in range(T)])
    args = [a.astype(np.float64) for a in (S0, Q, K, V, A, beta)]
    assert np.allclose(O, _delta_matrix_form(*args), atol=2e-5)
    assert np.allclose(O, _delta_backward_form(*args), atol=2e-5)


def test_delta_rule_special_cases(oracle):
    rng = np.random.default_rng(11)
    dk = dv = 8
    S0 = rng.standard_normal((dv, dk)).astype(np.float32)
    # beta = 0: pure decay, S_t = (prod alpha) S_0
    S = S0.copy()
    for a in (0.9, 0.5, 0.8):
        oracle.delta_step(S, np.zeros(dk), np.ones(dk) / math.sqrt(dk), rng.standard_normal(dv), np.full(dk, a), 0.0)
    assert np.allclose(S, S0 * (0.9 * 0.5 * 0.8), rtol=1e-6)
    # alpha = 1, beta = 1 and orthonormal keys: the state maps each written key to its value
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    S = S0.copy()
    vals = rng.standard_normal((3, dv)).astype(np.float32)
    for t in range(3):
        oracle.delta_step(S, np.zeros(dk), Qm[:, t], vals[t], np.ones(dk), 1.0)
    for t in range(3):
        assert np.allclose(S @ Qm[:, t], vals[t], atol=1e-5)


# ---- latent attention ----------------------------------------------------------------------------

def test_mla_absorbed_equals_naive_mha(oracle):
    rng = np.random.default_rng(12)
    heads, nope, rp, rank, vd, L = 3, 16, 8, 32, 12, 20
    wuk = bf16_bits(rng.standard_normal((heads * nope, rank)) * 0.2)
    wuv = bf16_bits(rng.standard_normal((heads * vd, rank)) * 0.2)
    cache = bf16_bits(rng.standard_normal((L + 4, rank + rp)))
    q = rng.standard_normal(heads * (nope + rp)).astype(np.float32)
    out = oracle.mla_attend(q, heads, nope, rp, wuk, wuv, rank, vd, cache, L).reshape(heads, vd)
    Wk, Wv, C = bf16_val(wuk).astype(np.float64), bf16_val(wuv).astype(np.float64), bf16_val(cache).astype(np.float64)
    for h in range(heads):
        keys = np.concatenate([C[:L, :rank] @ Wk[h * nope:(h + 1) * nope].T, C[:L, rank:]], axis=1)  # materialised k
        vals = C[:L, :rank] @ Wv[h * vd:(h + 1) * vd].T  # materialised v
        s = keys @ q[h * (nope + rp):(h + 1) * (nope + rp)].astype(np.float64) / math.sqrt(nope + rp)
        p = np.exp(s - s.max())
        p /= p.sum()
        assert np.allclose(out[h], p @ vals, rtol=1e-4, atol=1e-5)


# ---- mixture of experts --------------------------------------------------------------------------

class _MoECfg:
    def __init__(self, E, k, H, F):
        self.ffns = ("moe",)
        self.n_experts, self.top_k, self.hidden, self.expert_ffn, self.n_shared = E, k, H, F, 1


def _moe_weights(rng, E, H, F):
    W = {"l0.router": bf16_bits(rng.standard_normal((E, H)) * 0.3)}
    for name in ["s0"] + [f"e{e}" for e in range(E)]:
        W[f"l0.{name}.wg"] = bf16_bits(rng.standard_normal((F, H)) * 0.2)
        W[f"l0.{name}.wu"] = bf16_bits(rng.standard_normal((F, H)) * 0.2)
        W[f"l0.{name}.wd"] = bf16_bits(rng.standard_normal((H, F)) * 0.2)
    return W


def test_moe_topk_equal_to_e_is_dense_weighted_sum(oracle):
    rng = np.random.default_rng(13)
    E, H, F = 6, 32, 24
    W = _moe_weights(rng, E, H, F)
    y = rng.standard_normal((2, H)).astype(np.float32)
    out = oracle._ffn(_MoECfg(E, E, H, F), W, 0, y, None)
    z = y.astype(np.float64) @ bf16_val(W["l0.router"]).astype(np.float64).T
    s = 1 / (1 + np.exp(-z))
    for b in range(2):
        dense = oracle._swiglu(W, "l0.s0.", y[b]).astype(np.float64)
        for e in range(E):
            dense += s[b, e] / s[b].sum() * oracle._swiglu(W, f"l0.e{e}.", y[b])
        assert np.allclose(out[b], dense, rtol=1e-4, atol=1e-5)


def test_moe_routes_to_the_selected_experts_only(oracle):
    rng = np.random.default_rng(14)
    E, H, F = 5, 32, 16
    W = _moe_weights(rng, E, H, F)
    y = rng.standard_normal((1, H)).astype(np.float32)
    log = {}
    out = oracle._ffn(_MoECfg(E, 2, H, F), W, 0, y, log)
    idx, gw, z, _ = log[0]
    top2 = np.argsort(-z[0], kind="stable")[:2]
    assert list(idx[0]) == list(top2)
    # zeroing an unselected expert changes nothing; zeroing a selected one does
    other = [e for e in range(E) if e not in top2][0]
    W2 = dict(W)
    W2[f"l0.e{other}.wd"] = np.zeros_like(W[f"l0.e{other}.wd"])
    assert np.array_equal(oracle._ffn(_MoECfg(E, 2, H, F), W2, 0, y, None), out)
    W3 = dict(W)
    W3[f"l0.e{int(top2[0])}.wd"] = np.zeros_like(W[f"l0.e{int(top2[0])}.wd"])
    assert not np.allclose(oracle._ffn(_MoECfg(E, 2, H, F), W3, 0, y, None), out)


# ---- whole steps ---------------------------------------------------------------------------------

def test_kda_with_equal_channel_gates_equals_gdn(oracle, synth):
    from dataclasses import replace
    cfg_g = replace(synth.CONFIGS["c1s"], n_layers=1, mixers=("gdn",), ffns=("dense",), vocab=0)
    cfg_k = replace(cfg_g, mixers=("kda",))
    Wg = synth.LazyWeights(cfg_g)
    Wk = dict((n, Wg[n]) for n in Wg.keys())
    Wk["l0.wa"] = np.ascontiguousarray(np.repeat(Wg["l0.wa"], cfg_g.d_k, axis=0))  # every channel of a head alike
    Sg = synth.make_states(cfg_g)
    Sk = oracle.copy_states(Sg)
    x = synth.make_inputs(cfg_g)["hidden_in"]
    og = oracle.decode_step(cfg_g, Wg, Sg, {"hidden_in": x}, cfg_g.ctx)["hidden_out"]
    ok = oracle.decode_step(cfg_k, Wk, Sk, {"hidden_in": x}, cfg_k.ctx)["hidden_out"]
    assert np.array_equal(og, ok)
    assert np.array_equal(Sg["l0.lstate"], Sk["l0.lstate"])


def test_zero_layers_reduce_to_norm_and_lm_head(oracle, synth):
    cfg = synth.CONFIGS["c0"]
    W = {n: synth.LazyWeights(cfg)[n] for n in synth.LazyWeights(cfg).keys()}
    for l in range(cfg.n_layers):  # zero output projections: every residual block adds exactly 0
        W[f"l{l}.wo"] = np.zeros_like(W[f"l{l}.wo"])
        W[f"l{l}.wd"] = np.zeros_like(W[f"l{l}.wd"])
    W["final_norm"] = bf16_bits(np.ones(cfg.hidden))
    W["embed"] = W["embed"].copy()
    tok = 17
    W["embed"][tok] = bf16_bits(np.full(cfg.hidden, -0.75))  # constant row: the norm gives -1/sqrt(1+eps/c^2)
    S = synth.make_states(cfg)
    out = oracle.decode_step(cfg, W, S, {"tokens": np.array([tok], np.int32)}, cfg.ctx)
    r = -1.0 / math.sqrt(1 + cfg.eps / 0.75 ** 2)
    ref = bf16_val(W["lm_head"]).astype(np.float64).sum(axis=1) * r
    assert np.allclose(out["logits"][0], ref, rtol=1e-5, atol=1e-5)
    assert out["argmax"][0] == int(np.argmax(ref))


def test_verify_block_equals_eight_sequential_decodes(oracle, synth):
    from dataclasses import replace
    cfg_v = synth.CONFIGS["c2s"]
    cfg_d = replace(cfg_v, verify_rows=0)
    W = synth.LazyWeights(cfg_v)
    S0 = synth.make_states(cfg_v)
    rng = np.random.default_rng(15)
    toks = rng.integers(0, cfg_v.vocab, 8).astype(np.int32)
    pos = cfg_v.ctx
    Sv = oracle.copy_states(S0)
    ver = oracle.verify_step(cfg_v, W, Sv, toks, pos)
    Sd = oracle.copy_states(S0)
    lin = [l for l in range(cfg_v.n_layers) if cfg_v.mixers[l] == "gdn"]
    for j in range(8):
        dec = oracle.decode_step(cfg_d, W, Sd, {"tokens": toks[j:j + 1]}, pos + j)
        assert np.array_equal(dec["logits"][0], ver["logits"][j])
        for l in lin:
            assert np.array_equal(Sd[f"l{l}.lstate"], ver["snapshots"][l][j])
    for l in range(cfg_v.n_layers):
        if cfg_v.mixers[l] == "gqa":
            assert np.array_equal(Sd[f"l{l}.kcache"], Sv[f"l{l}.kcache"])
            assert np.array_equal(Sd[f"l{l}.vcache"], Sv[f"l{l}.vcache"])
    a = ver["accepted"]
    for l in lin:
        assert np.array_equal(Sv[f"l{l}.lstate"], ver["snapshots"][l][a])


def test_verify_acceptance_counts_matching_prefix(oracle, synth):
    # drafts equal to the greedy continuation are all accepted; a wrong draft at position i stops at i-1
    from dataclasses import replace
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
    ver = oracle.verify_step(cfg_v, W, oracle.copy_states(S0), np.array(toks, np.int32), pos)
    assert ver["accepted"] == 7
    bad = list(toks)
    bad[4] = (bad[4] + 1) % cfg_v.vocab
    ver = oracle.verify_step(cfg_v, W, oracle.copy_states(S0), np.array(bad, np.int32), pos)
    assert ver["accepted"] == 3 and ver["bonus"] == toks[4]
