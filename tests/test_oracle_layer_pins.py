"""Layer-level pins for the CPU oracle: each mixer layer and the per-layer composition of the oracle
against a float64 restatement written here from the definitions (complex-exponential RoPE, a
library softmax, the matrix form of one gated-delta-rule step with gates from the identity
exp(-softplus(a)) = sigmoid(-a), materialised rather than absorbed latent attention), and against
closed forms of special cases (decay gates that are exactly 0 or 1, a two-key softmax). They fix the
wiring that the per-op pins cannot see: which vectors are L2-normalised, the attention scale, that
keys are rotated before they are appended, which slice of a latent-attention query is rotated, the
sign of the decay gate, and the pre-norm residual composition. CPU only.

Sources: page "Kimi K3's TPU megakernel: 92 layers in one Pallas call, and what 709 tokens a second
measures", section "How it maps onto a TPU v7" (per-layer norm, mixer, residual, norm, FFN,
residual; KDA and MLA layers); page "TPU megakernels for Kimi K3, Qwen3.8-27B, and Muse-Spark-Open"
(gated-delta-net and grouped-query attention layers of the dense stack)."""
import math
from types import SimpleNamespace

import numpy as np
import pytest
import torch
from scipy.special import expit, softmax


def bits(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def val(b):
    """bf16 bits -> float64"""
    return torch.tensor(np.asarray(b, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).double().numpy()


def rope64(x, pos, theta, rot):
    """Rotary embedding in complex form: entries (i, i + rot/2), i < rot/2, are the real and imaginary
    parts of z_i, multiplied by exp(1j * pos * theta^(-2i/rot)). Acts on the last axis's first rot
    entries (float64)."""
    x = np.array(x, dtype=np.float64)
    half = rot // 2
    z = x[..., :half] + 1j * x[..., half:rot]
    z = z * np.exp(1j * pos * theta ** (-2.0 * np.arange(half) / rot))
    x[..., :half], x[..., half:rot] = z.real, z.imag
    return x


def bf16_ulps(a_bits, b_bits):
    """distance in bf16 units in the last place between two arrays of bf16 bits of the same sign"""
    a = a_bits.astype(np.int32)
    b = b_bits.astype(np.int32)
    a = np.where(a & 0x8000, -(a & 0x7FFF), a)
    b = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(a - b)


def rms64(x, g, eps):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * val(g)


# ---- L2 normalisation -----------------------------------------------------------------------------

def test_l2norm_gives_unit_vectors_in_the_same_direction(oracle):
    rng = np.random.default_rng(30)
    d = 128
    v = (rng.standard_normal((3, d)) * np.array([[0.01], [1.0], [40.0]])).astype(np.float32)
    eps = 1e-6
    u = oracle.l2norm(v, d, eps).astype(np.float64)
    n = np.linalg.norm(v.astype(np.float64), axis=1)
    # |u| = |v| / sqrt(|v|^2 + eps): 1 up to the eps term (an RMS normalisation would give sqrt(d))
    assert np.allclose(np.linalg.norm(u, axis=1), n / np.sqrt(n * n + eps), rtol=1e-6)
    ref = v.astype(np.float64) / np.sqrt(n * n + eps)[:, None]
    assert np.allclose(u, ref, rtol=1e-5, atol=1e-7)


# ---- attention scale ------------------------------------------------------------------------------

def test_attention_matches_float64_softmax(oracle):
    rng = np.random.default_rng(31)
    nq, nkv, d, cap, L = 6, 2, 64, 48, 37
    kc = bits(rng.standard_normal((nkv, cap, d)))
    vc = bits(rng.standard_normal((nkv, cap, d)))
    q = (rng.standard_normal(nq * d) * 2.0).astype(np.float32)
    o = oracle.attention(q, nq, d, kc, vc, L).reshape(nq, d)
    K, V = val(kc), val(vc)
    for h in range(nq):
        g = h // (nq // nkv)
        p = softmax(K[g, :L] @ q[h * d:(h + 1) * d].astype(np.float64) / math.sqrt(d))
        assert np.allclose(o[h], p @ V[g, :L], rtol=2e-5, atol=2e-6), h


def test_attention_two_keys_closed_form(oracle):
    # k_0 = 0 and k_1 = 2 e_0 with q = 8 e_0: scores 0 and 16 / sqrt(64) = 2, so the weights are
    # 1 / (1 + e^2) and e^2 / (1 + e^2) (a 1/d scale would give 0.25 instead of 2)
    d = 64
    kc = np.zeros((1, 2, d), np.uint16)
    kc[0, 1, 0] = bits(2.0)
    vc = bits(np.stack([np.full(d, 1.0), np.full(d, -3.0)]))[None]
    q = np.zeros(d, np.float32)
    q[0] = 8.0
    o = oracle.attention(q, 1, d, kc, vc, 2)
    w1 = math.exp(2) / (1 + math.exp(2))
    assert np.allclose(o, (1 - w1) * 1.0 + w1 * -3.0, rtol=1e-6)


def test_attention_is_invariant_to_cache_permutation(oracle):
    # permuting cache positions changes nothing (softmax attention is a function of the set of keys)
    rng = np.random.default_rng(8)
    d, L = 64, 40
    kc, vc = bits(rng.standard_normal((1, L, d))), bits(rng.standard_normal((1, L, d)))
    q = rng.standard_normal(d).astype(np.float32)
    perm = rng.permutation(L)
    o1 = oracle.attention(q, 1, d, kc, vc, L)
    o2 = oracle.attention(q, 1, d, np.ascontiguousarray(kc[:, perm]), np.ascontiguousarray(vc[:, perm]), L)
    assert np.allclose(o1, o2, rtol=1e-5, atol=1e-6)


# ---- grouped-query attention layer ----------------------------------------------------------------

def _gqa_setup(rng, H=96, nq=4, nkv=2, d=32, cap=40, B=2):
    cfg = SimpleNamespace(n_q_heads=nq, n_kv_heads=nkv, head_dim=d, rope_theta=1e4)
    W = {"l0.wq": bits(rng.standard_normal((nq * d, H)) * 0.2), "l0.wk": bits(rng.standard_normal((nkv * d, H)) * 0.2),
         "l0.wv": bits(rng.standard_normal((nkv * d, H)) * 0.2), "l0.wo": bits(rng.standard_normal((H, nq * d)) * 0.2)}
    S = {"l0.kcache": bits(rng.standard_normal((B, nkv, cap, d))), "l0.vcache": bits(rng.standard_normal((B, nkv, cap, d)))}
    return cfg, W, S


def test_gqa_layer_matches_float64_restatement(oracle):
    """Two sequences at different positions: each appends its rotated key and its value at its own
    position, then attends to its own positions 0..p with scale 1/sqrt(d)."""
    rng = np.random.default_rng(32)
    cfg, W, S = _gqa_setup(rng)
    nq, nkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    S0 = {k: v.copy() for k, v in S.items()}
    y = rng.standard_normal((2, 96)).astype(np.float32)
    pos = [23, 9]
    out = oracle._gqa_rows(cfg, W, S, 0, y, [0, 1], pos)
    Y = y.astype(np.float64)
    for r, (b, p) in enumerate(zip([0, 1], pos)):
        q = (val(W["l0.wq"]) @ Y[r]).reshape(nq, d)
        k = (val(W["l0.wk"]) @ Y[r]).reshape(nkv, d)
        v = (val(W["l0.wv"]) @ Y[r]).reshape(nkv, d)
        # the appended key is rotated by its position before it is stored (one bf16 rounding apart)
        assert bf16_ulps(S["l0.kcache"][b, :, p], bits(rope64(k, p, cfg.rope_theta, d))).max() <= 1
        assert bf16_ulps(S["l0.vcache"][b, :, p], bits(v)).max() <= 1
        # nothing else of either cache moved
        mask = np.ones(S0["l0.kcache"].shape[2], bool)
        mask[p] = False
        assert np.array_equal(S["l0.kcache"][b][:, mask], S0["l0.kcache"][b][:, mask])
        assert np.array_equal(S["l0.vcache"][b][:, mask], S0["l0.vcache"][b][:, mask])
        qr = rope64(q, p, cfg.rope_theta, d)
        K, V = val(S["l0.kcache"][b]), val(S["l0.vcache"][b])
        o = np.concatenate([softmax(K[h // 2, :p + 1] @ qr[h] / math.sqrt(d)) @ V[h // 2, :p + 1] for h in range(nq)])
        ref = val(W["l0.wo"]) @ o
        assert np.allclose(out[r], ref, rtol=1e-4, atol=1e-4 * np.abs(ref).max()), r


# ---- gated delta rule layers (GDN: a decay per head; KDA: a decay per key channel) ----------------

def _linear_setup(rng, kind, H=64, h=2, dk=16, dv=8, B=1):
    cfg = SimpleNamespace(mixers=(kind,), lin_heads=h, d_k=dk, d_v=dv)
    na = h * dk if kind == "kda" else h
    W = {"l0.wq": bits(rng.standard_normal((h * dk, H)) * 0.3), "l0.wk": bits(rng.standard_normal((h * dk, H)) * 0.3),
         "l0.wv": bits(rng.standard_normal((h * dv, H)) * 0.3), "l0.wa": bits(rng.standard_normal((na, H)) * 0.3),
         "l0.wb": bits(rng.standard_normal((h, H)) * 0.3), "l0.wo": bits(rng.standard_normal((H, h * dv)) * 0.3)}
    S = {"l0.lstate": (rng.standard_normal((B, h, dv, dk)) * 0.2).astype(np.float32)}
    return cfg, W, S


def _linear64(cfg, W, S0, y):
    """One token of the gated delta rule per head, float64: q and k L2-normalised, decay
    alpha = sigmoid(-a) (= exp(-softplus(a))), write strength beta = sigmoid(b),
    S' = S Diag(alpha) (I - beta k k^T) + beta v k^T, o = S' q, output W_o o."""
    h, dk, dv = cfg.lin_heads, cfg.d_k, cfg.d_v
    Y = np.asarray(y, np.float64)
    q = (val(W["l0.wq"]) @ Y).reshape(h, dk)
    k = (val(W["l0.wk"]) @ Y).reshape(h, dk)
    v = (val(W["l0.wv"]) @ Y).reshape(h, dv)
    a = val(W["l0.wa"]) @ Y
    beta = expit(val(W["l0.wb"]) @ Y)
    alpha = expit(-a).reshape(h, -1) * np.ones((h, dk))  # a scalar per head broadcasts over the channels
    o = np.zeros((h, dv))
    S1 = np.zeros((h, dv, dk))
    for i in range(h):
        qh, kh = q[i] / np.linalg.norm(q[i]), k[i] / np.linalg.norm(k[i])
        Sd = S0[i].astype(np.float64) @ np.diag(alpha[i])
        S1[i] = Sd @ (np.eye(dk) - beta[i] * np.outer(kh, kh)) + beta[i] * np.outer(v[i], kh)
        o[i] = S1[i] @ qh
    return val(W["l0.wo"]) @ o.reshape(-1), S1


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_linear_layer_matches_float64_restatement(oracle, kind):
    rng = np.random.default_rng(33 + (kind == "kda"))
    cfg, W, S = _linear_setup(rng, kind)
    S0 = S["l0.lstate"][0].copy()
    y = rng.standard_normal((1, 64)).astype(np.float32)
    out = oracle._linear_rows(cfg, W, S, 0, y, [0], None)
    ref, S1 = _linear64(cfg, W, S0, y[0])
    assert np.allclose(S["l0.lstate"][0], S1, rtol=1e-5, atol=1e-6)
    assert np.allclose(out[0], ref, rtol=1e-5, atol=1e-5 * np.abs(ref).max())


def _one_hot_weights(h, dk, dv, H, q, k, v, a, b):
    """Weights whose products with y = e_0 are exactly the given vectors (bf16-representable entries)."""
    def col(vec, rows):
        m = np.zeros((rows, H), np.float32)
        m[:, 0] = vec
        return bits(m)
    Wo = np.zeros((H, h * dv), np.float32)
    Wo[np.arange(h * dv), np.arange(h * dv)] = 1.0  # the layer output reads o directly
    return {"l0.wq": col(q, h * dk), "l0.wk": col(k, h * dk), "l0.wv": col(v, h * dv), "l0.wa": col(a, len(a)),
            "l0.wb": col(b, h), "l0.wo": bits(Wo)}


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_linear_layer_gates_at_zero_and_one(oracle, kind):
    """Decay inputs of +40 and -40 give decays of 0 and 1 up to 4e-18 (exp(-softplus(40)) = e^-40;
    exp(-softplus(-40)) rounds to 1 in fp32), and b = 0 gives beta = 1/2 exactly. Then the update has closed
    forms: a decay of 0 forgets the state (S' = v k^T / 2), a decay of 1 keeps it
    (S' = S - (S k) k^T / 2 + v k^T / 2), per head for GDN and per key channel for KDA. q has norm 3
    and k norm 2, so a missing L2 normalisation of either shows."""
    h, dk, dv, H = 2, 8, 4, 16
    q1 = np.array([1.5, -2.0, 0.5, 0.5, 1.0, 0.5, 0.0, -1.0])  # |q| = sqrt(9) = 3
    k1 = np.array([0.0, 1.0, 1.0, 0.0, -1.0, 0.0, 1.0, 0.0])   # |k| = 2
    q = np.concatenate([q1, q1[::-1]])
    k = np.concatenate([k1, -k1])
    v = np.array([1.0, -2.0, 0.5, 3.0, -1.0, 0.25, 2.0, -0.5])
    if kind == "gdn":
        a = np.array([40.0, -40.0])                 # head 0 forgets, head 1 keeps
        keep = np.array([[0.0] * dk, [1.0] * dk])
    else:
        a = np.array([40.0, -40.0] * dk)            # alternating channels, both heads
        keep = np.tile([0.0, 1.0], (h, dk // 2))
    W = _one_hot_weights(h, dk, dv, H, q, k, v, a, np.zeros(h))
    cfg = SimpleNamespace(mixers=(kind,), lin_heads=h, d_k=dk, d_v=dv)
    rng = np.random.default_rng(35)
    S0 = rng.standard_normal((1, h, dv, dk)).astype(np.float32)
    S = {"l0.lstate": S0.copy()}
    y = np.zeros((1, H), np.float32)
    y[0, 0] = 1.0
    out = oracle._linear_rows(cfg, W, S, 0, y, [0], None)
    for i in range(h):
        kh = k[i * dk:(i + 1) * dk] / 2.0
        qh = q[i * dk:(i + 1) * dk] / 3.0
        Sk = S0[0, i].astype(np.float64) * keep[i]  # the state with the forgotten channels zeroed
        S1 = Sk - 0.5 * np.outer(Sk @ kh, kh) + 0.5 * np.outer(v[i * dv:(i + 1) * dv], kh)
        assert np.allclose(S["l0.lstate"][0, i], S1, atol=1e-6), i
        assert np.allclose(out[0, i * dv:(i + 1) * dv], S1 @ qh, atol=1e-6), i


# ---- latent attention layer -----------------------------------------------------------------------

def test_mla_layer_matches_float64_restatement(oracle):
    """Latent attention materialised per head: keys [W_uk,h c_j ; k_r,j], values W_uv,h c_j, query
    [q_nope ; rope(q_rope)], scale 1/sqrt(nope + rope). Only the last rope entries of each query head
    and of the key are rotated; the latent is stored unrotated."""
    rng = np.random.default_rng(36)
    H, h, nope, rp, rank, vd, cap, theta = 64, 3, 16, 8, 32, 12, 30, 1e4
    cfg = SimpleNamespace(mla_heads=h, nope_dim=nope, rope_dim=rp, kv_rank=rank, v_dim=vd, rope_theta=theta)
    W = {"l0.wq": bits(rng.standard_normal((h * (nope + rp), H)) * 0.2),
         "l0.wdkv": bits(rng.standard_normal((rank, H)) * 0.2), "l0.wkr": bits(rng.standard_normal((rp, H)) * 0.2),
         "l0.wuk": bits(rng.standard_normal((h * nope, rank)) * 0.3),
         "l0.wuv": bits(rng.standard_normal((h * vd, rank)) * 0.3), "l0.wo": bits(rng.standard_normal((H, h * vd)) * 0.2)}
    S = {"l0.latent": bits(rng.standard_normal((1, cap, rank + rp)))}
    y = rng.standard_normal((1, H)).astype(np.float32)
    p = 21
    out = oracle._mla_rows(cfg, W, S, 0, y, [0], [p])
    Y = y[0].astype(np.float64)
    c = val(W["l0.wdkv"]) @ Y
    kr = val(W["l0.wkr"]) @ Y
    assert bf16_ulps(S["l0.latent"][0, p, :rank], bits(c)).max() <= 1
    assert bf16_ulps(S["l0.latent"][0, p, rank:], bits(rope64(kr, p, theta, rp))).max() <= 1
    q = (val(W["l0.wq"]) @ Y).reshape(h, nope + rp)
    C = val(S["l0.latent"][0, :p + 1])
    Wk, Wv = val(W["l0.wuk"]), val(W["l0.wuv"])
    o = []
    for i in range(h):
        qh = np.concatenate([q[i, :nope], rope64(q[i, nope:], p, theta, rp)])
        keys = np.concatenate([C[:, :rank] @ Wk[i * nope:(i + 1) * nope].T, C[:, rank:]], axis=1)
        vals = C[:, :rank] @ Wv[i * vd:(i + 1) * vd].T
        o.append(softmax(keys @ qh / math.sqrt(nope + rp)) @ vals)
    ref = val(W["l0.wo"]) @ np.concatenate(o)
    assert np.allclose(out[0], ref, rtol=1e-4, atol=1e-4 * np.abs(ref).max())


# ---- per-layer composition ------------------------------------------------------------------------

def test_one_layer_step_is_prenorm_residual(oracle, synth):
    """A one-layer GDN + dense SwiGLU step with a vocabulary, restated in float64 from the embedding
    row to the logits: x1 = x + mixer(rms(x) g1), x2 = x1 + W_d(silu(W_g u) * W_u u) with
    u = rms(x1) g2, logits = W_lm (rms(x2) g_f)."""
    from dataclasses import replace
    cfg = replace(synth.CONFIGS["c1s"], n_layers=1, mixers=("gdn",), ffns=("dense",), ffn=256, vocab=300, batch=1)
    Wl = synth.LazyWeights(cfg)
    W = {n: Wl[n] for n in Wl.keys()}
    S = synth.make_states(cfg)
    S0 = S["l0.lstate"][0].copy()
    tok = np.array([123], np.int32)
    out = oracle.decode_step(cfg, W, S, {"tokens": tok}, cfg.ctx)
    x = val(W["embed"][123])
    mix, _ = _linear64(SimpleNamespace(lin_heads=cfg.lin_heads, d_k=cfg.d_k, d_v=cfg.d_v), W, S0,
                       rms64(x, W["l0.attn_norm"], cfg.eps))
    x1 = x + mix
    u = rms64(x1, W["l0.ffn_norm"], cfg.eps)
    g, up = val(W["l0.wg"]) @ u, val(W["l0.wu"]) @ u
    x2 = x1 + val(W["l0.wd"]) @ (g * expit(g) * up)
    logits = val(W["lm_head"]) @ rms64(x2, W["final_norm"], cfg.eps)
    scale = np.abs(logits).max()
    assert np.allclose(out["logits"][0], logits, rtol=1e-4, atol=1e-4 * scale)
