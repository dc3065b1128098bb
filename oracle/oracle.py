"""CPU oracle for one decode step / one speculative-verify step of a hybrid decoder stack.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py``. The product path never imports it, and it imports nothing from the product package.

The arithmetic lives in ``oracle_ops.cpp`` (fp32, sequential sums, built with g++); this file only
orders the calls the way the decoder step defines them. Sources on the pages:

* "Kimi K3's TPU megakernel: 92 layers in one Pallas call, and what 709 tokens a second measures",
  section "What a megakernel is, and what it fixes on a TPU": fusing the step into one kernel moves
  op boundaries, not arithmetic, so the reference is the plain step.
* same page, section "How it maps onto a TPU v7": per layer, a norm, the mixer (KDA or MLA chosen per
  layer index), the router with top-16 as sequential argmax passes, shared then routed experts, and
  the residual; the decode position and the linear-attention state are the step's scalar inputs.
* same page, section "What DSpark changes per step": the verifier runs an anchor plus seven drafts as
  eight rows of one sequence and emits the accepted prefix plus one bonus token; the embedding gather
  and LM head sit around the stack.
* page "TPU megakernels for Kimi K3, Qwen3.8-27B, and Muse-Spark-Open": the dense stack is a hybrid
  of gated-delta-net and grouped-query attention layers; the third model is NVFP4.

The dimensions, gate forms (L2-normalised q/k, beta = sigmoid, alpha = exp(-softplus)), initial values
and the remaining readings where the pages are silent are listed, one by one, in the repository's
design notes; each function below states the reading it takes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_ops.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib: Optional[ctypes.CDLL] = None


def build(force: bool = False) -> str:
    """Compile the oracle's C++ ops (plain -O2, OpenMP over output rows, no fused multiply-add)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["g++", "-std=c++17", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        vp, i64, i32, f32, f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
        sig = {
            "orc_bf16_to_f32": ([ctypes.c_uint16], f32),
            "orc_f32_to_bf16": ([f32], ctypes.c_uint16),
            "orc_widen_bf16": ([vp, i64, vp], None),
            "orc_round_bf16": ([vp, i64, vp], None),
            "orc_gemv_bf16": ([vp, i64, i64, vp, i32, vp], None),
            "orc_e2m1_value": ([ctypes.c_uint8], f32),
            "orc_e4m3_value": ([ctypes.c_uint8], f32),
            "orc_nvfp4_dequant_row": ([vp, vp, f32, i64, vp], None),
            "orc_gemv_nvfp4": ([vp, vp, f32, i64, i64, vp, i32, vp], None),
            "orc_rmsnorm": ([vp, vp, i32, i64, f32, vp], None),
            "orc_l2norm": ([vp, i32, i32, f32], None),
            "orc_rope": ([vp, i32, i32, i32, i32, i64, f64], None),
            "orc_attention": ([vp, i32, i32, vp, vp, i32, i64, i64, vp], None),
            "orc_sigmoid": ([f32], f32),
            "orc_softplus": ([f32], f32),
            "orc_decay_gates": ([vp, i32, vp], None),
            "orc_sigmoid_vec": ([vp, i32, vp], None),
            "orc_delta_step": ([vp, i32, i32, vp, vp, vp, vp, f32, vp], None),
            "orc_mla_attend": ([vp, i32, i32, i32, vp, vp, i32, i32, vp, i64, vp], None),
            "orc_topk": ([vp, i32, i32, vp, vp], None),
            "orc_silu_mul": ([vp, vp, i64, vp], None),
            "orc_argmax": ([vp, i64], i64),
            "orc_residual_add": ([vp, vp, i64], None),
            "orc_e8m0_value": ([ctypes.c_uint8], f32),
            "orc_mxfp4_dequant_row": ([vp, vp, i64, vp], None),
            "orc_gemv_mxfp4": ([vp, vp, i64, i64, vp, i32, vp], None),
            "orc_fp8_reencode": ([vp, vp, i64, i64, vp, vp], i64),
            "orc_gemv_fp8r": ([vp, vp, i64, i64, vp, i32, vp], None),
            "orc_moe_accumulate": ([vp, vp, f32, i64], None),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes, fn.restype = args, res
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle ops take contiguous arrays"
    return a.ctypes.data


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


# ---- thin op wrappers (numpy in, numpy out) ----------------------------------------------------

class FP8RTensor:
    """FP8 E4M3 values [N][K] with one bf16 scale per 256 consecutive elements of a row [N][K/256]."""

    def __init__(self, fp8: np.ndarray, bscale: np.ndarray):
        self.fp8, self.bscale = fp8, bscale


def fp8_reencode(W) -> FP8RTensor:
    """The loader's lossless re-encoding of an MXFP4 gate or up matrix into FP8 with a bf16 scale per 256
    (orc_fp8_reencode); raises when it is not lossless, as the loader does."""
    codes, scales = np.ascontiguousarray(W.codes), np.ascontiguousarray(W.scales)
    N, K = codes.shape[0], codes.shape[1] * 2
    fp8 = np.empty((N, K), dtype=np.uint8)
    bs = np.empty((N, K // 256), dtype=np.uint16)
    bad = lib().orc_fp8_reencode(_p(codes), _p(scales), N, K, _p(fp8), _p(bs))
    if bad:
        raise ValueError(f"FP8 re-encoding of an MXFP4 matrix is not lossless ({bad} elements differ)")
    return FP8RTensor(fp8, bs)


def gemv(W, X: np.ndarray) -> np.ndarray:
    """Y[b] = W X[b]; W is bf16 bits [N][K], an NVFP4 tensor (codes/scales/tensor_scale), an MXFP4 tensor
    (codes/scales, format "mxfp4") or an FP8 re-encoding (FP8RTensor)."""
    X = _f32(X)
    if X.ndim == 1:
        return gemv(W, X[None, :])[0]
    B, K = X.shape
    if isinstance(W, FP8RTensor):
        N = W.fp8.shape[0]
        assert W.fp8.shape[1] == K
        Y = np.empty((B, N), dtype=np.float32)
        lib().orc_gemv_fp8r(_p(W.fp8), _p(W.bscale), N, K, _p(X), B, _p(Y))
        return Y
    if getattr(W, "format", None) == "mxfp4":
        codes, scales = np.ascontiguousarray(W.codes), np.ascontiguousarray(W.scales)
        N = codes.shape[0]
        assert codes.shape[1] * 2 == K
        Y = np.empty((B, N), dtype=np.float32)
        lib().orc_gemv_mxfp4(_p(codes), _p(scales), N, K, _p(X), B, _p(Y))
        return Y
    if hasattr(W, "codes"):
        N = W.codes.shape[0]
        assert W.codes.shape[1] * 2 == K
        Y = np.empty((B, N), dtype=np.float32)
        lib().orc_gemv_nvfp4(_p(W.codes), _p(W.scales), float(W.tensor_scale), N, K, _p(X), B, _p(Y))
        return Y
    W = np.ascontiguousarray(W)
    N, K2 = W.shape
    assert K2 == K, (W.shape, X.shape)
    Y = np.empty((B, N), dtype=np.float32)
    lib().orc_gemv_bf16(_p(W), N, K, _p(X), B, _p(Y))
    return Y


def widen(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.uint16)
    out = np.empty(a.shape, dtype=np.float32)
    lib().orc_widen_bf16(_p(a), a.size, _p(out))
    return out


def round_bf16(a: np.ndarray) -> np.ndarray:
    a = _f32(a)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().orc_round_bf16(_p(a), a.size, _p(out))
    return out


def rmsnorm(X: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    X = _f32(X)
    B, H = X.shape
    Y = np.empty_like(X)
    g = np.ascontiguousarray(g, dtype=np.uint16)  # keep every temporary alive across the call
    lib().orc_rmsnorm(_p(X), _p(g), B, H, eps, _p(Y))
    return Y


def l2norm(v: np.ndarray, d: int, eps: float = 1e-6) -> np.ndarray:
    v = _f32(v).copy()
    lib().orc_l2norm(_p(v), v.size // d, d, eps)
    return v


def rope(v: np.ndarray, n_vec: int, stride: int, offset: int, rot: int, pos: int, theta: float) -> np.ndarray:
    v = _f32(v).copy()
    lib().orc_rope(_p(v), n_vec, stride, offset, rot, int(pos), float(theta))
    return v


def attention(q: np.ndarray, nq: int, d: int, kc: np.ndarray, vc: np.ndarray, L: int) -> np.ndarray:
    """q [nq*d]; kc/vc one sequence's caches [nkv][cap][d] bf16; attend positions 0..L-1."""
    q = _f32(q)
    nkv, cap, d2 = kc.shape
    assert d2 == d and L <= cap
    o = np.empty(nq * d, dtype=np.float32)
    kc, vc = np.ascontiguousarray(kc), np.ascontiguousarray(vc)
    lib().orc_attention(_p(q), nq, d, _p(kc), _p(vc), nkv, cap * d, L, _p(o))
    return o


def decay_gates(a: np.ndarray) -> np.ndarray:
    a = _f32(a)
    out = np.empty_like(a)
    lib().orc_decay_gates(_p(a), a.size, _p(out))
    return out


def sigmoid(z: np.ndarray) -> np.ndarray:
    z = _f32(z)
    out = np.empty_like(z)
    lib().orc_sigmoid_vec(_p(z), z.size, _p(out))
    return out


def delta_step(S: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray, alpha: np.ndarray, beta: float) -> np.ndarray:
    """One gated-delta-rule update of state S [dv][dk] (in place); returns o [dv]."""
    assert S.dtype == np.float32 and S.flags["C_CONTIGUOUS"]
    dv, dk = S.shape
    o = np.empty(dv, dtype=np.float32)
    q, k, v, alpha = _f32(q), _f32(k), _f32(v), _f32(alpha)  # keep every temporary alive across the call
    lib().orc_delta_step(_p(S), dk, dv, _p(q), _p(k), _p(v), _p(alpha), float(beta), _p(o))
    return o


def mla_attend(q: np.ndarray, heads: int, nope: int, rope_d: int, wuk: np.ndarray, wuv: np.ndarray, rank: int,
               vdim: int, cache: np.ndarray, L: int) -> np.ndarray:
    out = np.empty(heads * vdim, dtype=np.float32)
    q, wuk, wuv, cache = _f32(q), np.ascontiguousarray(wuk), np.ascontiguousarray(wuv), np.ascontiguousarray(cache)
    lib().orc_mla_attend(_p(q), heads, nope, rope_d, _p(wuk), _p(wuv), rank, vdim, _p(cache), L, _p(out))
    return out


def topk(z: np.ndarray, k: int):
    z = _f32(z)
    idx = np.empty(k, dtype=np.int32)
    g = np.empty(k, dtype=np.float32)
    lib().orc_topk(_p(z), z.size, k, _p(idx), _p(g))
    return idx, g


def silu_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g, u = _f32(g), _f32(u)
    h = np.empty_like(g)
    lib().orc_silu_mul(_p(g), _p(u), g.size, _p(h))
    return h


def residual_add(x: np.ndarray, o: np.ndarray) -> np.ndarray:
    """x + o, elementwise in fp32 (a new array)."""
    out = _f32(x).copy()
    o = _f32(o)
    assert out.shape == o.shape
    lib().orc_residual_add(_p(out), _p(o), out.size)
    return out


def moe_accumulate(acc: np.ndarray, y: np.ndarray, w: float) -> None:
    """acc += w * y in place (acc fp32, contiguous)."""
    assert acc.dtype == np.float32 and acc.flags["C_CONTIGUOUS"]
    y = _f32(y)
    assert acc.shape == y.shape
    lib().orc_moe_accumulate(_p(acc), _p(y), float(w), acc.size)


def argmax(x: np.ndarray) -> int:
    x = _f32(x)
    return int(lib().orc_argmax(_p(x), x.size))


# ---- the step ----------------------------------------------------------------------------------

def _swiglu(W, pre: str, y: np.ndarray, reencoded: Optional[dict] = None) -> np.ndarray:
    """SwiGLU FFN: W_d (silu(W_g y) * (W_u y)). MXFP4 experts take gate and up through their FP8
    re-encoding and down as MXFP4 (page "Kimi K3's TPU megakernel ...", section "How it maps onto a TPU
    v7", the precision paragraph); `reencoded` caches the re-encodings within one FFN evaluation."""
    wg, wu = W[pre + "wg"], W[pre + "wu"]
    if getattr(wg, "format", None) == "mxfp4":
        if reencoded is None:
            reencoded = {}
        key = (id(wg), id(wu))  # the entry keeps both sources alive, so their identities stay unique
        if key not in reencoded:
            reencoded[key] = (wg, wu, fp8_reencode(wg), fp8_reencode(wu))
        wg, wu = reencoded[key][2:]
    g = gemv(wg, y)
    u = gemv(wu, y)
    return gemv(W[pre + "wd"], silu_mul(g, u))


def _ffn(cfg, W, l: int, y: np.ndarray, route_log: Optional[dict]) -> np.ndarray:
    if cfg.ffns[l] == "dense":
        return _swiglu(W, f"l{l}.", y)
    # Mixture of experts: shared expert(s) with weight 1 plus the top-k routed experts weighted by
    # their normalised sigmoid scores (page "Kimi K3's TPU megakernel ...", section "How it maps onto
    # a TPU v7": router, then shared expert, then routed experts).
    B = y.shape[0]
    z = gemv(W[f"l{l}.router"], y)
    out = np.zeros_like(y)
    idxs = np.empty((B, cfg.top_k), dtype=np.int32)
    gws = np.empty((B, cfg.top_k), dtype=np.float32)
    reencoded: dict = {}
    for b in range(B):
        idx, gw = topk(z[b], cfg.top_k)
        idxs[b], gws[b] = idx, gw
        acc = np.zeros(cfg.hidden, dtype=np.float32)
        for s in range(cfg.n_shared):
            moe_accumulate(acc, _swiglu(W, f"l{l}.s{s}.", y[b], reencoded), 1.0)
        for t in range(cfg.top_k):
            moe_accumulate(acc, _swiglu(W, f"l{l}.e{int(idx[t])}.", y[b], reencoded), float(gw[t]))
        out[b] = acc
    if route_log is not None:
        route_log[l] = (idxs, gws, z, y)  # y: the router's input, for the callers' rounding bounds
    return out


def _gqa_rows(cfg, W, S, l: int, y: np.ndarray, b_of_row: List[int], pos_of_row: List[int]) -> np.ndarray:
    """Grouped-query attention for a set of rows; row r belongs to sequence b_of_row[r] and sits at
    position pos_of_row[r]. Every row's rotated k and bf16-rounded k, v are appended first; row r then
    attends to its own sequence's positions 0..pos_of_row[r] (so a new token sees itself, and within a
    verify block row j sees rows 0..j)."""
    hq, hk, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    q = gemv(W[f"l{l}.wq"], y)
    k = gemv(W[f"l{l}.wk"], y)
    v = gemv(W[f"l{l}.wv"], y)
    kc, vc = S[f"l{l}.kcache"], S[f"l{l}.vcache"]
    R = y.shape[0]
    qr = np.empty_like(q)
    for r in range(R):
        b, p = b_of_row[r], pos_of_row[r]
        qr[r] = rope(q[r], hq, d, 0, d, p, cfg.rope_theta)
        kr = rope(k[r], hk, d, 0, d, p, cfg.rope_theta)
        kc[b, :, p, :] = round_bf16(kr).reshape(hk, d)
        vc[b, :, p, :] = round_bf16(v[r]).reshape(hk, d)
    att = np.empty((R, hq * d), dtype=np.float32)
    for r in range(R):
        b, p = b_of_row[r], pos_of_row[r]
        att[r] = attention(qr[r], hq, d, kc[b], vc[b], p + 1)
    return gemv(W[f"l{l}.wo"], att)


def _linear_rows(cfg, W, S, l: int, y: np.ndarray, b_of_row: List[int], snapshots: Optional[list]) -> np.ndarray:
    """Gated delta rule (scalar gate per head for GDN, per-channel gate for KDA). Rows are processed in
    order, so rows of one sequence advance its state one token at a time; after each row the state is
    recorded when ``snapshots`` is given."""
    kda = cfg.mixers[l] == "kda"
    h, dk, dv = cfg.lin_heads, cfg.d_k, cfg.d_v
    q = gemv(W[f"l{l}.wq"], y)
    k = gemv(W[f"l{l}.wk"], y)
    v = gemv(W[f"l{l}.wv"], y)
    a = gemv(W[f"l{l}.wa"], y)
    bg = gemv(W[f"l{l}.wb"], y)
    st = S[f"l{l}.lstate"]
    R = y.shape[0]
    o = np.empty((R, h * dv), dtype=np.float32)
    for r in range(R):
        b = b_of_row[r]
        qh = l2norm(q[r], dk)
        kh = l2norm(k[r], dk)
        alpha = decay_gates(a[r])
        beta = sigmoid(bg[r])
        for hh in range(h):
            al = alpha[hh * dk:(hh + 1) * dk] if kda else np.full(dk, alpha[hh], dtype=np.float32)
            Sh = st[b, hh]
            o[r, hh * dv:(hh + 1) * dv] = delta_step(Sh, qh[hh * dk:(hh + 1) * dk], kh[hh * dk:(hh + 1) * dk],
                                                     v[r, hh * dv:(hh + 1) * dv], al, float(beta[hh]))
        if snapshots is not None:
            snapshots.append(st.copy())
    return gemv(W[f"l{l}.wo"], o)


def _mla_rows(cfg, W, S, l: int, y: np.ndarray, b_of_row: List[int], pos_of_row: List[int]) -> np.ndarray:
    """Multi-head latent attention in its absorbed decode form over a [c | k_rope] latent cache."""
    h, nope, rp, rank, vd = cfg.mla_heads, cfg.nope_dim, cfg.rope_dim, cfg.kv_rank, cfg.v_dim
    q = gemv(W[f"l{l}.wq"], y)
    c = gemv(W[f"l{l}.wdkv"], y)
    kr = gemv(W[f"l{l}.wkr"], y)
    cache = S[f"l{l}.latent"]
    R = y.shape[0]
    qr = np.empty_like(q)
    for r in range(R):
        b, p = b_of_row[r], pos_of_row[r]
        qr[r] = rope(q[r], h, nope + rp, nope, rp, p, cfg.rope_theta)
        krr = rope(kr[r], 1, rp, 0, rp, p, cfg.rope_theta)
        cache[b, p, :rank] = round_bf16(c[r])
        cache[b, p, rank:] = round_bf16(krr)
    att = np.empty((R, h * vd), dtype=np.float32)
    for r in range(R):
        b, p = b_of_row[r], pos_of_row[r]
        att[r] = mla_attend(qr[r], h, nope, rp, W[f"l{l}.wuk"], W[f"l{l}.wuv"], rank, vd, cache[b], p + 1)
    return gemv(W[f"l{l}.wo"], att)


def _stack(cfg, W, S, x: np.ndarray, b_of_row, pos_of_row, snapshots=None, route_log=None) -> np.ndarray:
    """Run all layers over the residual rows x [R][H] (pre-norm residual blocks)."""
    for l in range(cfg.n_layers):
        y = rmsnorm(x, W[f"l{l}.attn_norm"], cfg.eps)
        mx = cfg.mixers[l]
        if mx == "gqa":
            o = _gqa_rows(cfg, W, S, l, y, b_of_row, pos_of_row)
        elif mx in ("gdn", "kda"):
            snaps = [] if snapshots is not None else None
            o = _linear_rows(cfg, W, S, l, y, b_of_row, snaps)
            if snapshots is not None:
                snapshots[l] = snaps
        elif mx == "mla":
            o = _mla_rows(cfg, W, S, l, y, b_of_row, pos_of_row)
        else:
            raise ValueError(mx)
        x = residual_add(x, o)
        y = rmsnorm(x, W[f"l{l}.ffn_norm"], cfg.eps)
        x = residual_add(x, _ffn(cfg, W, l, y, route_log))
    return x


def embed(W, tokens: np.ndarray) -> np.ndarray:
    E = W["embed"]
    return widen(np.ascontiguousarray(E[np.asarray(tokens, dtype=np.int64)]))


def decode_step(cfg, W, S: Dict[str, np.ndarray], inputs: Dict[str, np.ndarray], pos) -> dict:
    """One decode step for ``cfg.batch`` sequences at position ``pos`` (one int for all, or one per
    sequence). Caches and recurrent states in ``S`` are updated in place. Returns logits and their argmax
    (vocabulary configs) or the final hidden state (slice configs), plus per-layer routing for MoE
    layers."""
    B = cfg.batch
    positions = [int(p) for p in pos] if np.ndim(pos) else [int(pos)] * B
    assert len(positions) == B
    if cfg.vocab:
        x = embed(W, inputs["tokens"])
    else:
        x = _f32(inputs["hidden_in"]).copy()
    route_log: dict = {}
    x = _stack(cfg, W, S, x, list(range(B)), positions, route_log=route_log)
    out = {"routes": route_log}
    if cfg.vocab:
        y = rmsnorm(x, W["final_norm"], cfg.eps)
        logits = gemv(W["lm_head"], y)
        out["logits"] = logits
        out["final_y"] = y  # the LM head's input, for the callers' rounding bounds
        out["argmax"] = np.array([argmax(logits[b]) for b in range(B)], dtype=np.int32)
    else:
        out["hidden_out"] = x
    return out


def verify_step(cfg, W, S: Dict[str, np.ndarray], tokens: np.ndarray, pos: int) -> dict:
    """Speculative verify of one sequence: rows j = 0..R-1 hold [anchor, d_1 .. d_{R-1}] at positions
    pos..pos+R-1, evaluated as one block (all rows through a layer before the next layer). Returns the
    R x vocab logits, per-row argmax, the accepted count a (longest prefix with d_{j+1} == argmax of
    row j), the bonus token argmax(row a), and the per-row linear-state snapshots. Caches hold all R
    appended rows; each linear-attention state is committed to the snapshot after row a."""
    assert cfg.batch == 1 and cfg.vocab
    tokens = np.asarray(tokens, dtype=np.int32)
    R = tokens.shape[0]
    x = embed(W, tokens)
    snapshots: dict = {}
    x = _stack(cfg, W, S, x, [0] * R, [pos + j for j in range(R)], snapshots=snapshots)
    y = rmsnorm(x, W["final_norm"], cfg.eps)
    logits = gemv(W["lm_head"], y)
    am = np.array([argmax(logits[j]) for j in range(R)], dtype=np.int32)
    a = 0
    while a < R - 1 and int(tokens[a + 1]) == int(am[a]):
        a += 1
    for l, snaps in snapshots.items():
        S[f"l{l}.lstate"][...] = snaps[a]
    return {"logits": logits, "argmax": am, "accepted": a, "bonus": int(am[a]), "snapshots": snapshots, "final_y": y}


def copy_states(S: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    return {k: v.copy() for k, v in S.items()}
