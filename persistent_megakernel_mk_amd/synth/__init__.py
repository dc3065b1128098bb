"""Seeded synthetic workloads for the decode-step megakernel: shapes, tensor lists and generators.

This module defines *inputs only* (model dimensions, random weights, caches, recurrent states and
tokens). It contains none of the decoder's arithmetic; both the CPU oracle (via the test harness)
and the HIP path consume the arrays it produces.

Workloads follow the decode problem statement of the TPU-megakernel pages (one small-batch decode
step, or one 8-row speculative verify step, over a whole hybrid decoder stack). The dimensions are
those of the five named configurations:

* ``c0``  tiny dense decode: 2 GQA layers, hidden 256, 4 q / 2 kv heads of 64, SwiGLU 1024, vocab 1024,
          KV cache of 128 positions, batch 1.
* ``c1``  hybrid 27B-class dense stack: 64 layers, 3 GDN : 1 GQA, hidden 5120, SwiGLU 17408,
          vocab 151936, GDN 16 heads of 128, GQA 24 q / 4 kv heads of 128, KV 4096, batch 1/2/4/8.
* ``c2``  8-row speculative verify on the ``c1`` stack (anchor + 7 drafts).
* ``c3``  Kimi-style MoE slice: 4 layers 3 KDA : 1 MLA, hidden 7168, 384 experts of 2048, top-8
          + 1 shared, batch 8.
* ``c4``  NVFP4 MoE decode: 8 GQA layers, hidden 6144, 256 experts of 2048, top-8 + 1 shared,
          48 q / 8 kv heads, KV 2048, batch 1/4/8.

Smaller variants with the same structure (``*s`` names) serve as parity cases that the oracle
finishes in seconds while still spanning many tiles and ragged tails.
"""
from __future__ import annotations

import ctypes
import os
import zlib
from dataclasses import dataclass, field, replace
from typing import Dict, Iterator, List, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmksynth.so")
_GPU_LIB_PATH = os.path.join(_HERE, "libmksynth_gpu.so")

# ----------------------------------------------------------------------------------------------
# configurations
# ----------------------------------------------------------------------------------------------


@dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    hidden: int
    vocab: int  # 0: slice mode (hidden state in, hidden state out)
    mixers: Tuple[str, ...]  # per layer: "gqa" | "gdn" | "kda" | "mla"
    ffns: Tuple[str, ...]  # per layer: "dense" | "moe"
    ffn: int = 0
    n_q_heads: int = 0
    n_kv_heads: int = 0
    head_dim: int = 0
    lin_heads: int = 0
    d_k: int = 0
    d_v: int = 0
    mla_heads: int = 0
    kv_rank: int = 0
    rope_dim: int = 0
    nope_dim: int = 0
    v_dim: int = 0
    n_experts: int = 0
    top_k: int = 0
    expert_ffn: int = 0
    n_shared: int = 0
    expert_format: str = "bf16"  # "bf16" | "nvfp4" | "mxfp4" (gate/up re-encoded to FP8 when loaded)
    ctx: int = 0  # cached positions 0..ctx-1; the new token sits at position ctx
    batch: int = 1
    eps: float = 1e-6
    rope_theta: float = 1e6
    seed: int = 1000
    verify_rows: int = 0  # 0: decode step; 8: speculative verify (anchor + 7 drafts)

    @property
    def max_ctx(self) -> int:
        """Cache capacity: the cached positions plus room for an 8-row verify block."""
        return self.ctx + 8

    def with_batch(self, b: int) -> "ModelConfig":
        return replace(self, batch=b)


def _pattern(n: int, every: int, other: str, base: str) -> Tuple[str, ...]:
    """Layer index l uses ``other`` when l % every == every - 1, else ``base``."""
    return tuple(other if (l % every) == every - 1 else base for l in range(n))


CONFIGS: Dict[str, ModelConfig] = {}


def _reg(c: ModelConfig) -> None:
    CONFIGS[c.name] = c


_reg(ModelConfig(name="c0", n_layers=2, hidden=256, vocab=1024, mixers=("gqa", "gqa"), ffns=("dense", "dense"),
                 ffn=1024, n_q_heads=4, n_kv_heads=2, head_dim=64, ctx=128, batch=1, seed=1000))
_reg(ModelConfig(name="c1", n_layers=64, hidden=5120, vocab=151936, mixers=_pattern(64, 4, "gqa", "gdn"),
                 ffns=("dense",) * 64, ffn=17408, n_q_heads=24, n_kv_heads=4, head_dim=128, lin_heads=16,
                 d_k=128, d_v=128, ctx=4096, batch=1, seed=1001))
_reg(replace(CONFIGS["c1"], name="c2", verify_rows=8, seed=1002))
_reg(ModelConfig(name="c3", n_layers=4, hidden=7168, vocab=0, mixers=_pattern(4, 4, "mla", "kda"),
                 ffns=("moe",) * 4, lin_heads=32, d_k=128, d_v=128, mla_heads=64, kv_rank=512, rope_dim=64,
                 nope_dim=128, v_dim=128, n_experts=384, top_k=8, expert_ffn=2048, n_shared=1, ctx=4096,
                 batch=8, seed=1003))
_reg(ModelConfig(name="c4", n_layers=8, hidden=6144, vocab=0, mixers=("gqa",) * 8, ffns=("moe",) * 8,
                 n_q_heads=48, n_kv_heads=8, head_dim=128, n_experts=256, top_k=8, expert_ffn=2048, n_shared=1,
                 expert_format="nvfp4", ctx=2048, batch=1, seed=1004))
# small structural variants (parity cases): ragged multiples of the 16-row tile and 256-column block
_reg(ModelConfig(name="c1s", n_layers=4, hidden=1280, vocab=4000, mixers=_pattern(4, 4, "gqa", "gdn"),
                 ffns=("dense",) * 4, ffn=3328, n_q_heads=6, n_kv_heads=2, head_dim=128, lin_heads=4, d_k=128,
                 d_v=128, ctx=300, batch=1, seed=2001))
_reg(replace(CONFIGS["c1s"], name="c2s", verify_rows=8, seed=2002))
_reg(ModelConfig(name="c3s", n_layers=4, hidden=1024, vocab=0, mixers=_pattern(4, 4, "mla", "kda"),
                 ffns=("moe",) * 4, lin_heads=4, d_k=128, d_v=128, mla_heads=4, kv_rank=512, rope_dim=64,
                 nope_dim=128, v_dim=128, n_experts=24, top_k=4, expert_ffn=512, n_shared=1, ctx=200, batch=8,
                 seed=2003))
# variants that isolate one part of the path: Kimi delta attention with dense FFNs, and the NVFP4
# mixture-of-experts slice with bf16 experts
_reg(replace(CONFIGS["c1s"], name="c1s_kda", mixers=_pattern(4, 4, "gqa", "kda"), seed=2005))
# latent attention with dense FFNs and a vocabulary (decode and verify)
_reg(replace(CONFIGS["c1s"], name="c1s_mla", mixers=_pattern(4, 4, "mla", "gdn"), mla_heads=12, kv_rank=256,
             rope_dim=64, nope_dim=128, v_dim=64, seed=2007))
_reg(ModelConfig(name="c4s", n_layers=2, hidden=1024, vocab=0, mixers=("gqa",) * 2, ffns=("moe",) * 2,
                 n_q_heads=8, n_kv_heads=2, head_dim=128, n_experts=16, top_k=4, expert_ffn=512, n_shared=1,
                 expert_format="nvfp4", ctx=160, batch=4, seed=2004))


# ----------------------------------------------------------------------------------------------
# tensor list
# ----------------------------------------------------------------------------------------------


@dataclass(frozen=True)
class TensorSpec:
    name: str
    shape: Tuple[int, ...]
    kind: str  # "bf16" | "f32" | "nvfp4" | "mxfp4" | "i32"
    sigma: float = 0.0
    mean: float = 0.0
    valid_positions: int = -1  # caches: positions >= this are zero
    group: str = "weight"  # "weight" | "state" | "input"

    @property
    def tid(self) -> int:
        return zlib.crc32(self.name.encode())

    @property
    def numel(self) -> int:
        n = 1
        for s in self.shape:
            n *= s
        return n


W_SIGMA = 0.02  # matrices ~ N(0, 0.02)
NORM_SIGMA = 0.02  # RMSNorm gains 1 + N(0, 0.02)
CACHE_SIGMA = 1.0  # KV / latent caches ~ N(0, 1)
STATE_SIGMA = 0.1  # recurrent states ~ N(0, 0.1)


def layer_weight_specs(cfg: ModelConfig, l: int) -> List[TensorSpec]:
    H = cfg.hidden
    out: List[TensorSpec] = [
        TensorSpec(f"l{l}.attn_norm", (H,), "bf16", NORM_SIGMA, 1.0),
        TensorSpec(f"l{l}.ffn_norm", (H,), "bf16", NORM_SIGMA, 1.0),
    ]
    mx = cfg.mixers[l]
    w = lambda n, r, c: TensorSpec(f"l{l}.{n}", (r, c), "bf16", W_SIGMA)  # noqa: E731
    if mx == "gqa":
        hq, hk, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
        out += [w("wq", hq * d, H), w("wk", hk * d, H), w("wv", hk * d, H), w("wo", H, hq * d)]
    elif mx in ("gdn", "kda"):
        h, dk, dv = cfg.lin_heads, cfg.d_k, cfg.d_v
        na = h if mx == "gdn" else h * dk
        out += [w("wq", h * dk, H), w("wk", h * dk, H), w("wv", h * dv, H), w("wa", na, H), w("wb", h, H),
                w("wo", H, h * dv)]
    elif mx == "mla":
        h = cfg.mla_heads
        out += [w("wq", h * (cfg.nope_dim + cfg.rope_dim), H), w("wdkv", cfg.kv_rank, H), w("wkr", cfg.rope_dim, H),
                w("wuk", h * cfg.nope_dim, cfg.kv_rank), w("wuv", h * cfg.v_dim, cfg.kv_rank),
                w("wo", H, h * cfg.v_dim)]
    else:
        raise ValueError(mx)
    if cfg.ffns[l] == "dense":
        F = cfg.ffn
        out += [w("wg", F, H), w("wu", F, H), w("wd", H, F)]
    else:
        F = cfg.expert_ffn
        kind = cfg.expert_format
        out.append(w("router", cfg.n_experts, H))
        for s in range(cfg.n_shared):
            out += [TensorSpec(f"l{l}.s{s}.wg", (F, H), kind, W_SIGMA), TensorSpec(f"l{l}.s{s}.wu", (F, H), kind, W_SIGMA),
                    TensorSpec(f"l{l}.s{s}.wd", (H, F), kind, W_SIGMA)]
        for e in range(cfg.n_experts):
            out += [TensorSpec(f"l{l}.e{e}.wg", (F, H), kind, W_SIGMA), TensorSpec(f"l{l}.e{e}.wu", (F, H), kind, W_SIGMA),
                    TensorSpec(f"l{l}.e{e}.wd", (H, F), kind, W_SIGMA)]
    return out


def weight_specs(cfg: ModelConfig) -> List[TensorSpec]:
    out: List[TensorSpec] = []
    if cfg.vocab:
        out.append(TensorSpec("embed", (cfg.vocab, cfg.hidden), "bf16", W_SIGMA))
    for l in range(cfg.n_layers):
        out += layer_weight_specs(cfg, l)
    if cfg.vocab:
        out.append(TensorSpec("final_norm", (cfg.hidden,), "bf16", NORM_SIGMA, 1.0))
        out.append(TensorSpec("lm_head", (cfg.vocab, cfg.hidden), "bf16", W_SIGMA))
    return out


def state_specs(cfg: ModelConfig) -> List[TensorSpec]:
    B, out = cfg.batch, []
    for l in range(cfg.n_layers):
        mx = cfg.mixers[l]
        if mx == "gqa":
            shp = (B, cfg.n_kv_heads, cfg.max_ctx, cfg.head_dim)
            out.append(TensorSpec(f"l{l}.kcache", shp, "bf16", CACHE_SIGMA, valid_positions=cfg.ctx, group="state"))
            out.append(TensorSpec(f"l{l}.vcache", shp, "bf16", CACHE_SIGMA, valid_positions=cfg.ctx, group="state"))
        elif mx in ("gdn", "kda"):
            out.append(TensorSpec(f"l{l}.lstate", (B, cfg.lin_heads, cfg.d_v, cfg.d_k), "f32", STATE_SIGMA,
                                  group="state"))
        elif mx == "mla":
            out.append(TensorSpec(f"l{l}.latent", (B, cfg.max_ctx, cfg.kv_rank + cfg.rope_dim), "bf16", CACHE_SIGMA,
                                  valid_positions=cfg.ctx, group="state"))
    return out


def input_specs(cfg: ModelConfig) -> List[TensorSpec]:
    if cfg.vocab:
        return [TensorSpec("tokens", (cfg.batch,), "i32", group="input")]
    return [TensorSpec("hidden_in", (cfg.batch, cfg.hidden), "f32", 1.0, group="input")]


# ----------------------------------------------------------------------------------------------
# host generator (ctypes over libmksynth.so)
# ----------------------------------------------------------------------------------------------

_lib: Optional[ctypes.CDLL] = None


def build_host_lib(force: bool = False) -> str:
    """Compile the host generator (gcc, OpenMP, no fused multiply-add)."""
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        import subprocess

        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-o", tmp, src,
                               "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_gpu_lib() -> str:
    """Compile the device generator (hipcc, gfx950)."""
    import subprocess

    src = os.path.join(_HERE, "synth_gpu.hip")
    tmp = _GPU_LIB_PATH + ".tmp"
    subprocess.check_call(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-ffp-contract=off",
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", tmp, src],
                          stderr=subprocess.DEVNULL)
    os.replace(tmp, _GPU_LIB_PATH)
    return _GPU_LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_host_lib()
        L = ctypes.CDLL(_LIB_PATH)
        u64, i64, f32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
        L.synth_key.argtypes, L.synth_key.restype = [u64, u64], u64
        L.synth_normal_bf16.argtypes = [u64, u64, u64, i64, f32, f32, vp]
        L.synth_normal_f32.argtypes = [u64, u64, u64, i64, f32, f32, vp]
        L.synth_uniform_int.argtypes = [u64, u64, u64, i64, ctypes.c_uint32, vp]
        L.synth_nvfp4_encode.argtypes = [vp, i64, i64, vp, vp, vp]
        L.synth_mxfp4_encode.argtypes = [vp, i64, i64, vp, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def normal_bf16(seed: int, tid: int, n: int, sigma: float, mean: float = 0.0, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    lib().synth_normal_bf16(seed, tid, offset, n, sigma, mean, _ptr(out))
    return out


def normal_f32(seed: int, tid: int, n: int, sigma: float, mean: float = 0.0, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    lib().synth_normal_f32(seed, tid, offset, n, sigma, mean, _ptr(out))
    return out


def uniform_int(seed: int, tid: int, n: int, bound: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    lib().synth_uniform_int(seed, tid, offset, n, bound, _ptr(out))
    return out


@dataclass
class NVFP4Tensor:
    """FP4 E2M1 codes [rows][k/2] (element 2i low nibble), E4M3 scales [rows][k/16], fp32 tensor scale."""
    codes: np.ndarray
    scales: np.ndarray
    tensor_scale: float

    @property
    def shape(self) -> Tuple[int, int]:
        return (self.codes.shape[0], self.codes.shape[1] * 2)


def nvfp4_encode(w: np.ndarray) -> NVFP4Tensor:
    rows, k = w.shape
    assert k % 16 == 0
    w = np.ascontiguousarray(w, dtype=np.float32)
    codes = np.empty((rows, k // 2), dtype=np.uint8)
    scales = np.empty((rows, k // 16), dtype=np.uint8)
    ts = np.zeros(1, dtype=np.float32)
    lib().synth_nvfp4_encode(_ptr(w), rows, k, _ptr(codes), _ptr(scales), _ptr(ts))
    return NVFP4Tensor(codes, scales, float(ts[0]))


@dataclass
class MXFP4Tensor:
    """MXFP4: FP4 E2M1 codes [rows][k/2] (element 2i low nibble), E8M0 scales [rows][k/32]."""
    codes: np.ndarray
    scales: np.ndarray
    format: str = "mxfp4"

    @property
    def shape(self) -> Tuple[int, int]:
        return (self.codes.shape[0], self.codes.shape[1] * 2)


def mxfp4_encode(w: np.ndarray) -> MXFP4Tensor:
    rows, k = w.shape
    assert k % 32 == 0
    w = np.ascontiguousarray(w, dtype=np.float32)
    codes = np.empty((rows, k // 2), dtype=np.uint8)
    scales = np.empty((rows, k // 32), dtype=np.uint8)
    lib().synth_mxfp4_encode(_ptr(w), rows, k, _ptr(codes), _ptr(scales))
    return MXFP4Tensor(codes, scales)


def generate(spec: TensorSpec, seed: int):
    """Materialise one tensor on the host as numpy (bf16 as uint16 bits)."""
    if spec.kind == "bf16":
        a = normal_bf16(seed, spec.tid, spec.numel, spec.sigma, spec.mean).reshape(spec.shape)
        if spec.valid_positions >= 0:
            _zero_invalid_positions(a, spec)
        return a
    if spec.kind == "f32":
        return normal_f32(seed, spec.tid, spec.numel, spec.sigma, spec.mean).reshape(spec.shape)
    if spec.kind == "nvfp4":
        w = normal_f32(seed, spec.tid, spec.numel, spec.sigma, spec.mean).reshape(spec.shape)
        return nvfp4_encode(w)
    if spec.kind == "mxfp4":
        w = normal_f32(seed, spec.tid, spec.numel, spec.sigma, spec.mean).reshape(spec.shape)
        return mxfp4_encode(w)
    raise ValueError(spec.kind)


def _zero_invalid_positions(a: np.ndarray, spec: TensorSpec) -> None:
    vp = spec.valid_positions
    if spec.name.endswith("latent"):
        a[:, vp:, :] = 0
    else:
        a[:, :, vp:, :] = 0


class LazyWeights:
    """Mapping name -> host array that generates each tensor on first access (and caches it unless
    ``cache=False``). Lets the oracle touch only the experts a step routes to."""

    def __init__(self, cfg: ModelConfig, cache: bool = True):
        self.cfg = cfg
        self.specs = {s.name: s for s in weight_specs(cfg)}
        self._cache: Dict[str, object] = {}
        self._keep = cache

    def __getitem__(self, name: str):
        if name in self._cache:
            return self._cache[name]
        a = generate(self.specs[name], self.cfg.seed)
        if self._keep:
            self._cache[name] = a
        return a

    def __contains__(self, name: str) -> bool:
        return name in self.specs

    def keys(self):
        return self.specs.keys()


def make_states(cfg: ModelConfig) -> Dict[str, np.ndarray]:
    return {s.name: generate(s, cfg.seed) for s in state_specs(cfg)}


def make_inputs(cfg: ModelConfig, step: int = 0) -> Dict[str, np.ndarray]:
    """Tokens uniform in [0, vocab) or hidden states ~N(0,1); ``step`` selects an independent draw."""
    out = {}
    for s in input_specs(cfg):
        tid = s.tid + 7919 * step
        if s.kind == "i32":
            out[s.name] = uniform_int(cfg.seed, tid, s.numel, cfg.vocab).reshape(s.shape)
        else:
            out[s.name] = normal_f32(cfg.seed, tid, s.numel, s.sigma).reshape(s.shape)
    return out


# ----------------------------------------------------------------------------------------------
# device generator (same values, generated in device memory; libmksynth_gpu.so)
# ----------------------------------------------------------------------------------------------

_gpu_lib: Optional[ctypes.CDLL] = None


def gpu_lib() -> ctypes.CDLL:
    global _gpu_lib
    if _gpu_lib is None:
        if not os.path.exists(_GPU_LIB_PATH):
            raise RuntimeError(f"{_GPU_LIB_PATH} is not built (persistent_megakernel_mk_amd/build.py)")
        L = ctypes.CDLL(_GPU_LIB_PATH)
        u64, i64, f32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
        L.synth_gpu_normal_bf16.argtypes = [u64, u64, i64, f32, f32, i64, i64, i64, vp, vp]
        L.synth_gpu_normal_bf16.restype = ctypes.c_int
        L.synth_gpu_normal_f32.argtypes = [u64, u64, i64, f32, f32, vp, vp]
        L.synth_gpu_normal_f32.restype = ctypes.c_int
        _gpu_lib = L
    return _gpu_lib


def generate_gpu(spec: TensorSpec, seed: int, device="cuda"):
    """Materialise one bf16/f32 tensor directly in device memory (torch), bit-identical to generate()."""
    import torch

    key = lib().synth_key(seed, spec.tid)
    stream = torch.cuda.current_stream(device).cuda_stream
    if spec.kind == "bf16":
        out = torch.empty(spec.shape, dtype=torch.bfloat16, device=device)
        inner = positions = 1
        valid = -1
        if spec.valid_positions >= 0:
            if spec.name.endswith("latent"):
                inner, positions = spec.shape[2], spec.shape[1]
            else:
                inner, positions = spec.shape[3], spec.shape[2]
            valid = spec.valid_positions
        rc = gpu_lib().synth_gpu_normal_bf16(key, 0, spec.numel, spec.sigma, spec.mean, inner, positions, valid,
                                             out.data_ptr(), stream)
    elif spec.kind == "f32":
        out = torch.empty(spec.shape, dtype=torch.float32, device=device)
        rc = gpu_lib().synth_gpu_normal_f32(key, 0, spec.numel, spec.sigma, spec.mean, out.data_ptr(), stream)
    else:
        raise ValueError(f"device generation of {spec.kind} is not provided")
    if rc != 0:
        raise RuntimeError(f"device generator launch failed ({rc})")
    return out


def draft_uniforms(cfg: ModelConfig, n: int) -> np.ndarray:
    """Uniform [0,1) draws (24-bit) used to build seeded speculative drafts."""
    tid = zlib.crc32(b"drafts")
    r = uniform_int(cfg.seed, tid, n, 1 << 24)
    return r.astype(np.float64) / float(1 << 24)


def draft_tokens_other(cfg: ModelConfig, n: int) -> np.ndarray:
    """Uniform integers in [0, vocab-1), used as 'a token other than the greedy one'."""
    tid = zlib.crc32(b"draft-other")
    return uniform_int(cfg.seed, tid, n, max(cfg.vocab - 1, 1))

_reg(replace(CONFIGS["c4s"], name="c4s_bf16", expert_format="bf16", seed=2006))
# the Kimi-class slice with the pages' expert formats: experts shipped in MXFP4, gate/up re-encoded to FP8
# E4M3 with a bf16 scale per 256 when loaded, down kept in MXFP4
_reg(replace(CONFIGS["c3"], name="c3m", expert_format="mxfp4", seed=1005))
_reg(replace(CONFIGS["c3s"], name="c3ms", expert_format="mxfp4", seed=2008))
