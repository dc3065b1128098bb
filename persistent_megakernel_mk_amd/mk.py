"""Python binding of libmk.so (the C ABI in include/mk.h).

Argument marshalling only: every step of the decode path runs in the library's HIP kernels. PyTorch
supplies device memory (caller-owned buffers) and streams. Importing this module never falls back to
any other implementation: if libmk.so is missing or cannot load, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Iterable, List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmk.so")

MK_MAX_LAYERS = 128
MK_MAX_BATCH = 16
MK_VERIFY_ROWS = 8

STATUS = {0: "MK_OK", 1: "MK_E_ARG", 2: "MK_E_SHAPE", 3: "MK_E_UNSUPPORTED", 4: "MK_E_CAPACITY", 5: "MK_E_HIP",
          6: "MK_E_DEVICE_TIMEOUT", 7: "MK_E_STATE", 8: "MK_E_INEXACT"}
MIXER = {"gqa": 0, "gdn": 1, "kda": 2, "mla": 3}
FFN = {"dense": 0, "moe": 1}
DTYPE = {"bf16": 0, "nvfp4": 1, "mxfp4": 2}
(W_EMBED, W_FINAL_NORM, W_LM_HEAD, W_ATTN_NORM, W_FFN_NORM, W_Q, W_K, W_V, W_A, W_B, W_O, W_DKV, W_KR, W_UK, W_UV,
 W_GATE, W_UP, W_DOWN, W_ROUTER) = range(19)
_KIND_BY_SUFFIX = {"attn_norm": W_ATTN_NORM, "ffn_norm": W_FFN_NORM, "wq": W_Q, "wk": W_K, "wv": W_V, "wa": W_A,
                   "wb": W_B, "wo": W_O, "wdkv": W_DKV, "wkr": W_KR, "wuk": W_UK, "wuv": W_UV, "wg": W_GATE,
                   "wu": W_UP, "wd": W_DOWN, "router": W_ROUTER}

i32, i64, u64, f32, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float, ctypes.c_void_p


class Config(ctypes.Structure):
    _fields_ = [("n_layers", i32), ("hidden", i32), ("vocab", i32), ("mixer", i32 * MK_MAX_LAYERS),
                ("ffn_kind", i32 * MK_MAX_LAYERS), ("ffn", i32), ("n_q_heads", i32), ("n_kv_heads", i32),
                ("head_dim", i32), ("lin_heads", i32), ("d_k", i32), ("d_v", i32), ("mla_heads", i32),
                ("kv_rank", i32), ("rope_dim", i32), ("nope_dim", i32), ("v_dim", i32), ("n_experts", i32),
                ("top_k", i32), ("expert_ffn", i32), ("n_shared", i32), ("expert_format", i32), ("max_ctx", i32),
                ("max_batch", i32), ("eps", f32), ("rope_theta", f32)]


class Sizes(ctypes.Structure):
    _fields_ = [("packed_weights", u64), ("scratch", u64), ("kv_cache_per_layer", u64),
                ("lin_state_per_layer", u64), ("latent_per_layer", u64), ("n_phases", i32), ("n_workgroups", i32)]


class Buffers(ctypes.Structure):
    _fields_ = [("packed_weights", vp), ("scratch", vp), ("k_cache", vp * MK_MAX_LAYERS),
                ("v_cache", vp * MK_MAX_LAYERS), ("lin_state", vp * MK_MAX_LAYERS), ("latent", vp * MK_MAX_LAYERS)]


class WeightDesc(ctypes.Structure):
    _fields_ = [("layer", i32), ("kind", i32), ("expert", i32), ("dtype", i32), ("rows", i64), ("cols", i64),
                ("data", vp), ("scales", vp), ("tensor_scale", f32)]


class StepIO(ctypes.Structure):
    _fields_ = [("tokens", vp), ("hidden_in", vp), ("positions", vp), ("logits", vp), ("hidden_out", vp),
                ("argmax", vp), ("route_idx", vp), ("route_w", vp)]


_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load libmk.so; raises if it is not built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run persistent_megakernel_mk_amd/build.py "
                           "(or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    L.mk_create.argtypes, L.mk_create.restype = [P(Config), ctypes.c_int, P(vp)], ctypes.c_int
    L.mk_query_sizes.argtypes, L.mk_query_sizes.restype = [vp, P(Sizes)], ctypes.c_int
    L.mk_bind_buffers.argtypes, L.mk_bind_buffers.restype = [vp, P(Buffers)], ctypes.c_int
    L.mk_load_weights.argtypes, L.mk_load_weights.restype = [vp, P(WeightDesc), ctypes.c_int, vp], ctypes.c_int
    L.mk_decode_step.argtypes, L.mk_decode_step.restype = [vp, P(StepIO), ctypes.c_int, vp], ctypes.c_int
    L.mk_verify_step.argtypes, L.mk_verify_step.restype = [vp, P(StepIO), vp, vp, vp], ctypes.c_int
    L.mk_decode_step_noalloc.argtypes, L.mk_decode_step_noalloc.restype = [vp, P(StepIO), ctypes.c_int, vp], ctypes.c_int
    L.mk_decode_loop.argtypes = [vp, P(StepIO), ctypes.c_int, ctypes.c_int, vp, vp]
    L.mk_decode_loop.restype = ctypes.c_int
    L.mk_decode_step_perop.argtypes = [vp, P(StepIO), ctypes.c_int, ctypes.c_int, vp]
    L.mk_decode_step_perop.restype = ctypes.c_int
    L.mk_read_device_status.argtypes = [vp, P(i32), P(i32)]
    L.mk_read_device_status.restype = ctypes.c_int
    L.mk_destroy.argtypes, L.mk_destroy.restype = [vp], None
    L.mk_last_error.argtypes, L.mk_last_error.restype = [], ctypes.c_char_p
    L.mk_set_trace.argtypes, L.mk_set_trace.restype = [vp, vp, ctypes.c_int64], ctypes.c_int
    L.mk_set_launch_mode.argtypes, L.mk_set_launch_mode.restype = [vp, ctypes.c_int], ctypes.c_int
    L.mk_debug_phase_count.argtypes, L.mk_debug_phase_count.restype = [vp, ctypes.c_int], ctypes.c_int
    L.mk_debug_phase.argtypes, L.mk_debug_phase.restype = [vp, ctypes.c_int, ctypes.c_int, P(i32)], ctypes.c_int
    _lib = L
    return L


class MKError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def check(status: int) -> None:
    if status != 0:
        raise MKError(status, load().mk_last_error().decode())


def make_config(cfg, max_batch: Optional[int] = None) -> Config:
    c = Config()
    c.n_layers, c.hidden, c.vocab = cfg.n_layers, cfg.hidden, cfg.vocab
    for l in range(cfg.n_layers):
        c.mixer[l] = MIXER[cfg.mixers[l]]
        c.ffn_kind[l] = FFN[cfg.ffns[l]]
    c.ffn = cfg.ffn
    c.n_q_heads, c.n_kv_heads, c.head_dim = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    c.lin_heads, c.d_k, c.d_v = cfg.lin_heads, cfg.d_k, cfg.d_v
    c.mla_heads, c.kv_rank, c.rope_dim, c.nope_dim, c.v_dim = (cfg.mla_heads, cfg.kv_rank, cfg.rope_dim,
                                                                cfg.nope_dim, cfg.v_dim)
    c.n_experts, c.top_k, c.expert_ffn, c.n_shared = cfg.n_experts, cfg.top_k, cfg.expert_ffn, cfg.n_shared
    c.expert_format = DTYPE[cfg.expert_format]
    c.max_ctx = cfg.max_ctx
    c.max_batch = max_batch if max_batch is not None else cfg.batch
    c.eps, c.rope_theta = cfg.eps, cfg.rope_theta
    return c


def weight_target(name: str):
    """(layer, kind, expert) for a tensor name of the synthetic workloads."""
    if name == "embed":
        return -1, W_EMBED, -1
    if name == "final_norm":
        return -1, W_FINAL_NORM, -1
    if name == "lm_head":
        return -1, W_LM_HEAD, -1
    parts = name.split(".")
    layer = int(parts[0][1:])
    expert = -1
    if len(parts) == 3:
        tag = parts[1]
        expert = int(tag[1:]) if tag[0] == "e" else -2 - int(tag[1:])  # shared expert s -> -2 - s
    return layer, _KIND_BY_SUFFIX[parts[-1]], expert


def _stream_ptr(stream) -> int:
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


class Megakernel:
    """A bound context: caller-owned device buffers (torch) plus the library context."""

    def __init__(self, cfg, device: int = 0, max_batch: Optional[int] = None):
        import torch

        self.lib = load()
        self.cfg = cfg
        self.device = torch.device("cuda", device)
        self.max_batch = max_batch if max_batch is not None else cfg.batch
        self._c = make_config(cfg, self.max_batch)
        ctx = vp()
        check(self.lib.mk_create(ctypes.byref(self._c), device, ctypes.byref(ctx)))
        self.ctx = ctx
        sz = Sizes()
        check(self.lib.mk_query_sizes(self.ctx, ctypes.byref(sz)))
        self.sizes = sz
        dev = self.device
        self.wbuf = torch.empty(int(sz.packed_weights), dtype=torch.uint8, device=dev)
        self.scratch = torch.empty(max(int(sz.scratch), 256), dtype=torch.uint8, device=dev)
        self.k_cache: Dict[int, "torch.Tensor"] = {}
        self.v_cache: Dict[int, "torch.Tensor"] = {}
        self.lin_state: Dict[int, "torch.Tensor"] = {}
        self.latent: Dict[int, "torch.Tensor"] = {}
        B = self.max_batch
        b = Buffers()
        b.packed_weights = self.wbuf.data_ptr()
        b.scratch = self.scratch.data_ptr()
        for l in range(cfg.n_layers):
            m = cfg.mixers[l]
            if m == "gqa":
                shp = (B, cfg.n_kv_heads, cfg.max_ctx, cfg.head_dim)
                self.k_cache[l] = torch.zeros(shp, dtype=torch.bfloat16, device=dev)
                self.v_cache[l] = torch.zeros(shp, dtype=torch.bfloat16, device=dev)
                b.k_cache[l] = self.k_cache[l].data_ptr()
                b.v_cache[l] = self.v_cache[l].data_ptr()
            elif m in ("gdn", "kda"):
                self.lin_state[l] = torch.zeros((B, cfg.lin_heads, cfg.d_v, cfg.d_k), dtype=torch.float32, device=dev)
                b.lin_state[l] = self.lin_state[l].data_ptr()
            elif m == "mla":
                shp = (B, cfg.max_ctx, cfg.kv_rank + cfg.rope_dim)
                self.latent[l] = torch.zeros(shp, dtype=torch.bfloat16, device=dev)
                b.latent[l] = self.latent[l].data_ptr()
        check(self.lib.mk_bind_buffers(self.ctx, ctypes.byref(b)))
        self._bufs = b

    # ---- weights --------------------------------------------------------------------------
    def load_weights(self, W, names: Optional[Iterable[str]] = None, chunk_bytes: int = 1 << 30) -> None:
        """Upload host tensors (bf16 bits as uint16 numpy) and let the library repack them."""
        import torch

        names = list(names) if names is not None else list(W.keys())
        pending: List = []
        pend_bytes = 0

        def flush():
            nonlocal pending, pend_bytes
            if not pending:
                return
            arr = (WeightDesc * len(pending))()
            for i, (desc, _) in enumerate(pending):
                arr[i] = desc
            check(self.lib.mk_load_weights(self.ctx, arr, len(pending), _stream_ptr(None)))
            torch.cuda.current_stream().synchronize()
            pending, pend_bytes = [], 0

        for name in names:
            a = W[name]
            layer, kind, expert = weight_target(name)
            d = WeightDesc()
            d.layer, d.kind, d.expert = layer, kind, expert
            if hasattr(a, "codes"):  # NVFP4 (codes, E4M3 scales, tensor scale) or MXFP4 (codes, E8M0 scales)
                codes = torch.from_numpy(np.ascontiguousarray(a.codes)).to(self.device)
                scales = torch.from_numpy(np.ascontiguousarray(a.scales)).to(self.device)
                mx = getattr(a, "format", None) == "mxfp4"
                d.dtype = DTYPE["mxfp4" if mx else "nvfp4"]
                d.rows, d.cols = a.shape
                d.data, d.scales = codes.data_ptr(), scales.data_ptr()
                d.tensor_scale = 1.0 if mx else float(a.tensor_scale)
                pending.append((d, (codes, scales)))
                pend_bytes += codes.numel() + scales.numel()
            else:
                t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(self.device)
                d.dtype = DTYPE["bf16"]
                d.rows, d.cols = (1, a.shape[0]) if a.ndim == 1 else a.shape
                d.data = t.data_ptr()
                pending.append((d, t))
                pend_bytes += t.numel() * 2
            if pend_bytes >= chunk_bytes:
                flush()
        flush()

    # ---- states ---------------------------------------------------------------------------
    def set_states(self, S: Dict[str, np.ndarray]) -> None:
        import torch

        for name, a in S.items():
            layer = int(name.split(".")[0][1:])
            kind = name.split(".")[1]
            if kind == "kcache":
                dst = self.k_cache[layer]
            elif kind == "vcache":
                dst = self.v_cache[layer]
            elif kind == "lstate":
                dst = self.lin_state[layer]
            elif kind == "latent":
                dst = self.latent[layer]
            else:
                raise KeyError(name)
            src = torch.from_numpy(np.ascontiguousarray(a))
            if src.dtype == torch.uint16 or a.dtype == np.uint16:
                src = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
            dst[: src.shape[0]].copy_(src.to(self.device))
        torch.cuda.synchronize(self.device)

    def get_states(self, batch: Optional[int] = None) -> Dict[str, np.ndarray]:
        B = batch if batch is not None else self.cfg.batch
        out = {}
        for l, t in self.k_cache.items():
            out[f"l{l}.kcache"] = t[:B].view(dtype=__import__("torch").int16).cpu().numpy().view(np.uint16)
            out[f"l{l}.vcache"] = self.v_cache[l][:B].view(dtype=__import__("torch").int16).cpu().numpy().view(np.uint16)
        for l, t in self.lin_state.items():
            out[f"l{l}.lstate"] = t[:B].cpu().numpy()
        for l, t in self.latent.items():
            out[f"l{l}.latent"] = t[:B].view(dtype=__import__("torch").int16).cpu().numpy().view(np.uint16)
        return out

    # ---- steps ----------------------------------------------------------------------------
    def _check(self, name, t, shape, dtype):
        """A device tensor the kernel reads or writes through a raw pointer: its shape, dtype, device
        and layout must be exactly what the step assumes (a wrong one would be read or written past
        its end)."""
        import torch

        if t is None:
            return
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor")
        if t.device != self.device:
            raise ValueError(f"{name} is on {t.device}, the context's device is {self.device}")
        if t.dtype != dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")

    def _io(self, rows, tokens, hidden_in, positions, logits, hidden_out, argmax, route=None):
        import torch

        cfg = self.cfg
        self._check("tokens", tokens, (rows,), torch.int32)
        self._check("hidden_in", hidden_in, (rows, cfg.hidden), torch.float32)
        self._check("logits", logits, (rows, cfg.vocab), torch.float32)
        self._check("hidden_out", hidden_out, (rows, cfg.hidden), torch.float32)
        self._check("argmax", argmax, (rows,), torch.int32)
        if route is not None:
            self._check("route indices", route[0], (self.n_moe, rows, cfg.top_k), torch.int32)
            self._check("route gates", route[1], (self.n_moe, rows, cfg.top_k), torch.float32)
        io = StepIO()
        if route is not None:
            io.route_idx = route[0].data_ptr()
            io.route_w = route[1].data_ptr()
        io.tokens = tokens.data_ptr() if tokens is not None else None
        io.hidden_in = hidden_in.data_ptr() if hidden_in is not None else None
        self._pos = (i32 * MK_MAX_BATCH)(*[int(p) for p in positions])
        io.positions = ctypes.cast(self._pos, vp)
        io.logits = logits.data_ptr() if logits is not None else None
        io.hidden_out = hidden_out.data_ptr() if hidden_out is not None else None
        io.argmax = argmax.data_ptr() if argmax is not None else None
        return io

    def outputs(self, rows: int):
        import torch

        d = self.device
        if self.cfg.vocab:
            return (torch.empty((rows, self.cfg.vocab), dtype=torch.float32, device=d), None,
                    torch.empty(rows, dtype=torch.int32, device=d))
        return None, torch.empty((rows, self.cfg.hidden), dtype=torch.float32, device=d), None

    @property
    def n_moe(self) -> int:
        return sum(1 for f in self.cfg.ffns if f == "moe")

    def route_outputs(self, rows: int):
        """Device buffers for the routing of every MoE layer: indices int32 and gates fp32 [n_moe][rows][top_k]."""
        import torch

        shp = (self.n_moe, rows, self.cfg.top_k)
        return (torch.full(shp, -1, dtype=torch.int32, device=self.device),
                torch.zeros(shp, dtype=torch.float32, device=self.device))

    def decode(self, positions, tokens=None, hidden_in=None, out=None, stream=None, perop: bool = False, route=None,
               noalloc: bool = False, graph: bool = False):
        """One decode step for len(positions) sequences. tokens/hidden_in are device tensors; route is an
        optional (indices, gates) pair from route_outputs(). perop runs the per-op baseline (one launch per
        phase; with graph, replayed as a HIP graph); noalloc runs the step on the library-held working memory
        (mk_decode_step_noalloc)."""
        B = len(positions)
        logits, hidden_out, argmax = out if out is not None else self.outputs(B)
        io = self._io(B, tokens, hidden_in, positions, logits, hidden_out, argmax, route)
        if perop:
            check(self.lib.mk_decode_step_perop(self.ctx, ctypes.byref(io), B, int(graph), _stream_ptr(stream)))
        elif noalloc:
            check(self.lib.mk_decode_step_noalloc(self.ctx, ctypes.byref(io), B, _stream_ptr(stream)))
        else:
            check(self.lib.mk_decode_step(self.ctx, ctypes.byref(io), B, _stream_ptr(stream)))
        return {"logits": logits, "hidden_out": hidden_out, "argmax": argmax, "route": route}

    def decode_loop(self, positions, tokens, n_steps: int, out=None, tokens_out=None, stream=None):
        """n_steps greedy decode steps in one launch: step s runs at positions[b] + s on the token step s - 1
        emitted (its argmax), step 0 on `tokens`. Returns the emitted tokens [n_steps][B] and the last
        step's logits and argmax."""
        import torch

        B = len(positions)
        logits, hidden_out, argmax = out if out is not None else self.outputs(B)
        if tokens_out is None:
            tokens_out = torch.empty((n_steps, B), dtype=torch.int32, device=self.device)
        self._check("tokens_out", tokens_out, (n_steps, B), torch.int32)
        io = self._io(B, tokens, None, positions, logits, hidden_out, argmax)
        check(self.lib.mk_decode_loop(self.ctx, ctypes.byref(io), B, int(n_steps), tokens_out.data_ptr(),
                                      _stream_ptr(stream)))
        return {"tokens": tokens_out, "logits": logits, "argmax": argmax}

    def verify(self, position: int, tokens, out=None, acc=None, stream=None):
        import torch

        logits, _, argmax = out if out is not None else self.outputs(MK_VERIFY_ROWS)
        acc = acc if acc is not None else torch.zeros(2, dtype=torch.int32, device=self.device)
        io = self._io(MK_VERIFY_ROWS, tokens, None, [position], logits, None, argmax)
        self._check("accepted/bonus", acc, (2,), torch.int32)
        check(self.lib.mk_verify_step(self.ctx, ctypes.byref(io), ctypes.c_void_p(acc.data_ptr()),
                                      ctypes.c_void_p(acc.data_ptr() + 4), _stream_ptr(stream)))
        return {"logits": logits, "argmax": argmax, "accepted_bonus": acc}

    def set_trace(self, buf) -> None:
        """buf: torch uint8/int64 device tensor (or None) receiving [phase][workgroup][2] timestamps."""
        if buf is None:
            check(self.lib.mk_set_trace(self.ctx, None, 0))
        else:
            check(self.lib.mk_set_trace(self.ctx, ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size()))

    def set_launch_mode(self, cooperative: bool) -> None:
        check(self.lib.mk_set_launch_mode(self.ctx, 1 if cooperative else 0))

    def device_status(self):
        s, p = i32(), i32()
        check(self.lib.mk_read_device_status(self.ctx, ctypes.byref(s), ctypes.byref(p)))
        return s.value, p.value

    def phases(self, rows: int = 1):
        n = self.lib.mk_debug_phase_count(self.ctx, rows)
        out = []
        buf = (i32 * 16)()
        for i in range(n):
            self.lib.mk_debug_phase(self.ctx, rows, i, buf)
            out.append(list(buf))
        return out

    def close(self) -> None:
        if getattr(self, "ctx", None):
            self.lib.mk_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class HostContext:
    """Host-only context (no GPU): schedule and sizes, for testing the host logic."""

    def __init__(self, cfg, max_batch: Optional[int] = None):
        self.lib = load()
        self._c = make_config(cfg, max_batch)
        ctx = vp()
        check(self.lib.mk_create(ctypes.byref(self._c), -1, ctypes.byref(ctx)))
        self.ctx = ctx
        sz = Sizes()
        check(self.lib.mk_query_sizes(self.ctx, ctypes.byref(sz)))
        self.sizes = sz

    def phases(self, rows: int = 1):
        n = self.lib.mk_debug_phase_count(self.ctx, rows)
        out = []
        buf = (i32 * 16)()
        for i in range(n):
            self.lib.mk_debug_phase(self.ctx, rows, i, buf)
            out.append(list(buf))
        return out

    def __del__(self):
        try:
            if self.ctx:
                self.lib.mk_destroy(self.ctx)
        except Exception:
            pass
