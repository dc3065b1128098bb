#!/usr/bin/env python3
"""Benchmark of the persistent decode megakernel on one MI355X.

Workload (default): the hybrid 27B-class dense stack (64 layers, 3 gated-delta-net : 1 grouped-query
attention, hidden 5120, SwiGLU 17408, vocab 151936, 4096-token KV cache), one decode step at batch 1,
random bf16 weights from the seeded generator (generated in device memory). A step is one launch of the
megakernel: embedding, all 64 layers, final norm, LM head and argmax. Timed with HIP events on the
stream the kernel runs on. Also reported: batch 8, the per-op (one launch per phase) baseline, and the
CPU oracle on a bounded sample of the same workload.

Other workloads (--config): c2, the same stack's 8-row verify step (anchor + 7 drafts); c3, a Kimi-class
slice (3 Kimi-delta-attention : 1 absorbed latent attention layer, 384 bf16 experts top-8 + 1 shared,
hidden 7168) at batch 8; c4, an NVFP4-expert slice (8 GQA layers, 256 experts top-8 + 1 shared, hidden
6144) at batch 1 and 8. Mixture-of-experts steps count the experts of the batch's actual union.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config c1|c2|c3|c4] [--batches 1,8]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/s and achieved HBM GB/s (% of peak) at batch 1/8, one MI355X"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def build_gpu(cfg, max_batch, expert_pool=8):
    """Generates the configuration's weights and states in device memory and packs them. bf16 tensors come
    from the device generator. NVFP4 expert matrices are encoded on the host (seeded normals quantised
    onto the E2M1 x E4M3 grid); to keep that bounded, each projection kind uses a pool of `expert_pool`
    distinct encoded matrices, assigned to the experts in turn. Every expert still has its own packed
    copy, so the bytes a step streams are those of distinct experts; only the values repeat."""
    import torch

    from persistent_megakernel_mk_amd import mk, synth

    m = mk.Megakernel(cfg, device=0, max_batch=max_batch)
    t0 = time.time()
    pool = {}
    n_fp4 = 0
    for spec in synth.weight_specs(cfg):
        layer, kind, expert = mk.weight_target(spec.name)
        d = mk.WeightDesc()
        d.layer, d.kind, d.expert = layer, kind, expert
        if spec.kind in ("nvfp4", "mxfp4"):
            key, src = pooled_source(cfg, spec, expert_pool)
            if key not in pool:
                a = synth.generate(src, cfg.seed)
                pool[key] = (torch.from_numpy(a.codes).cuda(), torch.from_numpy(a.scales).cuda(),
                             float(getattr(a, "tensor_scale", 1.0)))
            codes, scales, ts = pool[key]
            d.dtype = mk.DTYPE[spec.kind]
            d.rows, d.cols = spec.shape
            d.data, d.scales, d.tensor_scale = codes.data_ptr(), scales.data_ptr(), ts
            t = None
            n_fp4 += 1
        else:
            t = synth.generate_gpu(spec, cfg.seed)
            d.dtype = mk.DTYPE["bf16"]
            d.rows, d.cols = (1, spec.shape[0]) if len(spec.shape) == 1 else spec.shape
            d.data = t.data_ptr()
        arr = (mk.WeightDesc * 1)(d)
        mk.check(m.lib.mk_load_weights(m.ctx, arr, 1, torch.cuda.current_stream().cuda_stream))
        torch.cuda.current_stream().synchronize()
        del t
    del pool
    wcfg = cfg.with_batch(max_batch)
    for spec in synth.state_specs(wcfg):
        t = synth.generate_gpu(spec, cfg.seed)
        layer, kind = int(spec.name.split(".")[0][1:]), spec.name.split(".")[1]
        dst = {"kcache": m.k_cache, "vcache": m.v_cache, "lstate": m.lin_state, "latent": m.latent}[kind][layer]
        dst.copy_(t)
        del t
    torch.cuda.synchronize()
    log(f"weights and states generated and packed in {time.time() - t0:.1f} s "
        f"({m.sizes.packed_weights / 1e9:.2f} GB packed"
        + (f"; {n_fp4} {cfg.expert_format.upper()} matrices from a pool of {expert_pool} per projection" if n_fp4 else "") + ")")
    return m


def pooled_source(cfg, spec, expert_pool=8):
    """The generator spec whose seeded values the NVFP4 expert matrix `spec` takes in build_gpu: per
    projection kind, `expert_pool` distinct encoded matrices assigned to the experts in turn. Returns
    (pool key, spec)."""
    import re

    layer = int(re.match(r"l(\d+)\.", spec.name).group(1))
    proj = spec.name.rsplit(".", 1)[1]
    e_idx = int(re.match(r"l\d+\.[se](\d+)\.", spec.name).group(1))
    key = (proj, (layer * (cfg.n_experts + cfg.n_shared) + e_idx) % expert_pool)
    return key, replace_name(spec, f"pool.{key[1]}.{proj}")


def replace_name(spec, name):
    from dataclasses import replace

    return replace(spec, name=name)


def save_states(m):
    return {(k, l): t.clone() for k, d in (("k", m.k_cache), ("v", m.v_cache), ("s", m.lin_state), ("lat", m.latent))
            for l, t in d.items()}


def restore_states(m, saved):
    for (k, l), t in saved.items():
        {"k": m.k_cache, "v": m.v_cache, "s": m.lin_state, "lat": m.latent}[k][l].copy_(t)


def seeded_drafts(m, cfg, p_greedy=0.8):
    """The verify workload's block: an anchor token and seven drafts at positions ctx..ctx+7. Draft i is,
    with probability p_greedy, the greedy (argmax) continuation of the anchor and drafts 1..i-1, else a
    uniform token other than it; the choice continues to condition the later drafts. The uniforms and
    the other tokens come from the seeded generator; the greedy tokens from decode steps of the same
    context, whose states are restored afterwards. Then P(a >= i) = p_greedy^i for the accepted count a."""
    import numpy as np
    import torch

    from persistent_megakernel_mk_amd import synth

    n = cfg.verify_rows - 1
    u = synth.draft_uniforms(cfg, n)
    other = synth.draft_tokens_other(cfg, n)
    toks = [int(synth.make_inputs(cfg.with_batch(1))["tokens"][0])]
    saved = save_states(m)
    out = m.outputs(1)
    for i in range(n):
        m.decode([cfg.ctx + i], tokens=torch.tensor(toks[i:i + 1], dtype=torch.int32, device="cuda"), out=out)
        t = int(out[2][0].item())
        toks.append(t if u[i] < p_greedy else int(other[i]) + (int(other[i]) >= t))
    torch.cuda.synchronize()
    restore_states(m, saved)
    del saved
    return np.array(toks, np.int32)


def make_runner(m, cfg, batch, perop=False, drafts=None, graph=False):
    """A closure that launches one step of the configuration: a decode step for `batch` sequences
    (tokens, or hidden states for slices without a vocabulary) at position ctx, or a verify step (anchor
    + 7 drafts, `drafts` or uniform tokens) when the configuration has verify rows. Returns (run, route
    buffers or None, verify, verify outputs or None)."""
    import torch

    from persistent_megakernel_mk_amd import synth

    inp = synth.make_inputs(cfg.with_batch(batch))
    verify = bool(cfg.verify_rows)
    route = None
    vout = None
    if verify:
        if drafts is None:
            drafts = synth.uniform_int(cfg.seed, 77, cfg.verify_rows, cfg.vocab).astype("int32")
        toks = torch.from_numpy(drafts).cuda()
        out = m.outputs(cfg.verify_rows)
        acc = torch.zeros(2, dtype=torch.int32, device="cuda")
        vout = acc
        run = lambda: m.verify(cfg.ctx, toks, out=out, acc=acc)  # noqa: E731
    else:
        pos = [cfg.ctx] * batch
        out = m.outputs(batch)
        route = m.route_outputs(batch) if m.n_moe else None
        if cfg.vocab:
            toks = torch.from_numpy(inp["tokens"]).cuda()
            run = lambda: m.decode(pos, tokens=toks, out=out, perop=perop, route=route, graph=graph)  # noqa: E731
        else:
            hid = torch.from_numpy(inp["hidden_in"]).cuda()
            run = lambda: m.decode(pos, hidden_in=hid, out=out, perop=perop, route=route, graph=graph)  # noqa: E731
    return run, route, verify, vout


def time_steps(m, cfg, batch, steps, warmup, perop=False, drafts=None, graph=False):
    """Times `steps` launches after `warmup` untimed ones with HIP events on the launch stream. A decode
    step takes tokens (or hidden states) for `batch` sequences at position ctx; a verify step (the
    configuration has verify rows) takes one anchor and seven drafts at position ctx. Returns the times,
    for mixture-of-experts layers the size of the batch's expert union per layer in the last step, and
    for verify the accepted count of the first (untimed) step from the context's initial states."""
    import torch

    run, route, verify, vout = make_runner(m, cfg, batch, perop, drafts, graph)
    accepted = None
    if verify:
        saved = save_states(m)
        run()
        torch.cuda.synchronize()
        accepted = int(vout[0].item())
        restore_states(m, saved)
        del saved
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record()
        run()
        ev[i][1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    per = sorted(a.elapsed_time(b) for a, b in ev)
    status = m.device_status()
    if status[0] != 0:
        raise RuntimeError(f"device status {status}")
    union = None
    if not verify and m.n_moe:
        idx = route[0].cpu().numpy()  # [n_moe][rows][top_k]
        union = [float(len(set(idx[l].reshape(-1).tolist()))) for l in range(idx.shape[0])]
    return {"mean_ms": statistics.fmean(per), "median_ms": statistics.median(per), "p10_ms": per[int(0.1 * (steps - 1))],
            "p90_ms": per[int(0.9 * (steps - 1))], "wall_ms": wall, "union": union, "accepted": accepted}


def time_loop(m, cfg, batch, n, reps=5):
    """Greedy decoding of n steps at positions ctx..ctx+n-1 two ways, both with the tokens staying on the
    device: one mk_decode_loop launch (the kernel picks and re-embeds each token), and n separate step
    launches each fed the previous step's argmax tensor. Median over `reps` of each, in ms per step."""
    import torch

    from persistent_megakernel_mk_amd import synth

    toks = torch.from_numpy(synth.make_inputs(cfg.with_batch(batch))["tokens"]).cuda()
    pos = [cfg.ctx] * batch
    out = m.outputs(batch)
    tout = torch.empty((n, batch), dtype=torch.int32, device="cuda")

    def loop():
        m.decode_loop(pos, toks, n, out=out, tokens_out=tout)

    outs = [m.outputs(batch) for _ in range(n)]

    def steps():
        t = toks
        for s in range(n):
            m.decode([c + s for c in pos], tokens=t, out=outs[s])
            t = outs[s][2]

    res = {}
    for name, fn in (("loop", loop), ("steps", steps)):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) / n)
        res[name] = statistics.median(ts)
    if m.device_status()[0] != 0:
        raise RuntimeError(f"device status {m.device_status()}")
    return res


def stream_read_gbs(gib: int = 8, reps: int = 10) -> float:
    """HBM read rate a plain library kernel reaches on this GPU: row sums of a float32 [rows][4096] matrix
    of `gib` GiB (each byte read once; the outputs are 1/4096 of the input), timed with HIP events; the
    best of `reps` passes, in GB/s. Of the torch kernels tried (full sum, max, copy, column sums) this
    one reads fastest. A practical ceiling to set the step kernel's rate against, beside the published
    8 TB/s."""
    import torch

    x = torch.ones((gib << 28) // 4096, 4096, dtype=torch.float32, device="cuda")
    x.sum(dim=1)
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        x.sum(dim=1)
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b))
    n = x.numel() * 4
    del x
    torch.cuda.empty_cache()
    return n / (best / 1e3) / 1e9


def describe(cfg, batch):
    if cfg.name in ("c1", "c2"):
        what = (f"hybrid 27B-class dense {'verify step (anchor + 7 drafts)' if cfg.verify_rows else 'decode step'}, "
                f"{cfg.n_layers} layers (3 GDN : 1 GQA), hidden {cfg.hidden}, SwiGLU {cfg.ffn}, vocab {cfg.vocab}, "
                f"{cfg.ctx}-token KV cache")
    elif cfg.name == "c3":
        what = (f"Kimi-class slice decode step, {cfg.n_layers} layers (3 KDA : 1 absorbed MLA), hidden {cfg.hidden}, "
                f"MoE {cfg.n_experts} experts top-{cfg.top_k} + {cfg.n_shared} shared (bf16, ffn {cfg.expert_ffn}), "
                f"{cfg.ctx}-token latent cache")
    elif cfg.name == "c3m":
        what = (f"Kimi-class slice decode step, {cfg.n_layers} layers (3 KDA : 1 absorbed MLA), hidden {cfg.hidden}, "
                f"MoE {cfg.n_experts} experts top-{cfg.top_k} + {cfg.n_shared} shared (MXFP4 shipped: gate/up re-encoded "
                f"to FP8 E4M3 + bf16 scale per 256, down MXFP4; ffn {cfg.expert_ffn}), {cfg.ctx}-token latent cache")
    elif cfg.name == "c4":
        what = (f"NVFP4-expert slice decode step, {cfg.n_layers} GQA layers, hidden {cfg.hidden}, MoE {cfg.n_experts} "
                f"experts top-{cfg.top_k} + {cfg.n_shared} shared (NVFP4, ffn {cfg.expert_ffn}), {cfg.ctx}-token KV cache")
    else:
        what = f"{cfg.n_layers}-layer decode step, hidden {cfg.hidden}"
    rows = f"{cfg.verify_rows} rows" if cfg.verify_rows else f"batch {batch}"
    return f"{cfg.name}: {what}, {rows}"


PHASE_NAMES = {1: "embed", 2: "product", 3: "delta-rule", 4: "attention", 5: "merge", 6: "final", 7: "hidden-out",
               8: "latent-attention", 9: "latent-merge"}


def trace_step(m, cfg, batch):
    """One traced step: per phase, the span from the first workgroup's start to the last one's end of
    work, and the gap to the next phase (grid barrier). Summed by phase kind (products by shape)."""
    import numpy as np
    import torch

    from persistent_megakernel_mk_amd import synth

    G = m.sizes.n_workgroups
    ph = m.phases(batch)
    buf = torch.zeros(len(ph) * G * 2, dtype=torch.int64, device="cuda")
    m.set_trace(buf)
    run, _, _, _ = make_runner(m, cfg, batch)
    for _ in range(2):
        run()
    torch.cuda.synchronize()
    m.set_trace(None)
    t = buf.cpu().numpy().reshape(len(ph), G, 2).astype(np.float64) / 100.0  # microseconds
    if os.environ.get("MK_TRACE_DUMP"):
        np.save(os.environ["MK_TRACE_DUMP"] + f"_b{batch}.npy", t)
        np.save(os.environ["MK_TRACE_DUMP"] + f"_b{batch}_phases.npy", np.array(ph))
    start, end = t[:, :, 0], t[:, :, 1]
    agg = {}
    total = (end[-1].max() - start[0].min())
    for i, p in enumerate(ph):
        key = PHASE_NAMES.get(p[0], str(p[0]))
        if p[0] == 2:
            key += f" {p[2]}x{p[3]} S={p[6]}"
        span = end[i].max() - start[i].min()
        work_med = float(np.median(end[i] - start[i]))
        gap = (start[i + 1].min() - end[i].max()) if i + 1 < len(ph) else 0.0
        a = agg.setdefault(key, [0, 0.0, 0.0, 0.0])
        a[0] += 1; a[1] += span; a[2] += work_med; a[3] += gap
    log(f"trace batch {batch}: step {total:.0f} us over {len(ph)} phases")
    # a representative layer in detail (layer 4..7: three GDN layers and one GQA layer)
    for i, p in enumerate(ph):
        if p[1] in (4, 7) and p[0] != 1:
            st = start[i] - start[i].min()
            wk = end[i] - start[i]
            gap = (start[i + 1].min() - end[i].max()) if i + 1 < len(ph) else 0.0
            log(f"  L{p[1]} {PHASE_NAMES.get(p[0], p[0]):10s} N={p[2]:6d} K={p[3]:6d} S={p[6]:2d}: start skew p50 {np.median(st):5.1f} "
                f"max {st.max():5.1f} | work p10 {np.percentile(wk, 10):6.1f} p50 {np.median(wk):6.1f} max {wk.max():6.1f} "
                f"| span {end[i].max() - start[i].min():6.1f} | barrier {gap:5.1f} us")
    for k, (n, span, wm, gap) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        log(f"  {k:40s} x{n:3d}: span {span:8.0f} us (median wg work {wm:8.0f}), barrier gaps {gap:7.0f} us")
    return agg


def _omp_threads(n):
    """Sets the OpenMP thread count of this process (the oracle's C++ ops run their output rows on it)."""
    import ctypes

    ctypes.CDLL("libgomp.so.1", mode=ctypes.RTLD_GLOBAL).omp_set_num_threads(int(n))


def cpu_baseline(cfg_full, layers=4, repeats=3):
    """The CPU oracle, as it stands, on a bounded sample of the same workload: the first `layers` layers
    (one full 3 GDN : 1 GQA group) plus the final norm and LM head, batch 1, timed `repeats` times with
    all host threads and again with one thread (medians); the per-token time is scaled to all layers as
    (layer time) * n_layers / layers + (head time)."""
    from dataclasses import replace

    import numpy as np

    from oracle import oracle as O
    from persistent_megakernel_mk_amd import synth

    O.build()
    cfg = replace(cfg_full, n_layers=layers, mixers=cfg_full.mixers[:layers], ffns=cfg_full.ffns[:layers], batch=1)

    class Rows:  # embedding rows generated on demand (only the gathered row is ever read)
        def __init__(self, spec, seed):
            self.spec, self.seed = spec, seed

        def __getitem__(self, idx):
            H = self.spec.shape[1]
            return np.stack([synth.normal_bf16(self.seed, self.spec.tid, H, self.spec.sigma, 0.0, offset=int(t) * H)
                             for t in np.atleast_1d(idx)])

    W = synth.LazyWeights(cfg)
    emb_spec = W.specs["embed"]
    W._cache["embed"] = Rows(emb_spec, cfg.seed)
    for n in W.keys():
        W[n]
    S0 = synth.make_states(cfg)
    inp = synth.make_inputs(cfg)
    all_threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))

    def one_token():
        S = O.copy_states(S0)
        t0 = time.perf_counter()
        x = O.embed(W, inp["tokens"])
        x = O._stack(cfg, W, S, x, [0], [cfg.ctx])
        t1 = time.perf_counter()
        logits = O.gemv(W["lm_head"], O.rmsnorm(x, W["final_norm"], cfg.eps))
        O.argmax(logits[0])
        t2 = time.perf_counter()
        return (t1 - t0) * cfg_full.n_layers / layers + (t2 - t1), t1 - t0, t2 - t1

    res = {}
    for threads in (all_threads, 1):
        _omp_threads(threads)
        one_token()  # warm (page faults, thread pool)
        runs = sorted(one_token() for _ in range(repeats))
        res[threads] = runs[len(runs) // 2]
    _omp_threads(all_threads)
    per, lay, head = res[all_threads]
    per1, lay1, head1 = res[1]
    return {"value": 1.0 / per, "unit": "tokens/s", "cores": all_threads, "kind": "oracle",
            "sample": f"first {layers} of {cfg_full.n_layers} layers + final norm + LM head at batch 1, median of "
                      f"{repeats}: {lay:.2f} s for the layers and {head:.2f} s for the head on {all_threads} threads, "
                      f"scaled to {cfg_full.n_layers} layers ({per:.2f} s per token)",
            "single_thread": {"value": 1.0 / per1, "unit": "tokens/s", "cores": 1,
                              "sample": f"same sample, median of {repeats}: {lay1:.2f} s layers + {head1:.2f} s head "
                                        f"({per1:.2f} s per token)"}}


KERNEL_SOURCES = ("mk_device.h", "mk_step.hip", "mk_step_nvfp4.hip", "mk_step_wide.hip", "mk_host.cpp", "mk_internal.h")


def kernel_source_sha256():
    """Hash of the sources the step kernels are built from (a counter profile holds for exactly these)."""
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, "persistent_megakernel_mk_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def counter_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, scaled by
    the calibration factors it records), or None when the kernel sources have changed since it was taken."""
    import re

    path = os.path.join(ROOT, "profiles", "mk_step_kernel_c1_b1.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    info = json.loads(m.group(1))
    if kernel_source_sha256() != info.get("kernel_source_sha256"):
        return None
    return info["traffic_bytes_per_launch"]


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c1")
    ap.add_argument("--ctx", type=int, default=0, help="cached positions per sequence (default: the configuration's)")
    ap.add_argument("--batches", default=None,
                    help="first is the headline; others are reported alongside (default: 1,8; 1 for the verify "
                         "configuration c2; 8 for c3)")
    ap.add_argument("--no-perop", action="store_true")
    ap.add_argument("--no-loop", action="store_true", help="skip the on-device multi-step loop measurement")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--trace", action="store_true", help="print a per-phase breakdown of one traced step")
    ap.add_argument("--plain-launch", action="store_true",
                    help="ordinary (non-cooperative) launch of the same grid, for profilers")
    ap.add_argument("--no-stream-ref", action="store_true", help="skip the plain read-rate reference")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="also run one plain device-to-device copy of this many MiB (a counter calibration kernel)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the megakernel runs on a single MI355X with no collectives "
              f"(--gpus {args.gpus} is not supported; multi-GPU sharding is a design note only)", file=sys.stderr)
        return 2

    import torch

    from persistent_megakernel_mk_amd import accounting, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    default_batches = {"c0": "1", "c1": "1,2,4,8,16", "c2": "1", "c3": "8", "c3m": "8", "c4": "1,4,8"}
    batches = [int(b) for b in (args.batches or default_batches.get(args.config, "1,8")).split(",")]
    if args.calib_copy:
        src = torch.ones(args.calib_copy << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.calib_copy} MiB read, {args.calib_copy} MiB written")
        del src, dst
    cfg = synth.CONFIGS[args.config]
    if args.ctx:
        from dataclasses import replace

        cfg = replace(cfg, ctx=args.ctx)
    m = build_gpu(cfg, max(batches))
    if args.plain_launch:
        m.set_launch_mode(False)
    drafts = seeded_drafts(m, cfg) if cfg.verify_rows else None
    results = {}
    for b in batches:
        r = time_steps(m, cfg, b, args.steps, args.warmup, drafts=drafts)
        rows = cfg.verify_rows or 1
        by = accounting.step_bytes(cfg, b, cfg.ctx, rows=rows, union=r["union"])
        r["tokens_s"] = b * rows / (r["mean_ms"] / 1e3)
        r["alg_bytes"] = by["total"]
        r["alg_gbs"] = by["total"] / (r["mean_ms"] / 1e3) / 1e9
        results[b] = r
        log(f"{describe(cfg, b)}: mean {r['mean_ms']:.3f} ms median {r['median_ms']:.3f} ms -> {r['tokens_s']:.1f} "
            f"{'rows' if cfg.verify_rows else 'tok'}/s, {r['alg_gbs']:.0f} GB/s algorithmic "
            f"({100 * r['alg_gbs'] / accounting.HBM_PEAK_GBS:.1f}% of 8 TB/s, {by['total'] / 1e9:.3f} GB per step"
            + (f", expert union per layer {r['union']}" if r["union"] else "")
            + (f", accepted {r['accepted']} of 7 drafts -> {(r['accepted'] + 1) / (r['mean_ms'] / 1e3):.1f} emitted tok/s"
               if r["accepted"] is not None else "") + ")")
    loop = None
    if cfg.vocab and not cfg.verify_rows and not args.no_loop:
        lr = time_loop(m, cfg, batches[0], 8)
        loop = {"steps_per_launch": 8, "ms_per_step": round(lr["loop"], 4), "tokens_s": round(batches[0] / (lr["loop"] / 1e3), 2),
                "separate_launches_ms_per_step": round(lr["steps"], 4)}
        log(f"greedy decoding, 8 steps per launch: {lr['loop']:.3f} ms per step; as 8 launches: {lr['steps']:.3f} ms per step")
    if args.trace:
        for b in batches:
            trace_step(m, cfg, b)
    perop = None
    if not args.no_perop and not cfg.verify_rows:
        r = time_steps(m, cfg, batches[0], max(3, args.steps // 4), 2, perop=True)
        rg = time_steps(m, cfg, batches[0], max(3, args.steps // 4), 2, perop=True, graph=True)
        perop = {"ms_per_step": r["mean_ms"], "tokens_s": batches[0] / (r["mean_ms"] / 1e3),
                 "launches_per_step": m.sizes.n_phases,
                 "graph": {"ms_per_step": rg["mean_ms"], "tokens_s": batches[0] / (rg["mean_ms"] / 1e3)}}
        log(f"per-op baseline batch {batches[0]}: {r['mean_ms']:.3f} ms; as a HIP graph: {rg['mean_ms']:.3f} ms")
    m.close()
    del m
    torch.cuda.empty_cache()
    stream = None
    if not args.no_stream_ref:
        stream = stream_read_gbs()
        log(f"plain read reference (float32 row sums over 8 GiB): {stream:.0f} GB/s "
            f"({100 * stream / accounting.HBM_PEAK_GBS:.1f}% of 8 TB/s)")
    cpu = None
    if not args.no_cpu and cfg.name == "c1" and not args.ctx:
        try:
            cpu = cpu_baseline(cfg)
            log(f"cpu oracle: {cpu['value']:.4f} tok/s on {cpu['cores']} threads ({cpu['sample']})")
        except Exception as e:  # the CPU leg must not hide the GPU result
            log(f"cpu baseline failed: {e!r}")
    h = results[batches[0]]
    # a verify step emits the accepted drafts plus the bonus token: (a + 1) tokens, not its 8 rows
    value = (h["accepted"] + 1) / (h["mean_ms"] / 1e3) if h["accepted"] is not None else h["tokens_s"]
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["mean_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random weights, caches and states; tokens uniform"
                + ("; drafts seeded, greedy with probability 0.8)" if cfg.verify_rows else ")"),
        "config": {"workload": describe(cfg, batches[0]), "batch": batches[0], "kv_positions": cfg.ctx},
        "roofline": {"bound": "hbm", "achieved": round(h["alg_gbs"], 1), "peak": accounting.HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(h["alg_gbs"] / accounting.HBM_PEAK_GBS, 4),
                     # the counter profile covers the default workload only (c1, batch 1, its own cache length)
                     "traffic": counter_traffic() if (cfg.name == "c1" and batches[0] == 1
                                                      and cfg.ctx == synth.CONFIGS["c1"].ctx) else None,
                     "alg_bytes_per_launch": h["alg_bytes"], "kernel": "mk_step_kernel"},
        "cpu_baseline": cpu,
        "stream_read_ref": None if stream is None else {
            "gbs": round(stream, 1), "kind": "float32 row sums of an 8 GiB [rows][4096] matrix (torch), best of 10",
            "step_frac_of_ref": round(h["alg_gbs"] / stream, 4)},
        "latency_ms": {"median": round(h["median_ms"], 4), "p10": round(h["p10_ms"], 4), "p90": round(h["p90_ms"], 4)},
        "batches": {str(b): {"ms_per_step": round(r["mean_ms"], 4), "tokens_s": round(r["tokens_s"], 2),
                             "alg_gbs": round(r["alg_gbs"], 1),
                             "frac_of_peak": round(r["alg_gbs"] / accounting.HBM_PEAK_GBS, 4)}
                    for b, r in results.items()},
        "perop_baseline": perop,
        "decode_loop": loop,
    }
    if h["accepted"] is not None:
        line["verify"] = {"drafts": "seeded: each draft the greedy continuation with probability 0.8, else a uniform "
                                    "other token", "tokens": [int(t) for t in drafts], "accepted": h["accepted"],
                          "emitted_per_step": h["accepted"] + 1,
                          "emitted_tokens_s": round((h["accepted"] + 1) / (h["mean_ms"] / 1e3), 2),
                          "rows_s": round(h["tokens_s"], 2)}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
