// Persistent decode megakernel for MI355X (gfx950, CDNA4).
//
// One launch runs a whole decode (or 8-row verify) step of a hybrid decoder stack. It follows the
// design the pages give for TPU v7 ("Kimi K3's TPU megakernel: 92 layers in one Pallas call, and what
// 709 tokens a second measures", sections "What a megakernel is, and what it fixes on a TPU" and "How
// it maps onto a TPU v7"): the step is one program; weight loads are issued by the program itself as
// early as on-chip storage allows; the layer loop branches on the layer kind. On gfx950 the single
// sequential program becomes one workgroup per compute unit, all co-resident, walking the same phase
// table; a grid barrier separates phases whose inputs another workgroup produced. Weights stream
// through a per-wave register ring (nontemporal 16-byte loads, one 1 KiB MFMA fragment per wave per
// load) into v_mfma_f32_16x16x32_bf16, which plays the role of the TPU's matrix unit: the batch rows
// (at most 8, split into bf16 high and low halves so the fp32 activations keep 16 significant bits)
// fill the 16 columns, the way the TPU kernel broadcasts one row to its 16-row tile.
//
// Cross-workgroup data is written with agent-scope (sc1, write-through) stores and read with
// agent-scope loads, after the grid barrier or inside a phase; no cache is invalidated at a barrier.
//
// This header holds the whole step body; mk_step.hip and mk_step_nvfp4.hip each instantiate one
// build of it, so the two builds compile in parallel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_internal.h"

namespace mk {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
// The step's argument block, read in place from the kernel-argument segment (constant address space)
// wherever a member is used, rather than copied into registers.
typedef const __attribute__((address_space(4))) StepArgs CArgs;

// ---------------------------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ uint16_t f2bf(float f) {  // round to nearest even
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float ld_c(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_c(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_ci(const int32_t *p) {
  return __hip_atomic_load(const_cast<int32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_ci(int32_t *p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Device-coherent loads of 2 and 4 floats (8-byte atomic loads): read other workgroups' results of
// earlier phases without invalidating this XCD's caches at every grid barrier.
__device__ __forceinline__ float2 ld_c2(const float *p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<uint64_t *>(const_cast<float *>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}
__device__ __forceinline__ float4 ld_c4(const float *p) {
  const float2 lo = ld_c2(p), hi = ld_c2(p + 2);
  return make_float4(lo.x, lo.y, hi.x, hi.y);
}
// acc[e] += p[e], e < 8, from another workgroup's results (device-coherent; p 8-byte aligned)
__device__ __forceinline__ void add8(float (&acc)[8], const float *p) {
  const float4 lo = ld_c4(p), hi = ld_c4(p + 4);
  acc[0] += lo.x; acc[1] += lo.y; acc[2] += lo.z; acc[3] += lo.w;
  acc[4] += hi.x; acc[5] += hi.y; acc[6] += hi.z; acc[7] += hi.w;
}

// Sums over the k-split partials of an earlier product (S of them, stride floats apart), in k-split
// order as a loop would, but with the loads of CH splits in flight together: a runtime-length loop of
// dependent adds waits for each load in turn. (CH is kept small where the weight ring is live.)
template <int CH>
__device__ __forceinline__ float sum_splits(const float *p, size_t stride, int S) {
  float v = 0.0f;
  for (int s0 = 0; s0 < S; s0 += CH) {
    float x[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) x[i] = s0 + i < S ? ld_c(p + (size_t)(s0 + i) * stride) : 0.0f;
#pragma unroll
    for (int i = 0; i < CH; ++i)
      if (s0 + i < S) v += x[i];
  }
  return v;
}
template <int CH>
__device__ __forceinline__ float2 sum_splits2(const float *p, size_t stride, int S) {
  float2 v = make_float2(0.0f, 0.0f);
  for (int s0 = 0; s0 < S; s0 += CH) {
    float2 x[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) x[i] = s0 + i < S ? ld_c2(p + (size_t)(s0 + i) * stride) : make_float2(0.0f, 0.0f);
#pragma unroll
    for (int i = 0; i < CH; ++i)
      if (s0 + i < S) { v.x += x[i].x; v.y += x[i].y; }
  }
  return v;
}
__device__ __forceinline__ uint32_t ld_cu(const uint32_t *p) {
  return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint4 ld_nt(const uint4 *p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return uint4{v.x, v.y, v.z, v.w};
}

// Members of the argument block are only ever indexed with constants: a run-time index into the
// block would make the compiler keep the whole block in vector registers.
__device__ __forceinline__ float *part_of(CArgs &a, int i) {
  return i == 0 ? a.part[0] : (i == 1 ? a.part[1] : a.part[2]);
}
__device__ __forceinline__ int pos_of(CArgs &a, int i) {
  int p = a.pos[0];
#pragma unroll
  for (int k = 1; k < kMaxBatch; ++k)
    if (i == k) p = a.pos[k];
  return p;
}
// position of sequence i's new token in the decode step phase ph belongs to (a multi-step launch
// advances every sequence by one position per step)
__device__ __forceinline__ int pos_at(CArgs &a, const Phase &ph, int i) { return pos_of(a, i) + ph.step; }

// workgroup barrier that orders LDS only (global memory is ordered explicitly where needed)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// v from the lane CTRL (a DPP lane pattern) names, within its 16-lane row
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// sum over the wave, the same value in every lane: DPP exchanges inside each 16-lane row (lane i ^ 1,
// i ^ 2, then the mirrored lane of the 8-lane half and of the row: each step adds two equal-sized
// partial sums, so all lanes of a row hold the same row sum), then the four row sums read from lanes
// 0, 16, 32 and 48. No LDS round trips on this chain (a butterfly of lane shuffles takes six).
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  v += dpp_f<0x140>(v);  // row_mirror
  const int b = __float_as_int(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 0)), r1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 32)), r3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
  return (r0 + r1) + (r2 + r3);
}

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
// The (value, index) pair with the larger value (the smaller index on equal values) over the wave, in
// every lane: the same DPP row exchanges as wave_sum, then the four row results. The choice is symmetric,
// so the order of the exchanges does not change the result.
__device__ __forceinline__ void wave_argmax(float &v, int &e) {
  auto take = [&](float ov, int oe) {
    if (ov > v || (ov == v && oe < e)) { v = ov; e = oe; }
  };
  take(dpp_f<0xB1>(v), dpp_i<0xB1>(e));
  take(dpp_f<0x4E>(v), dpp_i<0x4E>(e));
  take(dpp_f<0x141>(v), dpp_i<0x141>(e));
  take(dpp_f<0x140>(v), dpp_i<0x140>(e));
  const int vb = __float_as_int(v);
  const float v1 = __int_as_float(__builtin_amdgcn_readlane(vb, 16)), v2 = __int_as_float(__builtin_amdgcn_readlane(vb, 32));
  const float v3 = __int_as_float(__builtin_amdgcn_readlane(vb, 48));
  const int e1 = __builtin_amdgcn_readlane(e, 16), e2 = __builtin_amdgcn_readlane(e, 32), e3 = __builtin_amdgcn_readlane(e, 48);
  v = __int_as_float(__builtin_amdgcn_readlane(vb, 0));
  e = __builtin_amdgcn_readlane(e, 0);
  take(v1, e1);
  take(v2, e2);
  take(v3, e3);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }
__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + __expf(-z)); }
__device__ __forceinline__ float softplusf_(float a) { return a > 20.0f ? a : log1pf(__expf(a)); }

// Writes activation value y of row b at column k into a staged buffer: the bf16 high half and the
// bf16 low half (y minus the high half) at the B-operand positions the LDS copy of a product expects
// ([k / 8][C][8]: up to 8 rows, columns b and R + b; above, row group b / 8 at columns 16 (b / 8) +
// (b % 8) and 16 (b / 8) + rows-in-group + (b % 8)).
__device__ __forceinline__ void stg_put(uint16_t *buf, int R, int k, int b, float y) {
  const bool wide = R > kMaxRows;
  const int C = wide ? 32 : 2 * R;
  const int grp = wide ? b >> 3 : 0, bl = wide ? b & 7 : b, Rg = wide ? min(8, R - 8 * grp) : R;
  const size_t u = (size_t)(k >> 3) * C + grp * 16 + bl;
  const uint16_t hi = f2bf(y), lo = f2bf(y - bf2f(hi));
  __hip_atomic_store(buf + u * 8 + (k & 7), hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // device-coherent
  __hip_atomic_store(buf + (u + Rg) * 8 + (k & 7), lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// x writers: x times the bf16 gain of the RMSNorm that reads it next, staged
__device__ __forceinline__ void stg_put_x(CArgs &a, const Phase &ph, int n, int b, float v) {
  const float g = bf2f(reinterpret_cast<const uint16_t *>(a.wbuf + ph.stg_gain_off)[n]);
  stg_put(a.stg[0], a.R, n, b, v * g);
}

// ---------------------------------------------------------------------------------------------
// grid barrier: two-level counters (kBarGroups groups, then one top counter), monotone across steps.
// Run by lane 0 of the sync wave; the caller brackets it with workgroup barriers.
// ---------------------------------------------------------------------------------------------
__device__ bool grid_arrive_wait(CArgs &a, uint32_t k, int phase) {
  const uint32_t G = gridDim.x;
  const uint32_t groups = G < (uint32_t)kBarGroups ? G : (uint32_t)kBarGroups;
  const uint32_t g = blockIdx.x % groups;
  const uint32_t cnt = G / groups + (g < (G % groups) ? 1u : 0u);
  uint32_t old = __hip_atomic_fetch_add(a.bar + g * 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (old + 1u == k * cnt) __hip_atomic_fetch_add(a.bar + kBarGroups * 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t tgt = k * groups;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  bool ok = true;
  for (uint32_t it = 0;; ++it) {
    // the barrier word and (every 16th poll) the abort flag are loaded together
    const uint32_t v = ld_cu(a.bar + kBarGroups * 32);
    const int32_t ab = (it & 15u) == 15u ? ld_ci(a.status + 2) : 0;
    if ((int32_t)(v - tgt) >= 0) break;
    if (ab != 0) { ok = false; break; }
    __builtin_amdgcn_s_sleep(1);
    if ((int64_t)(__builtin_amdgcn_s_memrealtime() - t0) > a.timeout_ticks) {
      st_ci(a.status + 1, phase);
      st_ci(a.status + 0, 6 /* MK_E_DEVICE_TIMEOUT */);
      st_ci(a.status + 2, 1);
      ok = false;
      break;
    }
  }
  // every later read of another workgroup's result is a device-coherent load, so no cache is
  // invalidated here; the fence keeps the compiler from moving those loads above the wait
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  return ok;
}

// wave-local LDS ordering (one wave writes, other lanes of the same wave read)
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// ---------------------------------------------------------------------------------------------
// the weight stream: each compute wave walks its fragments of every product phase of the launch in
// order; a register ring keeps kRing fragments in flight, across phase ends and grid barriers
// ---------------------------------------------------------------------------------------------
// phase descriptors are read through the constant address space, so they land in scalar registers
// (scalar loads: they never wait behind the weight stream's vector loads)
typedef const __attribute__((address_space(4))) Phase CPhase;
__device__ __forceinline__ CPhase *cphase(CArgs &a, int q) { return (CPhase *)(a.phases + q); }
__device__ __forceinline__ Phase load_phase(CArgs &a, int q) {
  typedef const __attribute__((address_space(4))) int32_t cint;
  Phase p;
  cint *src = (cint *)(a.phases + q);
  int32_t *dst = reinterpret_cast<int32_t *>(&p);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(Phase) / 4); ++i) dst[i] = src[i];
  return p;
}

// ---------------------------------------------------------------------------------------------
// product phases: units, routing, weight stream
// ---------------------------------------------------------------------------------------------

// Per-step routing of one MoE layer, in LDS (built by every workgroup at the start of the layer's
// first expert product and kept through the layer's second).
struct RouteLds {
  int32_t nseg;                     // shared experts + the routed union of the batch
  int32_t pad[3];
  int32_t expert[kMaxSeg];          // weight block of each segment (shared expert s -> n_exp + s)
  float wt[kMaxSeg][kMaxRows];      // mixing weight of each segment per row (shared: 1, unrouted: 0)
  int32_t idx[kMaxRows][kMaxTopK];  // top-k experts of each row in selection order
  float gw[kMaxRows][kMaxTopK];     // their normalised gates
};

constexpr int kRedSlots = 8;  // unit partials in flight between the compute waves and the sync wave
struct GemvLds {
  static constexpr int act = 0;                                                 // kActLdsBudget bytes
  static constexpr int red = kActLdsBudget;                                     // [kRedSlots][kCWaves][16][kMaxBatch] f32
  static constexpr int flags = red + kRedSlots * kCWaves * 16 * kMaxBatch * 4;  // posted[kRedSlots], consumed[kRedSlots]
  static constexpr int misc = flags + 2 * kRedSlots * 4;                        // rstd, finalizer flags, candidates
  static constexpr int route = misc + 8192;                                     // RouteLds
  static constexpr int end = route + (int)sizeof(RouteLds);
};
static_assert(GemvLds::end <= kLdsBytes, "product-phase LDS layout exceeds the workgroup's LDS");
static_assert((16 + kMaxUnits + 512 + 16 * kMaxBatch) * 4 <= GemvLds::route - GemvLds::misc,
              "product-phase scratch (1/rms, unit flags, argmax candidates, tile sums) exceeds its LDS region");

__device__ __forceinline__ const RouteLds *route_lds(const char *smem) {
  return reinterpret_cast<const RouteLds *>(smem + GemvLds::route);
}

// Units of a product phase: every k-split s gets gridDim.x / S workgroups (S divides the workgroup
// count); its units are the tiles of all segments in order (segment j, tile t -> unit j * seg_T + t),
// divided evenly over those workgroups, so every workgroup works inside one k-split: units [u0, u1).
__device__ __forceinline__ int phase_units(const Phase &ph, const char *smem) {
  return ph.seg == SEG_EXPERT ? route_lds(smem)->nseg * ph.seg_T : ph.T;
}
__device__ __forceinline__ void unit_range(int U, int S, int &s, int &u0, int &u1) {
  const int per = (int)gridDim.x / S, wg = blockIdx.x;
  s = wg / per;
  const int wl = wg - s * per;
  u0 = (int)(((int64_t)U * wl) / per);
  u1 = (int)(((int64_t)U * (wl + 1)) / per);
}

// Residual products finalise each tile in its last contributor. The workgroups of different k-splits
// that share a tile range walk it starting at different tiles (split s starts s/S of the way in and
// wraps), so the last contribution to the range's tiles, and with it the finalisation work, is spread
// over those workgroups instead of falling on whichever finishes last.
__device__ __forceinline__ bool rotated(const Phase &ph) {
  return ph.seg == SEG_NONE && ph.S > 1 && (ph.out == OUT_RESID || ph.out == OUT_LOGITS);
}
__device__ __forceinline__ int rot_start(int s, int S, int n) { return (int)(((int64_t)s * n) / S); }

// Router top-k and the batch's expert union (every workgroup computes the same table from the router
// logits z, so no extra grid barrier is needed). Per row: k passes of an argmax over z that keeps the
// first maximum (lowest expert index on ties); gates are the sigmoids of the selected logits divided
// by their sum, accumulated in selection order. Segments: the shared experts, then the union of the
// rows' selections in increasing expert index. Called by all waves (three workgroup barriers).
__device__ __forceinline__ void compute_route(CArgs &a, const Phase &ph, char *smem) {
  RouteLds *rt = reinterpret_cast<RouteLds *>(smem + GemvLds::route);
  const int R = a.R, E = ph.n_exp, K = ph.top_k, ns = ph.n_shared;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  float *zl = reinterpret_cast<float *>(smem + GemvLds::act);  // [R][E] router logits (staged before the product's activation)
  const float *zp = part_of(a, ph.z_part);
  for (int b = wave; b < R; b += kWavesTotal) {
    float *zr = zl + b * E;
    for (int e = lane; e < E; e += 64) zr[e] = sum_splits<8>(zp + (size_t)b * ph.z_N + e, (size_t)R * ph.z_N, ph.z_S);
    wave_lds_sync();
    float total = 0.0f;
    for (int t = 0; t < K; ++t) {
      float bv = -INFINITY;
      int be = 0x7fffffff;
      for (int e = lane; e < E; e += 64) {  // increasing e per lane: a strict > keeps the first maximum
        const float v = zr[e];
        if (v > bv || be == 0x7fffffff) { bv = v; be = e; }
      }
      wave_argmax(bv, be);
      be = __builtin_amdgcn_readfirstlane(be);
      const float sg = sigmoidf_(bv);
      total += sg;
      if (lane == 0) {
        zr[be] = -INFINITY;  // taken (a -inf logit is never selected over a finite one before it)
        rt->idx[b][t] = be;
        rt->gw[b][t] = sg;
      }
      wave_lds_sync();
    }
    if (lane < K) rt->gw[b][lane] = rt->gw[b][lane] / total;
  }
  lds_barrier();
  if (wave == 0) {  // union: lane w owns experts [32 w, 32 w + 32)
    uint32_t m = 0;
    for (int b = 0; b < R; ++b)
      for (int t = 0; t < K; ++t) {
        const int e = rt->idx[b][t];
        if ((e >> 5) == lane) m |= 1u << (e & 31);
      }
    const int c = __popc(m);
    int pre = c;  // inclusive scan of the counts over lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(pre, o);
      if (lane >= o) pre += v;
    }
    const int total = __shfl(pre, 63);
    int slot = ns + pre - c;
    while (m) {
      const int bit = __ffs(m) - 1;
      m &= m - 1;
      rt->expert[slot++] = lane * 32 + bit;
    }
    if (lane < ns) rt->expert[lane] = E + lane;
    if (lane == 0) rt->nseg = ns + total;
  }
  lds_barrier();
  const int nseg = rt->nseg;
  for (int i = threadIdx.x; i < nseg * R; i += kThreads) {
    const int j = i / R, b = i % R;
    float w = 0.0f;
    if (j < ns) {
      w = 1.0f;
    } else {
      const int e = rt->expert[j];
      for (int t = 0; t < K; ++t)
        if (rt->idx[b][t] == e) w = rt->gw[b][t];
    }
    rt->wt[j][b] = w;
  }
  if (blockIdx.x == 0 && a.route_idx && threadIdx.x < R * K) {
    const int b = threadIdx.x / K, t = threadIdx.x % K;
    a.route_idx[((size_t)ph.moe_idx * R + b) * K + t] = rt->idx[b][t];
    if (a.route_w) a.route_w[((size_t)ph.moe_idx * R + b) * K + t] = rt->gw[b][t];
  }
  lds_barrier();
}

// The weight stream of one compute wave: the wave's share of every product phase, in phase order.
// An item is one 1 KiB load per wave: a bf16 fragment (16 rows x 32 columns); for NVFP4 or MXFP4 the
// codes of four fragments (16 rows x 128 columns) with a load of their scales (128 B of E4M3, or 64 B of
// E8M0); for FP8 the values of two fragments (16 rows x 64 columns) with a load of the bf16 scales of
// their 256-column block (32 B, shared by the block's four items).
struct Stream {
  const uint4 *ptr;        // next item (or a valid dummy address once the stream is done)
  const uint32_t *sptr;    // its scales, or a fixed dummy word
  int q, left, j, nfw, skip, sstep;  // phase, units left, item in run, items per run, items between runs,
                                     // scale words per item (NVFP4 32, MXFP4 16; 0: none or FP8)
  int seg, seg_left;       // current segment, units left in it
  int route_q;             // routing this workgroup holds (phase index of its expert gate/up product)
  int blocked;             // expert phase the stream waits at until the routing is known (-1: none)
  int fmt;                 // WeightFmt of the current phase
  int sidx;                // this lane's word in an item's scale record (per lane)
  int kpos, kpos0;         // FP8: item index along the tile's row (current, first of the run)
  int tile_words;          // FP8: scale words per tile
  const uint32_t *sbase;   // FP8: the current tile's scales
};

__device__ __forceinline__ int items_per_frag_row(const Phase &ph) { return ph.KF / frags_per_item(ph.fmt); }

// The compute waves' shares of the n items of a k-split: contiguous runs, the first n % 4 waves one
// item longer (the schedule makes n a multiple of 4 up to kMaxRows rows; above, any n >= 4).
__device__ __forceinline__ int wave_items(int n, int w) { return n / kCWaves + (w < n % kCWaves ? 1 : 0); }
__device__ __forceinline__ int wave_first(int n, int w) { return w * (n / kCWaves) + min(w, n % kCWaves); }

// first item of segment seg, tile t (its own weight block for expert phases), this wave's run
__device__ __forceinline__ void stream_at(Stream &st, CArgs &a, CPhase *ph, const char *smem, int s, int seg,
                                          int t, int wave) {
  const int fpi = frags_per_item(ph->fmt);
  const int KI = ph->KF / fpi, nfi = ph->nf / fpi;
  const uint8_t *base = a.wbuf + ph->w_off;
  int64_t tile = t;
  if (ph->seg == SEG_EXPERT) base += (int64_t)__builtin_amdgcn_readfirstlane(route_lds(smem)->expert[seg]) * ph->seg_stride;
  else tile += (int64_t)seg * ph->seg_T;
  const int64_t item = tile * KI + s * nfi + wave_first(nfi, wave);
  st.ptr = reinterpret_cast<const uint4 *>(base) + item * 64;
  if (ph->fmt != FMT_BF16) {  // the scales follow the matrix's codes
    const int Tm = ph->seg == SEG_EXPERT ? ph->seg_T : ph->T;
    const uint32_t *sc = reinterpret_cast<const uint32_t *>(base + (int64_t)Tm * KI * 1024);
    if (ph->fmt == FMT_FP8R) {  // [tile][256-column block][16 rows] bf16: 8 words per (tile, block)
      st.tile_words = (KI / 4) * 8;
      st.sbase = sc + tile * st.tile_words;
      st.kpos = st.kpos0 = s * nfi + wave_first(nfi, wave);
      st.sptr = st.sbase + (st.kpos >> 2) * 8;
    } else {
      st.sptr = sc + item * st.sstep;
    }
  }
}

__device__ __forceinline__ void stream_seek(Stream &st, CArgs &a, const char *smem, int wave, int q) {
  st.q = -1;
  st.left = 0;
  st.blocked = -1;
  st.ptr = reinterpret_cast<const uint4 *>(a.wbuf);
  st.sptr = reinterpret_cast<const uint32_t *>(a.wbuf);  // scale loads of a done or blocked stream: a fixed
  st.sstep = 0;                                          // word of the weight buffer
  st.sidx = 0;
  st.fmt = FMT_BF16;
  while (q >= 0 && q < a.phase_end) {
    CPhase *ph = cphase(a, q);
    if (ph->type == PH_GEMV) {
      if (ph->seg == SEG_EXPERT && ph->route_q != st.route_q) {  // routing not known yet: wait there
        st.blocked = q;
        return;
      }
      const int U = ph->seg == SEG_EXPERT ? __builtin_amdgcn_readfirstlane(route_lds(smem)->nseg) * ph->seg_T : ph->T;
      int s, u0, u1;
      unit_range(U, ph->S, s, u0, u1);
      if (u1 > u0) {
        const int fpi = frags_per_item(ph->fmt);
        const int nfi = ph->nf / fpi;
        st.q = q;
        st.nfw = wave_items(nfi, wave);
        st.left = u1 - u0;
        st.j = 0;
        st.skip = ph->KF / fpi - st.nfw;
        st.fmt = ph->fmt;
        st.sstep = ph->fmt == FMT_NVFP4 ? 32 : (ph->fmt == FMT_MXFP4 ? 16 : 0);
        {  // the scale word of this lane's row: NVFP4 per half of the lane groups, MXFP4 one per row, FP8
           // two rows' bf16 per word
          const int ln = (int)threadIdx.x & 63;
          st.sidx = ph->fmt == FMT_NVFP4 ? (ln & 15) + 16 * (ln >> 5) : (ph->fmt == FMT_MXFP4 ? ln & 15 : (ln & 15) >> 1);
        }
        const int sT = ph->seg == SEG_EXPERT ? ph->seg_T : 0x40000000;
        st.seg = ph->seg == SEG_EXPERT ? u0 / sT : 0;
        int t = ph->seg == SEG_EXPERT ? u0 - st.seg * sT : u0;
        st.seg_left = sT - t;
        const bool rot = ph->seg == SEG_NONE && ph->S > 1 && (ph->out == OUT_RESID || ph->out == OUT_LOGITS);
        if (rot) {  // start r0 units in; after the range's end wrap to its first tile
          const int r0 = rot_start(s, ph->S, u1 - u0);
          t = u0 + r0;
          st.seg_left = (u1 - u0) - r0;
          st.seg = -1;  // marks the pending wrap
        }
        stream_at(st, a, ph, smem, s, st.seg < 0 ? 0 : st.seg, t, wave);
        return;
      }
    }
    q = ph->next_gemv;
  }
}

// Always issues its loads (dummies once the stream is done), so a ring slot is only ever written by a
// load and its register never needs a copy that would wait for the load. The build that decodes
// narrow formats loads a scale word with every item (for a bf16 item, one fixed word of the weight
// buffer), so every slot issues the same two loads and each slot's wait leaves the younger slots'
// loads in flight.
template <bool HAS_FP4>
__device__ __forceinline__ void stream_take(Stream &st, CArgs &a, const char *smem, int wave, int lane,
                                            uint4 &v, uint32_t &sv) {
  v = ld_nt(st.ptr + lane);
  if (HAS_FP4) sv = __builtin_nontemporal_load(st.sptr + st.sidx);
  if (st.q >= 0) {
    st.ptr += 64;
    st.sptr += st.sstep;
    if (__builtin_expect(st.fmt == FMT_FP8R, 0) && (++st.kpos & 3) == 0) st.sptr += 8;  // FP8: next 256-column block
    if (__builtin_expect(++st.j == st.nfw, 0)) {  // end of a run: rare next to the items (laid out away from them)
      st.j = 0;
      if (__builtin_expect(--st.left == 0, 0)) {
        stream_seek(st, a, smem, wave, cphase(a, st.q)->next_gemv);
      } else if (__builtin_expect(--st.seg_left == 0, 0)) {  // next expert block, or the wrap of a rotated range
        CPhase *ph = cphase(a, st.q);
        const int per = (int)gridDim.x / ph->S;
        const int s = (int)blockIdx.x / per;
        if (st.seg < 0) {  // back to the range's first tile
          int s1, w0, w1;
          unit_range(ph->T, ph->S, s1, w0, w1);
          st.seg = 0;
          st.seg_left = 0x40000000;
          stream_at(st, a, ph, smem, s, 0, w0, wave);
        } else {
          ++st.seg;
          st.seg_left = ph->seg_T;
          stream_at(st, a, ph, smem, s, st.seg, 0, wave);
        }
      } else {
        st.ptr += (int64_t)st.skip * 64;
        if (st.fmt == FMT_FP8R) {  // the run of the next tile
          st.kpos = st.kpos0;
          st.sbase += st.tile_words;
          st.sptr = st.sbase + (st.kpos >> 2) * 8;
        } else {
          st.sptr += (int64_t)st.skip * st.sstep;
        }
      }
    }
  }
}

// r[i] <- r[(i + head) % D]: puts the oldest in-flight item in slot 0 (waits for the ring to land)
template <int D, typename T>
__device__ __forceinline__ void ring_rotate(T (&r)[D], int head) {
  T t[D];
#pragma unroll
  for (int i = 0; i < D; ++i) t[i] = r[i];
#pragma unroll
  for (int h = 1; h < D; ++h) {
    if (head == h) {
#pragma unroll
      for (int i = 0; i < D; ++i) r[i] = t[(i + h) % D];
    }
  }
}

// ---------------------------------------------------------------------------------------------
// GEMV phase: Y = W * act, W packed as [tile][fragment][lane][8] bf16 (or NVFP4 groups)
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t lds_ld(uint32_t *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP); }

// Bounded wait for an LDS counter written by another wave of this workgroup. On expiry the step is
// marked timed out (status word) and the wait gives up, so every wave still reaches the kernel's end.
__device__ __forceinline__ void lds_wait_ge(uint32_t *p, uint32_t v, CArgs &a) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (lds_ld(p) < v) {
    __builtin_amdgcn_s_sleep(1);
    if ((int64_t)(__builtin_amdgcn_s_memrealtime() - t0) > a.timeout_ticks) {
      st_ci(a.status + 0, 6 /* MK_E_DEVICE_TIMEOUT */);
      st_ci(a.status + 2, 1);
      return;
    }
  }
}

// Bounded wait until a finaliser counter (written by other workgroups) reaches v; the abort flag is
// polled too. On expiry the step is marked timed out; false on expiry or abort.
__device__ __forceinline__ bool fin_wait(CArgs &a, const uint32_t *cnt, uint32_t v) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (uint32_t it = 0;; ++it) {
    const uint32_t c = ld_cu(cnt);
    const int32_t ab = (it & 15u) == 15u ? ld_ci(a.status + 2) : 0;
    if (c >= v) return true;
    if (ab != 0) return false;
    __builtin_amdgcn_s_sleep(1);
    if ((int64_t)(__builtin_amdgcn_s_memrealtime() - t0) > a.timeout_ticks) {
      st_ci(a.status + 0, 6 /* MK_E_DEVICE_TIMEOUT */);
      st_ci(a.status + 2, 1);
      return false;
    }
  }
}

// Activation pieces of a workgroup: one per segment its units touch when every segment has its own
// activation; one for all (the RMSNorm input of expert gate/up products and of unsegmented products).
__device__ __forceinline__ bool shared_act(const Phase &ph) { return ph.seg == SEG_NONE || ph.act == ACT_NORM; }
__device__ __forceinline__ int first_piece_seg(const Phase &ph, int u0) { return shared_act(ph) ? 0 : u0 / ph.seg_T; }
// B-operand layout of the activation fragments: per group of up to 8 rows, 16 columns holding the group's
// bf16 high halves, then its low halves. One group (2R columns) up to kMaxRows rows; above, two groups
// (rows 0..7 and 8..R-1) of 16 columns each, multiplied by two MFMAs per weight fragment.
template <bool WIDE>
__device__ __forceinline__ int act_stride(int R) { return WIDE ? 32 : 2 * R; }

// Stages the activation fragments of k-split s in LDS: for each piece (segment), row b and column k
// the fp32 value y, split into a bf16 high part and a bf16 low part (y - high), laid out as the B
// operand of v_mfma_f32_16x16x32_bf16 (per row group of Rg rows: columns 0..Rg-1 high parts,
// Rg..2Rg-1 low parts). For an RMSNorm
// input, y is x * gain: the per-row factor 1/rms is applied to the product's outputs (the product is
// linear). Expert down products scale each row's activation by its routing weight.
template <bool WIDE>
__device__ __forceinline__ void prep_act(CArgs &a, const Phase &ph, int s, int u0, int u1, char *smem) {
  const int R = a.R;
  const int nk = ph.nf * kFragK;
  const int k0 = s * nk;
  uint4 *act = reinterpret_cast<uint4 *>(smem + GemvLds::act);
  const int j0 = first_piece_seg(ph, u0);
  const int np = shared_act(ph) ? 1 : (u1 - 1) / ph.seg_T - j0 + 1;
  const RouteLds *rt = route_lds(smem);
  // each thread keeps one row b and walks the 8-column groups with a fixed stride; the loads of NB of
  // its groups are issued together (addresses clamped to a valid group, so none is conditional), then
  // the groups are converted and stored
  const int tpr = kThreads / R;  // threads per row
  const int b = (int)threadIdx.x % R, kg0 = (int)threadIdx.x / R;
  const int ngroups = (nk / 8) * np;
  const int C = act_stride<WIDE>(R);
  const int grp = WIDE ? b >> 3 : 0, bl = WIDE ? b & 7 : b, Rg = WIDE ? min(8, R - 8 * grp) : R;
  auto locate = [&](int gi, int &pc, int &kg) {  // group -> activation piece and 8-column group in it
    pc = 0;
    kg = gi;
    while (kg >= nk / 8) { kg -= nk / 8; ++pc; }
  };
  auto store = [&](const float (&y)[8], int pc, int kg) {
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      uint16_t h0 = f2bf(y[e]), h1 = f2bf(y[e + 1]);
      uint16_t l0 = f2bf(y[e] - bf2f(h0)), l1 = f2bf(y[e + 1] - bf2f(h1));
      hi[e >> 1] = (uint32_t)h0 | ((uint32_t)h1 << 16);
      lo[e >> 1] = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
    const int f = kg >> 2, g4 = kg & 3;
    uint4 *pa = act + (size_t)pc * (nk / 8) * C + grp * 16;
    pa[(f * 4 + g4) * C + bl] = uint4{hi[0], hi[1], hi[2], hi[3]};
    pa[(f * 4 + g4) * C + Rg + bl] = uint4{lo[0], lo[1], lo[2], lo[3]};
  };
  if (ph.stg_in != STG_NONE && np == 1) {
    // the producer wrote the fragments in this layout: copy the K slice into LDS, 1 KiB per wave and
    // instruction (direct-to-LDS loads, device-coherent), and wait for the copies before the barrier
    const int bytes = (nk / 8) * C * 16;
    const char *src = reinterpret_cast<const char *>(a.stg[ph.stg_in - 1]) + (size_t)(k0 / 8) * C * 16;
    const int w = (int)threadIdx.x >> 6, ln = (int)threadIdx.x & 63;
    for (int c = w; c * 1024 < bytes; c += kWavesTotal) {
      const int o = c * 1024 + ln * 16;
      if (o < bytes)
        __builtin_amdgcn_global_load_lds(src + o, (__attribute__((address_space(3))) void *)(reinterpret_cast<char *>(act) + c * 1024),
                                         16, 0, 16 /* sc1: device-coherent */);
    }
    __builtin_amdgcn_s_waitcnt(0);
    return;
  }
  if (threadIdx.x >= tpr * R) return;
  if (ph.act == ACT_NORM || ph.act == ACT_MIX) {
    constexpr int NB = 2;
    for (int gb = kg0; gb < ngroups; gb += NB * tpr) {
      float4 v0[NB], v1[NB];
      uint4 gg[NB];
      int pcs[NB], kgs[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        locate(min(gb + i * tpr, ngroups - 1), pcs[i], kgs[i]);
        const int k = k0 + kgs[i] * 8;
        if (ph.act == ACT_NORM) {
          const float *xp = a.x + (size_t)b * a.H + k;
          v0[i] = ld_c4(xp);
          v1[i] = ld_c4(xp + 4);
          gg[i] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(a.wbuf + ph.gain_off) + k);
        } else {
          const float *mp = a.mix + (size_t)b * a.mix_stride + ph.src_off + (j0 + pcs[i]) * ph.src_seg + k;
          v0[i] = ld_c4(mp);
          v1[i] = ld_c4(mp + 4);
        }
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (gb + i * tpr >= ngroups) continue;
        float y[8] = {v0[i].x, v0[i].y, v0[i].z, v0[i].w, v1[i].x, v1[i].y, v1[i].z, v1[i].w};
        if (ph.act == ACT_NORM) {
          const uint32_t gw[4] = {gg[i].x, gg[i].y, gg[i].z, gg[i].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] *= bf2f((uint16_t)(gw[e >> 1] >> ((e & 1) * 16)));
        }
        store(y, pcs[i], kgs[i]);
      }
    }
  } else {  // partial sums of an earlier product (k-splits summed), SwiGLU of gate and up rows
    constexpr int NB = 1;  // (more would spill the compute waves, whose registers hold the weight ring)
    const float *src = part_of(a, ph.src_part);
    for (int gb = kg0; gb < ngroups; gb += NB * tpr) {
      float g[NB][8], u[NB][8];
      int pcs[NB], kgs[NB], offs[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        locate(min(gb + i * tpr, ngroups - 1), pcs[i], kgs[i]);
        offs[i] = ph.src_off + (j0 + pcs[i]) * ph.src_seg + k0 + kgs[i] * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) g[i][e] = u[i][e] = 0.0f;
      }
      for (int s2 = 0; s2 < ph.src_S; ++s2) {
        float4 p0[NB], p1[NB], q0[NB], q1[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const float *row = src + ((size_t)s2 * R + b) * ph.src_N + offs[i];
          p0[i] = ld_c4(row);
          p1[i] = ld_c4(row + 4);
          if (ph.act == ACT_SWIGLU) {  // up rows follow the gate rows
            q0[i] = ld_c4(row + ph.K);
            q1[i] = ld_c4(row + ph.K + 4);
          }
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          g[i][0] += p0[i].x; g[i][1] += p0[i].y; g[i][2] += p0[i].z; g[i][3] += p0[i].w;
          g[i][4] += p1[i].x; g[i][5] += p1[i].y; g[i][6] += p1[i].z; g[i][7] += p1[i].w;
          if (ph.act == ACT_SWIGLU) {
            u[i][0] += q0[i].x; u[i][1] += q0[i].y; u[i][2] += q0[i].z; u[i][3] += q0[i].w;
            u[i][4] += q1[i].x; u[i][5] += q1[i].y; u[i][6] += q1[i].z; u[i][7] += q1[i].w;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (gb + i * tpr >= ngroups) continue;
        const float w = ph.seg == SEG_EXPERT ? rt->wt[j0 + pcs[i]][b] : 1.0f;
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = (ph.act == ACT_SWIGLU) ? silu(g[i][e]) * u[i][e] * w : g[i][e];
        store(y, pcs[i], kgs[i]);
      }
    }
  }
}

// Product phases whose tiles are completed by their last contributor (residual adds, split logits).
__device__ __forceinline__ bool needs_finalise(const Phase &ph) {
  return ph.out == OUT_RESID || (ph.out == OUT_LOGITS && ph.S > 1);
}

// Finalisation of one tile by the sync wave: every lane sums its (row, b) values of the tile over the
// partials in partial order (plus the residual), with the loads of 16 (8 above 8 rows) partials in flight at a time
// (an expert down product has one partial per (expert, k-split), so a tile can have over a hundred);
// device-coherent loads read the other contributors' partials (no cache invalidation). Stores the
// residual and the tile's sums of squares, or the logits and the argmax candidate of each row (kept by
// lane b).
template <int NK>  // 64-lane groups of (row, b) values: 16 R / 64, so 2 up to 8 rows, 4 up to 16
__device__ __forceinline__ void finalise_tiles(CArgs &a, const Phase &ph, int tile, int S_eff, int TN, float &best_v,
                                               int &best_i) {
  constexpr int kFinBatch = 32 / NK;  // partial loads in flight per lane group: 16 up to 8 rows, 8 above
  const int R = a.R, lane = threadIdx.x & 63;
  const float *pp = part_of(a, ph.dst_part);
  const size_t pstride = (size_t)R * TN;
  const bool resid = ph.out == OUT_RESID;
  int row_k[NK], b_k[NK];
  bool ok_k[NK];
  size_t off[NK];  // element offsets within a partial (a valid dummy for lanes without a value)
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const int idx = lane + 64 * k;
    ok_k[k] = idx < 16 * R;
    b_k[k] = ok_k[k] ? idx >> 4 : 0;  // lanes 16 b .. 16 b + 15: the tile's 16 rows of row b
    row_k[k] = idx & 15;
    off[k] = ok_k[k] ? (size_t)b_k[k] * TN + tile * kTileRows + row_k[k] : 0;
  }
  float kb_v[NK], acc[NK];  // logits: best of this lane's (row b_k) values; the sums
  int kb_i[NK];
#pragma unroll
  for (int k = 0; k < NK; ++k) { kb_v[k] = -INFINITY; kb_i[k] = 0x7fffffff; acc[k] = 0.0f; }
  for (int s0 = 0; s0 < S_eff; s0 += kFinBatch) {
    float t[kFinBatch][NK];
#pragma unroll
    for (int j = 0; j < kFinBatch; ++j) {
      const float *ps = pp + (size_t)min(s0 + j, S_eff - 1) * pstride;  // in bounds past the last partial
#pragma unroll
      for (int k = 0; k < NK; ++k) t[j][k] = s0 + j < S_eff ? ld_c(ps + off[k]) : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < kFinBatch; ++j)
      if (s0 + j < S_eff) {
#pragma unroll
        for (int k = 0; k < NK; ++k) acc[k] += t[j][k];
      }
  }
  float xv[NK];  // the residual values this tile updates (loaded together)
#pragma unroll
  for (int k = 0; k < NK; ++k)
    xv[k] = resid ? ld_c(a.x + (ok_k[k] ? (size_t)b_k[k] * a.H + tile * kTileRows + row_k[k] : 0)) : 0.0f;
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const int n = tile * kTileRows + row_k[k], b = b_k[k];
    float v = acc[k];
    if (resid) {
      if (ok_k[k]) {
        v += xv[k];
        st_c(a.x + (size_t)b * a.H + n, v);
        if (ph.stg_out) stg_put_x(a, ph, n, b, v);
      }
      float q2 = ok_k[k] ? v * v : 0.0f;  // sum of squares over the tile's 16 rows (16 consecutive lanes)
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) q2 += __shfl_xor(q2, o);
      if (ok_k[k] && row_k[k] == 0) st_c(a.ss + (size_t)b * (a.H / kTileRows) + tile, q2);
    } else if (ok_k[k]) {
      a.logits[(size_t)b * a.V + n] = v;
      if (v > kb_v[k] || (v == kb_v[k] && n < kb_i[k])) { kb_v[k] = v; kb_i[k] = n; }
    }
  }
  if (!resid) {  // per row: the first maximum over the finalised tiles, kept by lane b
    for (int b = 0; b < R; ++b) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int k = 0; k < NK; ++k)
        if (ok_k[k] && b_k[k] == b) { bv = kb_v[k]; bi = kb_i[k]; }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      if (lane == b && (bv > best_v || (bv == best_v && bi < best_i))) { best_v = bv; best_i = bi; }
    }
  }
}

// Eight NVFP4 weights of one lane -> bf16 (exact: an E2M1 value times an E4M3 scale has at most six
// significant bits). Element 2i is the low nibble of byte i.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
__device__ __forceinline__ bf16x8 nvfp4_frag(uint32_t codes, float scale) {
  f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
  f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
  f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
  f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
  bf16x2 b0 = __builtin_convertvector(p0 * scale, bf16x2), b1 = __builtin_convertvector(p1 * scale, bf16x2);
  bf16x2 b2 = __builtin_convertvector(p2 * scale, bf16x2), b3 = __builtin_convertvector(p3 * scale, bf16x2);
  return bf16x8{b0.x, b0.y, b1.x, b1.y, b2.x, b2.y, b3.x, b3.y};
}

// The scaled conversions below (v_cvt_scalef32_pk_bf16_*) multiply by two to the power of the scale
// operand's exponent field only, so they take power-of-two scales: an E8M0 byte e is passed as the
// float whose exponent field is e. Each conversion gives two bf16 weights, exact (an E2M1 value has two
// significant bits, an E4M3 value four, and the scales keep the products in bf16's normal range).

// Eight MXFP4 weights of one lane times their E8M0 block scale e -> bf16. Element 2i is the low nibble of
// byte i.
__device__ __forceinline__ bf16x8 mxfp4_frag(uint32_t codes, uint32_t e) {
  const float sc = __uint_as_float(e << 23);
  bf16x2 b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 0), b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 1);
  bf16x2 b2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 2), b3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 3);
  return bf16x8{b0.x, b0.y, b1.x, b1.y, b2.x, b2.y, b3.x, b3.y};
}

// Eight FP8 E4M3 weights of one lane (bytes of lo, then hi) times their power-of-two bf16 block scale ->
// bf16.
__device__ __forceinline__ bf16x8 fp8_frag(uint32_t lo, uint32_t hi, float scale) {
  bf16x2 b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, false), b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, true);
  bf16x2 b2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, false), b3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, true);
  return bf16x8{b0.x, b0.y, b1.x, b1.y, b2.x, b2.y, b3.x, b3.y};
}

// compute waves: consume this phase's items from the ring, refilling each slot from the stream.
// A finished 16-row unit is handed to the sync wave through an LDS slot and a counter, without a
// workgroup barrier, so the four waves never wait for each other inside a phase.
template <bool HAS_FP4, int D, bool WIDE>
__device__ __forceinline__ void gemv_run(CArgs &a, const Phase &ph, char *smem, uint4 (&ring)[D], uint32_t (&sring)[D],
                                         Stream &st, int &head, int s, int u0, int u1) {
  const int R = a.R;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const bool FP4 = HAS_FP4 && (ph.fmt == FMT_NVFP4 || ph.fmt == FMT_MXFP4);  // four FP4 fragments per item
  const bool MX = HAS_FP4 && ph.fmt == FMT_MXFP4;                             // their scales: E8M0, else E4M3
  const bool FP8 = HAS_FP4 && ph.fmt == FMT_FP8R;                             // two FP8 fragments per item
  const int nfw = wave_items(ph.nf, wave);        // fragments per unit run of this wave (a multiple of the
                                                  // fragments per item)
  const int ipr = FP4 ? nfw / 4 : (FP8 ? nfw / 2 : nfw);  // ring items per unit run
  const int total = (u1 - u0) * ipr;
  float *red = reinterpret_cast<float *>(smem + GemvLds::red);
  uint32_t *posted = reinterpret_cast<uint32_t *>(smem + GemvLds::flags);
  uint32_t *consumed = posted + kRedSlots;
  const int C = act_stride<WIDE>(R);              // activation columns of the B operand (both groups)
  const int R1 = WIDE ? R - 8 : 0;                // rows of the second group
  const int piece_u4 = ph.nf * 4 * C;             // uint4 per activation piece
  const uint4 *actv = reinterpret_cast<const uint4 *>(smem + GemvLds::act);
  const bool per_seg = !shared_act(ph);
  const int j0 = first_piece_seg(ph, u0);
  int c_j = 0, unit = 0;
  int seg_left = per_seg ? ph.seg_T - (u0 - j0 * ph.seg_T) : 0x40000000;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};  // acc1: rows 8.. (WIDE)
  const int col = lane & 15, kgrp = lane >> 4;
  const uint4 *aw = actv + (size_t)wave_first(ph.nf, wave) * 4 * C;
  auto close_unit = [&]() {  // combine hi/lo columns and post this wave's 16 x R partials
    float v[4], v1[4];
    const int R0 = WIDE ? 8 : R;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = acc[e] + __shfl_down(acc[e], R0);
      v1[e] = WIDE ? acc1[e] + __shfl_down(acc1[e], R1) : 0.0f;
    }
    const int sl = unit % kRedSlots;
    const uint32_t use = (uint32_t)(unit / kRedSlots);
    if (lds_ld(consumed + sl) < use) lds_wait_ge(consumed + sl, use, a);  // slot free (the sync wave read it)
    float *rb = red + (sl * kCWaves + wave) * 16 * kMaxBatch;
    if (col < R0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) rb[(kgrp * 4 + e) * kMaxBatch + col] = v[e];
    }
    if (WIDE && col < R1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) rb[(kgrp * 4 + e) * kMaxBatch + 8 + col] = v1[e];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane == 0) __hip_atomic_fetch_add(posted + sl, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    ++unit;
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
    c_j = 0;
    if (--seg_left == 0) {  // next segment: its own activation piece
      aw += piece_u4;
      seg_left = ph.seg_T;
    }
  };
  // one ring item: MFMA(s) with the activation fragment(s), refill the slot from the stream
  auto slot = [&](uint4 &r, uint32_t &sc) {
    if (FP8) {  // the lane's row scale: half (lane & 1) of the scale word
      const float s8 = __uint_as_float(((sc >> ((lane & 1) * 16)) & 0xFFFFu) << 16);
      const uint32_t cw[4] = {r.x, r.y, r.z, r.w};
      uint4 bv[2];  // the item's two activation fragments: their LDS reads in flight together
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        bv[f] = uint4{0u, 0u, 0u, 0u};
        if (col < 2 * R) bv[f] = aw[((c_j * 2 + f) * 4 + kgrp) * C + col];
      }
#pragma unroll
      for (int f = 0; f < 2; ++f)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8_frag(cw[2 * f], cw[2 * f + 1], s8), __builtin_bit_cast(bf16x8, bv[f]),
                                                      acc, 0, 0, 0);
    } else if (FP4) {
      const uint32_t cw[4] = {r.x, r.y, r.z, r.w};
      uint4 bv[4];  // the item's four activation fragments: their LDS reads in flight together
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        bv[f] = uint4{0u, 0u, 0u, 0u};
        if (col < 2 * R) bv[f] = aw[((c_j * 4 + f) * 4 + kgrp) * C + col];
      }
      if (MX) {  // E8M0 scales: byte f of the scale word
#pragma unroll
        for (int f = 0; f < 4; ++f)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mxfp4_frag(cw[f], (sc >> (8 * f)) & 255u), __builtin_bit_cast(bf16x8, bv[f]),
                                                        acc, 0, 0, 0);
      } else {  // E4M3 scales (not powers of two): converted, then multiplied in fp32
        float sc4[4];
        sc4[0] = __builtin_amdgcn_cvt_f32_fp8((int)sc, 0);
        sc4[1] = __builtin_amdgcn_cvt_f32_fp8((int)sc, 1);
        sc4[2] = __builtin_amdgcn_cvt_f32_fp8((int)sc, 2);
        sc4[3] = __builtin_amdgcn_cvt_f32_fp8((int)sc, 3);
#pragma unroll
        for (int f = 0; f < 4; ++f)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(nvfp4_frag(cw[f], sc4[f]), __builtin_bit_cast(bf16x8, bv[f]), acc, 0, 0, 0);
      }
    } else {
      uint4 bv = uint4{0u, 0u, 0u, 0u};
      if (col < (WIDE ? 16 : 2 * R)) bv = aw[(c_j * 4 + kgrp) * C + col];
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r), __builtin_bit_cast(bf16x8, bv), acc, 0,
                                                    0, 0);
      if (WIDE) {  // the second row group: the same weight fragment against its 16 columns
        uint4 bv1 = uint4{0u, 0u, 0u, 0u};
        if (col < 2 * R1) bv1 = aw[(c_j * 4 + kgrp) * C + 16 + col];
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r), __builtin_bit_cast(bf16x8, bv1), acc1,
                                                       0, 0, 0);
      }
    }
    stream_take<HAS_FP4>(st, a, smem, wave, lane, r, sc);  // the slot's old item is consumed: refill it
    if (__builtin_expect(++c_j == ipr, 0)) close_unit();
  };
  // full turns of the ring: every slot consumed and refilled once per turn, so each item is waited
  // for with D - 1 younger items still in flight
  const int turns = total / D;
  for (int it = 0; it < turns; ++it) {
#pragma unroll
    for (int d = 0; d < D; ++d) slot(ring[d], sring[d]);
  }
  const int rem = total - turns * D;
#pragma unroll
  for (int d = 0; d < D - 1; ++d)
    if (d < rem) slot(ring[d], sring[d]);
  head = rem;
}

template <bool HAS_FP4, int D, bool WIDE>
__device__ __forceinline__ void gemv_compute(CArgs &a, const Phase &ph, char *smem, uint4 (&ring)[D], uint32_t (&sring)[D],
                                             Stream &st, int &head) {
  int s, u0, u1;
  unit_range(phase_units(ph, smem), ph.S, s, u0, u1);
  if (head != 0) {
    ring_rotate(ring, head);
    ring_rotate(sring, head);
    head = 0;
  }
  if (u1 > u0) prep_act<WIDE>(a, ph, s, u0, u1, smem);
  lds_barrier();  // activation fragments ready, handoff counters cleared
  gemv_run<HAS_FP4, D, WIDE>(a, ph, smem, ring, sring, st, head, s, u0, u1);
}

// Dense gate|up product whose SwiGLU is staged: the designated workgroup of a 16-row pair t (gate tile t
// and up tile t + T/2, every k-split) sums the k-split partials in k-split order, as the product that
// reads them would, and writes silu(gate) * up of the pair's 16 columns for each row.
// Pairs t0, t0 + G, ... (up to kSwiBatch of them, all below Th) at once: every partial load in flight
// together (two k-splits at a time), then the sums, SwiGLU and staged writes. Five pairs per batch up
// to 8 rows, two above (the sync wave's registers).
template <int NK>
__device__ __forceinline__ void swiglu_pairs(CArgs &a, const Phase &ph, int t0, int n) {
  constexpr int kSwiBatch = NK == 2 ? 5 : 2;
  const int R = a.R, lane = threadIdx.x & 63, Th = ph.T / 2, G = gridDim.x;
  const float *pp = part_of(a, ph.dst_part);
  float g[kSwiBatch][NK], u[kSwiBatch][NK];
#pragma unroll
  for (int i = 0; i < kSwiBatch; ++i)
#pragma unroll
    for (int k = 0; k < NK; ++k) g[i][k] = u[i][k] = 0.0f;
  for (int s2 = 0; s2 < ph.S; s2 += 2) {
    const bool two = s2 + 1 < ph.S;
    float pg[kSwiBatch][NK][2], pu[kSwiBatch][NK][2];
#pragma unroll
    for (int i = 0; i < kSwiBatch; ++i)
#pragma unroll
      for (int k = 0; k < NK; ++k)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int idx = lane + 64 * k, row = idx & 15, b = idx < 16 * R ? idx >> 4 : 0;  // (a valid dummy)
          const int t = t0 + (i < n ? i : 0) * G;
          const float *pr = pp + ((size_t)(two ? s2 + h : s2) * R + b) * ph.N + row;
          pg[i][k][h] = ld_c(pr + (size_t)t * kTileRows);
          pu[i][k][h] = ld_c(pr + (size_t)(t + Th) * kTileRows);
        }
#pragma unroll
    for (int i = 0; i < kSwiBatch; ++i)
#pragma unroll
      for (int k = 0; k < NK; ++k)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (h == 1 && !two) continue;
          g[i][k] += pg[i][k][h];
          u[i][k] += pu[i][k][h];
        }
  }
#pragma unroll
  for (int i = 0; i < kSwiBatch; ++i)
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int idx = lane + 64 * k;
      if (i < n && idx < 16 * R) stg_put(a.stg[2], R, (t0 + i * G) * kTileRows + (idx & 15), idx >> 4, silu(g[i][k]) * u[i][k]);
    }
}

// Logits of a product split over k (counted after the workgroup's units): the designated workgroup of
// tiles t0, t0 + G, ... (n of them, up to kLogitBatch) sums each tile's partials in k-split order, with
// two k-splits' loads for all n tiles in flight at a time, stores the logits and keeps each row's first
// maximum (lane b holds row b's).
template <int NK>
__device__ __forceinline__ void logit_tiles(CArgs &a, const Phase &ph, int t0, int n, float &best_v, int &best_i) {
  constexpr int kLogitBatch = NK == 2 ? 8 : 4;
  const int R = a.R, lane = threadIdx.x & 63, G = gridDim.x;
  const float *pp = part_of(a, ph.dst_part);
  float acc[kLogitBatch][NK];
#pragma unroll
  for (int i = 0; i < kLogitBatch; ++i)
#pragma unroll
    for (int k = 0; k < NK; ++k) acc[i][k] = 0.0f;
  for (int s2 = 0; s2 < ph.S; s2 += 2) {
    const bool two = s2 + 1 < ph.S;
    float p[kLogitBatch][NK][2];
#pragma unroll
    for (int i = 0; i < kLogitBatch; ++i)
#pragma unroll
      for (int k = 0; k < NK; ++k)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int idx = lane + 64 * k, row = idx & 15, b = idx < 16 * R ? idx >> 4 : 0;  // (a valid dummy)
          const int t = t0 + (i < n ? i : 0) * G;
          p[i][k][h] = ld_c(pp + ((size_t)(two ? s2 + h : s2) * R + b) * ph.N + (size_t)t * kTileRows + row);
        }
#pragma unroll
    for (int i = 0; i < kLogitBatch; ++i)
#pragma unroll
      for (int k = 0; k < NK; ++k)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (h == 1 && !two) continue;
          acc[i][k] += p[i][k][h];
        }
  }
  float kb_v[NK];  // per lane: the best of its (row b) values over the n tiles, in increasing row order
  int kb_i[NK];
#pragma unroll
  for (int k = 0; k < NK; ++k) { kb_v[k] = -INFINITY; kb_i[k] = 0x7fffffff; }
#pragma unroll
  for (int i = 0; i < kLogitBatch; ++i)
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int idx = lane + 64 * k;
      if (i < n && idx < 16 * R) {
        const int nr = (t0 + i * G) * kTileRows + (idx & 15);
        a.logits[(size_t)(idx >> 4) * a.V + nr] = acc[i][k];
        if (acc[i][k] > kb_v[k]) { kb_v[k] = acc[i][k]; kb_i[k] = nr; }
      }
    }
  for (int b = 0; b < R; ++b) {  // per row: the first maximum over the wave, kept by lane b
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int k = 0; k < NK; ++k)
      if (lane + 64 * k < 16 * R && ((lane + 64 * k) >> 4) == b) { bv = kb_v[k]; bi = kb_i[k]; }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (lane == b && (bv > best_v || (bv == best_v && bi < best_i))) { best_v = bv; best_i = bi; }
  }
}

// sync wave: activation staging (with the compute waves), norm statistics, per-unit reduction and
// stores, finalisation
template <bool WIDE>
__device__ __forceinline__ void gemv_sync(CArgs &a, const Phase &ph, char *smem) {
  const int R = a.R, lane = threadIdx.x & 63;
  int s, u0, u1;
  unit_range(phase_units(ph, smem), ph.S, s, u0, u1);
  const int nunits = u1 - u0;
  float *red = reinterpret_cast<float *>(smem + GemvLds::red);
  uint32_t *posted = reinterpret_cast<uint32_t *>(smem + GemvLds::flags);
  uint32_t *consumed = posted + kRedSlots;
  float *misc = reinterpret_cast<float *>(smem + GemvLds::misc);
  float *rstd = misc;                                        // [kMaxBatch]
  int *flags = reinterpret_cast<int *>(misc + 16);           // [kMaxUnits]
  float *cval = misc + 16 + kMaxUnits;                       // [256]
  int *cidx = reinterpret_cast<int *>(cval + 256);           // [256]
  const RouteLds *rt = route_lds(smem);
  const bool direct = ph.out == OUT_LOGITS && ph.S == 1;
  const bool expert = ph.seg == SEG_EXPERT;
  // residual (and logits) finalisation: k-split partials per tile; expert down products: one partial
  // per (segment, k-split), summed in segment-major order
  const int S_eff = expert ? rt->nseg * ph.S : ph.S;
  const int TN = expert ? ph.seg_T * kTileRows : ph.N;  // rows of the finalised output
  if (lane < 2 * kRedSlots) posted[lane] = 0u;  // posted[] and consumed[] (adjacent)
  if (nunits > 0) prep_act<WIDE>(a, ph, s, u0, u1, smem);
  lds_barrier();  // activation fragments ready, handoff counters cleared
  if (ph.act == ACT_NORM) {  // 1/rms of each row from the per-tile sums of squares (while the waves stream)
    // every row's tile sums are loaded together, two tiles per lane at a time (one memory round per 128
    // tiles, not one per row), and added in tile order as before
    const int nt = a.H / kTileRows;
    float v[kMaxBatch];
#pragma unroll
    for (int b = 0; b < kMaxBatch; ++b) v[b] = 0.0f;
    for (int t0 = lane; t0 < nt; t0 += 128) {
      float x[2][kMaxBatch];
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int b = 0; b < kMaxBatch; ++b) {
          const int t = t0 + 64 * q;
          x[q][b] = (b < R && t < nt) ? ld_c(a.ss + (size_t)b * nt + t) : 0.0f;
        }
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int b = 0; b < kMaxBatch; ++b)
          if (t0 + 64 * q < nt) v[b] += x[q][b];
    }
#pragma unroll
    for (int b = 0; b < kMaxBatch; ++b) {
      if (b >= R) continue;
      const float w = wave_sum(v[b]);
      if (lane == 0) rstd[b] = 1.0f / sqrtf(w / (float)a.H + a.eps);
    }
    wave_lds_sync();
  }
  // lane groups k hold (row = idx / R, b = idx % R) for idx = lane + 64 k < 16 R: 2 groups up to 8 rows, 4 up to 16
  constexpr int NK = WIDE ? 4 : 2;
  float rs[NK], best_v[NK];
  int best_i[NK];
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    rs[k] = (ph.act == ACT_NORM && lane + 64 * k < 16 * R) ? rstd[(lane + 64 * k) % R] : 1.0f;
    best_v[k] = -INFINITY;
    best_i[k] = 0x7fffffff;
  }
  const float *ts = reinterpret_cast<const float *>(a.wbuf + ph.ts_off);
  const int nrot = u1 - u0, r0 = rotated(ph) ? rot_start(s, ph.S, nrot) : 0;
  const bool fin = needs_finalise(ph);
  const bool direct_resid = ph.out == OUT_RESID && S_eff == 1;
  // expert down products (a tile has one partial per (expert, k-split) and a workgroup many small units),
  // logits split over k and residual products split 8 or more ways (a workgroup has ten or more units,
  // and a per-unit acknowledgement and counter round trip would outlast the unit's weights):
  // contributions are counted once after all of this workgroup's units, and each tile is finalised by
  // one designated workgroup (tile t by workgroup t mod G) once its count is complete
  const bool deferred = fin && (expert || ph.out == OUT_LOGITS || ph.S >= 8) && !direct_resid;
  const bool swi = ph.out == OUT_PART && ph.stg_out;  // dense gate|up: SwiGLU of complete pairs, staged
  for (int unit = 0; unit < nrot; ++unit) {
    const int u = u0 + (r0 + unit < nrot ? r0 + unit : r0 + unit - nrot);
    const int sl = unit % kRedSlots;
    const uint32_t need = (uint32_t)(kCWaves * (unit / kRedSlots + 1));
    int j = 0, tl = u;  // segment and tile inside it (expert phases)
    float sc = 1.0f;
    if (expert) {
      j = u / ph.seg_T;
      tl = u - j * ph.seg_T;
      if (ph.fmt == FMT_NVFP4) {  // tensor scale of this expert's gate, up or down matrix
        const int which = ph.out == OUT_RESID ? 2 : (tl < ph.seg_T / 2 ? 0 : 1);
        sc = ts[rt->expert[j] * 3 + which];
      }
    }
    if (lds_ld(posted + sl) < need) lds_wait_ge(posted + sl, need, a);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    const float *rb = red + sl * kCWaves * 16 * kMaxBatch;
    float xsq[NK];
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      xsq[k] = 0.0f;
      const int idx = lane + 64 * k;
      if (idx < 16 * R) {
        const int row = idx / R, b = idx % R;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < kCWaves; ++w) v += rb[(w * 16 + row) * kMaxBatch + b];
        v *= rs[k] * sc;
        if (direct) {
          const int n = u * kTileRows + row;
          a.logits[(size_t)b * a.V + n] = v;
          if (v > best_v[k]) { best_v[k] = v; best_i[k] = n; }
        } else if (direct_resid) {  // one contributor: the unit's values are final
          const int n = u * kTileRows + row;
          const float xn = ld_c(a.x + (size_t)b * a.H + n) + v;
          st_c(a.x + (size_t)b * a.H + n, xn);
          if (ph.stg_out) stg_put_x(a, ph, n, b, xn);
          xsq[k] = xn * xn;
        } else if (expert && ph.out == OUT_RESID) {
          st_c(part_of(a, ph.dst_part) + ((size_t)(j * ph.S + s) * R + b) * TN + tl * kTileRows + row, v);
        } else {
          st_c(part_of(a, ph.dst_part) + ((size_t)s * R + b) * ph.N + u * kTileRows + row, v);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane == 0) __hip_atomic_store(consumed + sl, (uint32_t)(unit / kRedSlots + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (direct_resid) {  // the tile's sum of squares per row: lanes hold (row = idx / R, b = idx % R)
      float *sqs = misc + 16 + kMaxUnits + 512;  // [16][kMaxBatch]
#pragma unroll
      for (int k = 0; k < NK; ++k)
        if (lane + 64 * k < 16 * R) sqs[lane + 64 * k] = xsq[k];
      wave_lds_sync();
      if (lane < R) {
        float v = 0.0f;
        for (int row = 0; row < 16; ++row) v += sqs[row * R + lane];
        st_c(a.ss + (size_t)lane * (a.H / kTileRows) + u, v);
      }
      wave_lds_sync();
    } else if (fin && !deferred) {
      // count this contribution as soon as its partials are acknowledged; the last contributor of the
      // tile finalises it right away (while the compute waves stream the remaining units) and resets
      // the tile's counter for the next step
      __builtin_amdgcn_s_waitcnt(0);
      int last = 0;
      if (lane == 0) {
        uint32_t *cnt = a.fin + ph.cnt_off + tl;
        const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = old + 1u == (uint32_t)S_eff;
        if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (__shfl(last, 0)) finalise_tiles<NK>(a, ph, tl, S_eff, TN, best_v[0], best_i[0]);
    }
  }
  if (deferred || swi) {
    // expert down tiles: one count per (segment, k-split); logit tiles: one per k-split; dense gate|up
    // pairs: one per (gate or up tile, k-split). All of this workgroup's partials are acknowledged once,
    // then counted; each tile or pair is finalised by its designated workgroup (index mod G) when its
    // count is complete.
    __builtin_amdgcn_s_waitcnt(0);
    const int Th = ph.T / 2;
    uint32_t *cnt0 = a.fin + (swi ? ph.swi_cnt_off : ph.cnt_off);
    for (int unit = lane; unit < nrot; unit += 64) {
      const int u = u0 + unit;
      __hip_atomic_fetch_add(cnt0 + (swi ? (u < Th ? u : u - Th) : u % ph.seg_T), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const int nfin = swi ? Th : ph.seg_T;
    const uint32_t need = swi ? 2u * (uint32_t)ph.S : (uint32_t)S_eff;
    if (swi) {  // pairs in batches: wait for all of a batch's counts, then one round of loads for all
      constexpr int kSwiBatch = NK == 2 ? 5 : 2;
      for (int t0 = blockIdx.x; t0 < nfin; t0 += kSwiBatch * gridDim.x) {
        int n = 0;
        bool ok = true;
        for (int t = t0; ok && n < kSwiBatch && t < nfin; t += gridDim.x, ++n) ok = fin_wait(a, cnt0 + t, need);
        if (!ok) break;
        swiglu_pairs<NK>(a, ph, t0, n);
        if (lane < n) __hip_atomic_store(cnt0 + t0 + lane * gridDim.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else if (ph.out == OUT_LOGITS) {  // tiles in batches, like the pairs
      constexpr int kLogitBatch = NK == 2 ? 8 : 4;
      for (int t0 = blockIdx.x; t0 < nfin; t0 += kLogitBatch * gridDim.x) {
        int n = 0;
        bool ok = true;
        for (int t = t0; ok && n < kLogitBatch && t < nfin; t += gridDim.x, ++n) ok = fin_wait(a, cnt0 + t, need);
        if (!ok) break;
        logit_tiles<NK>(a, ph, t0, n, best_v[0], best_i[0]);
        if (lane < n) __hip_atomic_store(cnt0 + t0 + lane * gridDim.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      for (int t = blockIdx.x; t < nfin; t += gridDim.x) {
        uint32_t *cnt = cnt0 + t;
        if (!fin_wait(a, cnt, need)) break;
        finalise_tiles<NK>(a, ph, t, S_eff, TN, best_v[0], best_i[0]);
        if (lane == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // for the next step
      }
    }
  }
  if (ph.out == OUT_LOGITS) {  // per-workgroup argmax candidate of each row (first index on ties)
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      cval[lane + 64 * k] = best_v[k];
      cidx[lane + 64 * k] = best_i[k];
    }
    wave_lds_sync();
    if (lane < R) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int idx = lane; idx < 16 * R; idx += R) {
        const float v = cval[idx];
        const int ix = cidx[idx];
        if (v > bv || (v == bv && ix < bi)) { bv = v; bi = ix; }
      }
      st_c(a.cand + ((size_t)blockIdx.x * R + lane) * 2, bv);
      st_ci(reinterpret_cast<int32_t *>(a.cand) + ((size_t)blockIdx.x * R + lane) * 2 + 1, bi);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// gated delta rule: per (sequence, head, block of RPU state rows)
// ---------------------------------------------------------------------------------------------
// Per unit the head's normalised query and key, decay gate(s), write strength and the block's values
// are formed once (all five waves, one vector per wave task) into LDS while the block's state rows are
// already loading; then each compute wave advances RPU/4 state rows (two key channels per lane): with
// a the decay of each channel, S_r <- a * S_r; u = S_r . k; S_r <- S_r + beta (v_r - u) k; o_r = S_r . q.
// A verify block advances each state row through its 8 token rows in order and records every
// intermediate row (the snapshots the commit selects from).
constexpr int kDeltaMaxRpw = 16;  // state rows per compute wave and unit (units of up to 64 rows)
template <bool SYNCW>  // SYNCW: the sync wave's copy (it forms gates only; no state rows)
__device__ __forceinline__ void delta_phase(CArgs &a, const Phase &ph, char *smem) {
  const int R = a.R, Hl = a.lin_heads, dk = a.dk, dv = a.dv;
  const int RPU = a.verify ? ph.chunk_verify : ph.chunk, RPW = RPU / kCWaves;  // state rows per unit / wave
  const int RB = dv / RPU;
  const int nseq = a.verify ? 1 : R;
  const int nj = a.verify ? R : 1;  // token rows applied to each state row, in order
  const int U = nseq * Hl * RB;
  const int G = gridDim.x, wg = blockIdx.x;
  const int u0 = (int)(((int64_t)U * wg) / G), u1 = (int)(((int64_t)U * (wg + 1)) / G);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const float *src = part_of(a, ph.src_part);
  float *qh = reinterpret_cast<float *>(smem);  // [nj][dk]
  float *kh = qh + kMaxRows * 128;              // [nj][dk]
  float *al = kh + kMaxRows * 128;              // [nj][dk] decay per key channel
  float *be = al + kMaxRows * 128;              // [nj] write strength
  float *vv = be + kMaxRows;                    // [nj][RPU] values of the block's rows
  float *ov = vv + kMaxRows * 64;               // [nj][RPU] outputs, staged by the sync wave
  const int c0 = lane * 2;
  for (int u = u0; u < u1; ++u) {
    const int b = u / (Hl * RB), h = (u / RB) % Hl, rb = u % RB;
    // this wave's state rows (all of them at once) start loading before the gates are formed
    float2 S[kDeltaMaxRpw];
    float *Sw = reinterpret_cast<float *>(a.ls[ph.layer]) + (((size_t)b * Hl + h) * dv + rb * RPU + wave * RPW) * dk + c0;
#pragma unroll
    for (int i = 0; i < kDeltaMaxRpw; ++i)
      if (!SYNCW && wave < kCWaves && i < RPW) S[i] = *reinterpret_cast<const float2 *>(Sw + (size_t)i * dk);
    // gates and vectors: task t = (token row j, kind) for kinds q, k, decay + strength + values
    for (int t = wave; t < 3 * nj; t += kWavesTotal) {
      const int j = t / 3, kind = t - j * 3;
      const int row = a.verify ? j : b;
      if (kind < 2) {
        const int off = (kind == 0 ? ph.q_off : ph.k_off) + h * dk + c0;
        const float2 p2 = sum_splits2<4>(src + (size_t)row * ph.src_N + off, (size_t)R * ph.src_N, ph.src_S);
        const float x0 = p2.x, x1 = p2.y;
        const float n = 1.0f / sqrtf(wave_sum(x0 * x0 + x1 * x1) + 1e-6f);
        float *dst = (kind == 0 ? qh : kh) + j * 128 + c0;
        dst[0] = x0 * n;
        dst[1] = x1 * n;
      } else {
        float a0, a1 = 0.0f, vr = 0.0f;
        const float *pr = src + (size_t)row * ph.src_N;
        const size_t sst = (size_t)R * ph.src_N;
        if (ph.per_channel_gate) {
          const float2 p2 = sum_splits2<4>(pr + ph.a_off + h * dk + c0, sst, ph.src_S);
          a0 = p2.x;
          a1 = p2.y;
        } else {
          a0 = sum_splits<4>(pr + ph.a_off + h, sst, ph.src_S);
        }
        const float bb = sum_splits<4>(pr + ph.b_off + h, sst, ph.src_S);
        if (lane < RPU) vr = sum_splits<4>(pr + ph.v_off + h * dv + rb * RPU + lane, sst, ph.src_S);
        if (!ph.per_channel_gate) a1 = a0;
        al[j * 128 + c0] = __expf(-softplusf_(a0));
        al[j * 128 + c0 + 1] = ph.per_channel_gate ? __expf(-softplusf_(a1)) : al[j * 128 + c0];
        if (lane == 0) be[j] = sigmoidf_(bb);
        if (lane < RPU) vv[j * RPU + lane] = vr;
      }
    }
    lds_barrier();
    if (!SYNCW && wave < kCWaves) {
#pragma unroll
      for (int i = 0; i < kDeltaMaxRpw; ++i) {
        if (i >= RPW) continue;  // (no break: the loop unrolls fully and S stays in registers)
        const int rl = wave * RPW + i, r = rb * RPU + rl;
        float2 st = S[i];
        for (int j = 0; j < nj; ++j) {
          const float2 q2 = *reinterpret_cast<const float2 *>(qh + j * 128 + c0);
          const float2 k2 = *reinterpret_cast<const float2 *>(kh + j * 128 + c0);
          const float2 a2 = *reinterpret_cast<const float2 *>(al + j * 128 + c0);
          st.x *= a2.x;
          st.y *= a2.y;
          const float uu = wave_sum(st.x * k2.x + st.y * k2.y);
          const float delta = be[j] * (vv[j * RPU + rl] - uu);
          st.x += delta * k2.x;
          st.y += delta * k2.y;
          const float o = wave_sum(st.x * q2.x + st.y * q2.y);
          const int orow = a.verify ? j : b;
          if (lane == 0) {
            st_c(a.mix + (size_t)orow * a.mix_stride + h * dv + r, o);
            ov[j * RPU + rl] = o;
          }
          if (a.verify) {
            float *sn = a.snap + ((((size_t)ph.lin_idx * kMaxRows + j) * Hl + h) * dv + r) * dk + c0;
            st_c(sn, st.x);
            st_c(sn + 1, st.y);
          }
        }
        if (!a.verify) *reinterpret_cast<float2 *>(Sw + (size_t)i * dk) = st;
      }
    }
    lds_barrier();  // LDS gates are reused by the next unit
    if (SYNCW && ph.stg_out)  // the block's outputs, staged for the output projection (read before the
      for (int i = lane; i < nj * RPU; i += 64) {  // next unit's first barrier, after which they are rewritten)
        const int j = i / RPU, rr = rb * RPU + (i - j * RPU);
        stg_put(a.stg[1], R, h * dv + rr, a.verify ? j : b, ov[i]);
      }
  }
}

// bf16 high part (or low part: value minus high part) of eight fp32 values, packed
__device__ __forceinline__ uint4 pack_hi_lo(const float (&y)[8], bool lo) {
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    uint16_t h0 = f2bf(y[e]), h1 = f2bf(y[e + 1]);
    if (lo) { h0 = f2bf(y[e] - bf2f(h0)); h1 = f2bf(y[e + 1] - bf2f(h1)); }
    w[e >> 1] = (uint32_t)h0 | ((uint32_t)h1 << 16);
  }
  return uint4{w[0], w[1], w[2], w[3]};
}

// ---------------------------------------------------------------------------------------------
// split-KV grouped-query attention: per (query row, kv head, chunk of positions)
// ---------------------------------------------------------------------------------------------
// The query heads of one kv head (at most 8) take the 16 MFMA columns as bf16 high/low halves; per
// 64-position block the scores K (64 x d) * Q^T and the readout V^T (d x 64) * P run on
// v_mfma_f32_16x16x32_bf16 with the cached bf16 K/V rows as exact operands, softmax statistics kept
// online across blocks; the block's new rows (this step's tokens) are rotated, rounded to bf16 and
// appended. Partials (m, l, sum p v) per (row, query head, chunk) go to the merge phase.
constexpr int kGqaSub = 64;
template <int HD>
struct GqaLds {
  static constexpr int rowb = HD * 2 + 16;                  // padded LDS row of a staged K or V row (bytes)
  static constexpr int q = 0;                               // [HD/32 ks][4 kg][16 col] uint4
  static constexpr int k = q + (HD / 32) * 4 * 16 * 16;     // [64][rowb]
  static constexpr int v = k + kGqaSub * rowb;              // [64][rowb]
  static constexpr int s = v + kGqaSub * rowb;              // [64][8] f32 scores
  static constexpr int p = s + kGqaSub * 8 * 4;             // [2 kp][4 kg][16 col] uint4
  static constexpr int st = p + 2 * 4 * 16 * 16;            // m, l, alpha [8]
};

template <int HD, bool SYNCW>  // SYNCW: the sync wave's copy (it stages K/V rows only)
__device__ __forceinline__ void attn_phase(CArgs &a, const Phase &ph, char *smem) {
  typedef GqaLds<HD> L;
  const int R = a.R, nq = a.nq, nkv = a.nkv, grp = nq / nkv;
  const int CS = ph.chunk, NC = ph.n_chunks;
  const int U = R * nkv * NC;  // units: (row, kv head, chunk)
  const int G = gridDim.x, wg = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int u0 = (int)(((int64_t)U * wg) / G), u1 = (int)(((int64_t)U * (wg + 1)) / G);
  const float scale = 1.0f / sqrtf((float)HD);
  constexpr int half = HD / 2, KS = HD / 32;
  uint4 *Qb = reinterpret_cast<uint4 *>(smem + L::q);
  char *Ks = smem + L::k, *Vs = smem + L::v;
  float *Sc = reinterpret_cast<float *>(smem + L::s);
  uint4 *Pb = reinterpret_cast<uint4 *>(smem + L::p);
  float *mst = reinterpret_cast<float *>(smem + L::st), *lst = mst + 8, *alp = lst + 8;
  const float *src = part_of(a, ph.src_part);
  uint16_t *kc = reinterpret_cast<uint16_t *>(a.kc[ph.layer]);
  uint16_t *vc = reinterpret_cast<uint16_t *>(a.vc[ph.layer]);
  const float2 *rt = reinterpret_cast<const float2 *>(a.rope);
  const int col = lane & 15, kg = lane >> 4;
  for (int u = u0; u < u1; ++u) {
    const int row = u / (nkv * NC), g = (u / NC) % nkv, c = u % NC;
    const int seq = a.verify ? 0 : row;
    const int pbase = pos_at(a, ph, seq);
    const int prow = pbase + (a.verify ? row : 0);
    const int j0 = c * CS, j1 = min(j0 + CS, prow + 1);
    const size_t cbase = ((size_t)seq * nkv + g) * a.max_ctx;
    lds_barrier();  // the previous unit's LDS reads are done
    // queries of the group (rotated at prow) as the B operand
    for (int it = SYNCW ? 8 * (HD / 8) : tid; it < 8 * (HD / 8); it += kCWaves * 64) {
      const int hl = it / (HD / 8), d0 = (it - hl * (HD / 8)) * 8;
      float y[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (hl < grp) {
        const int h = g * grp + hl, pr = d0 < half ? d0 + half : d0 - half;
        float x[8] = {0, 0, 0, 0, 0, 0, 0, 0}, xp[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int s2 = 0; s2 < ph.src_S; ++s2) {
          const float *qr = src + ((size_t)s2 * R + row) * ph.src_N + ph.q_off + h * HD;
          add8(x, qr + d0);
          add8(xp, qr + pr);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float2 cs = rt[(size_t)prow * half + (d0 + e) % half];
          y[e] = d0 < half ? x[e] * cs.x - xp[e] * cs.y : xp[e] * cs.y + x[e] * cs.x;
        }
      }
      const int ks = d0 >> 5, kk = (d0 >> 3) & 3;
      Qb[(ks * 4 + kk) * 16 + hl] = pack_hi_lo(y, false);
      Qb[(ks * 4 + kk) * 16 + hl + 8] = pack_hi_lo(y, true);
    }
    if (!SYNCW && tid < 8) { mst[tid] = -INFINITY; lst[tid] = 0.0f; }
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    for (int jb = j0; jb < j1; jb += kGqaSub) {
      lds_barrier();
      // K/V rows of the block; this step's rows from the projections (rotated K, bf16), appended once
      for (int it = tid; it < kGqaSub * (HD / 8); it += kThreads) {
        const int jj = it / (HD / 8), d0 = (it - jj * (HD / 8)) * 8, j = jb + jj;
        uint4 kv = uint4{0u, 0u, 0u, 0u}, vv = uint4{0u, 0u, 0u, 0u};
        if (j < j1) {
          if (j < pbase) {
            kv = *reinterpret_cast<const uint4 *>(kc + (cbase + j) * HD + d0);
            vv = *reinterpret_cast<const uint4 *>(vc + (cbase + j) * HD + d0);
          } else {
            const int rr = a.verify ? j - pbase : row;
            const int pr = d0 < half ? d0 + half : d0 - half;
            float yk[8], x[8] = {0, 0, 0, 0, 0, 0, 0, 0}, xp[8] = {0, 0, 0, 0, 0, 0, 0, 0}, yv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            for (int s2 = 0; s2 < ph.src_S; ++s2) {
              const float *pp = src + ((size_t)s2 * R + rr) * ph.src_N;
              add8(x, pp + ph.k_off + g * HD + d0);
              add8(xp, pp + ph.k_off + g * HD + pr);
              add8(yv, pp + ph.v_off + g * HD + d0);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float2 cs = rt[(size_t)j * half + (d0 + e) % half];
              yk[e] = d0 < half ? x[e] * cs.x - xp[e] * cs.y : xp[e] * cs.y + x[e] * cs.x;
            }
            kv = pack_hi_lo(yk, false);
            vv = pack_hi_lo(yv, false);
            if (a.verify ? row == R - 1 : true) {  // one unit appends each new row
              *reinterpret_cast<uint4 *>(kc + (cbase + j) * HD + d0) = kv;
              *reinterpret_cast<uint4 *>(vc + (cbase + j) * HD + d0) = vv;
            }
          }
        }
        *reinterpret_cast<uint4 *>(Ks + jj * L::rowb + d0 * 2) = kv;
        *reinterpret_cast<uint4 *>(Vs + jj * L::rowb + d0 * 2) = vv;
      }
      lds_barrier();
      if (!SYNCW && wave < kCWaves) {  // scores: wave w takes positions jb + 16 w .. +15
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint4 av = *reinterpret_cast<const uint4 *>(Ks + (wave * 16 + col) * L::rowb + (ks * 32 + kg * 8) * 2);
          const uint4 bv = Qb[(ks * 4 + kg) * 16 + col];
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), sacc, 0,
                                                         0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = sacc[e] + __shfl_down(sacc[e], 8);
          const int pl = wave * 16 + kg * 4 + e;
          if (col < 8) Sc[pl * 8 + col] = (jb + pl < j1) ? v * scale : -INFINITY;
        }
      }
      lds_barrier();
      if (!SYNCW && tid < 8 * 16) {  // online softmax: 16 lanes per query, 4 positions each
        const int h = tid >> 4, q = tid & 15;
        float sv[4], bm = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sv[e] = Sc[(q * 4 + e) * 8 + h];
          bm = fmaxf(bm, sv[e]);
        }
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) bm = fmaxf(bm, __shfl_xor(bm, o));
        const float mo = mst[h], mn = fmaxf(mo, bm);
        float pv[4], ls = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pv[e] = mn == -INFINITY ? 0.0f : __expf(sv[e] - mn);
          ls += pv[e];
        }
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) ls += __shfl_xor(ls, o);
        const float o4[4] = {__shfl_xor(pv[0], 1), __shfl_xor(pv[1], 1), __shfl_xor(pv[2], 1), __shfl_xor(pv[3], 1)};
        if ((q & 1) == 0) {
          const float y[8] = {pv[0], pv[1], pv[2], pv[3], o4[0], o4[1], o4[2], o4[3]};
          const int gg = q >> 1, kp = gg >> 2, kk = gg & 3;
          Pb[(kp * 4 + kk) * 16 + h] = pack_hi_lo(y, false);
          Pb[(kp * 4 + kk) * 16 + h + 8] = pack_hi_lo(y, true);
        }
        if (q == 0) {
          const float al = mo == -INFINITY ? 0.0f : __expf(mo - mn);
          alp[h] = al;
          mst[h] = mn;
          lst[h] = lst[h] * al + ls;
        }
      }
      lds_barrier();
      if (!SYNCW && wave < kCWaves) {  // out^T += V^T P: wave w takes dims w * HD/4 .. (HD/64 row blocks)
        const float al = alp[col & 7];
#pragma unroll
        for (int rb = 0; rb < HD / 64; ++rb)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[rb][e] *= al;
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          const uint4 bv = Pb[(kp * 4 + kg) * 16 + col];
#pragma unroll
          for (int rb = 0; rb < HD / 64; ++rb) {
            const int dim = wave * (HD / 4) + rb * 16 + col;
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
              const uint16_t lo16 = *reinterpret_cast<const uint16_t *>(Vs + (kp * 32 + kg * 8 + i) * L::rowb + dim * 2);
              const uint16_t hi16 = *reinterpret_cast<const uint16_t *>(Vs + (kp * 32 + kg * 8 + i + 1) * L::rowb + dim * 2);
              w[i >> 1] = (uint32_t)lo16 | ((uint32_t)hi16 << 16);
            }
            acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, uint4{w[0], w[1], w[2], w[3]}),
                                                              __builtin_bit_cast(bf16x8, bv), acc[rb], 0, 0, 0);
          }
        }
      }
    }
    lds_barrier();  // final statistics visible
    const int W = HD + 2;
    if (!SYNCW && wave < kCWaves) {
#pragma unroll
      for (int rb = 0; rb < HD / 64; ++rb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = acc[rb][e] + __shfl_down(acc[rb][e], 8);
          if (col < grp && col < 8) {
            const int dim = wave * (HD / 4) + rb * 16 + kg * 4 + e;
            st_c(a.attn + (((size_t)row * nq + g * grp + col) * NC + c) * W + 2 + dim, v);
          }
        }
    }
    if (!SYNCW && tid < grp) {
      float *dst = a.attn + (((size_t)row * nq + g * grp + tid) * NC + c) * W;
      st_c(dst, mst[tid]);
      st_c(dst + 1, lst[tid]);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// absorbed multi-head latent attention: split-KV partials per (query row, chunk, head group)
// ---------------------------------------------------------------------------------------------
// The page "Kimi K3's TPU megakernel ..." (section "How it maps onto a TPU v7") runs latent attention
// in its absorbed form over a cache of latents: with q~_h = W_uk,h^T q_nope,h, every head scores
// s_j = (q~_h . c_j + q_rope,h . k_rope,j) / sqrt(nope + rope) against the shared [c_j | k_rope,j] row
// and reads out sum_j p_j c_j (the value up-projection follows as a separate product). Both
// contractions are dense: per 64-position block, scores = C (64 x D) * Q^T (D x heads) and
// out^T += C^T (rank x 64) * P (64 x heads) run on v_mfma_f32_16x16x32_bf16 with the latent rows as
// the exact bf16 operand and the fp32 queries / probabilities split into bf16 high and low halves
// (8 heads x {high, low} fill the 16 columns). Softmax statistics are kept online across blocks.
constexpr int kMlaSub = 64;        // positions per block (four compute waves x 16)
constexpr int kMlaMaxD = 576;      // latent rank + rotary width
constexpr int kMlaRowB = kMlaMaxD * 2 + 16;  // LDS row stride of a staged latent (bytes, padded)
constexpr int kMlaHeads = 8;       // heads per unit: 8 x {high, low} fill the 16 MFMA columns
struct MlaLds {
  static constexpr int q = 0;                                  // [18 ks][4 kg][16 col] uint4
  static constexpr int c = q + (kMlaMaxD / 32) * 4 * 16 * 16;  // [64][kMlaRowB] bf16 latents
  static constexpr int s = c + kMlaSub * kMlaRowB;             // [64 pos][8 heads] f32 scores
  static constexpr int p = s + kMlaSub * kMlaHeads * 4;        // [2 kp][4 kg][16 col] uint4
  static constexpr int st = p + 2 * 4 * 16 * 16;               // m, l, alpha [8 heads] each
  static constexpr int end = st + 3 * kMlaHeads * 4;
};
static_assert(MlaLds::end <= kLdsBytes, "latent attention LDS layout exceeds the workgroup's LDS");


__device__ __forceinline__ void mla_phase(CArgs &a, const Phase &ph, char *smem) {
  const int R = a.R, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rank = ph.rank, rope = ph.rope, D = rank + rope, KS = D / 32, half = rope / 2;
  const int HG = kMlaHeads, NHG = (ph.heads + HG - 1) / HG;
  const int CS = ph.chunk, NC = ph.n_chunks;
  const int nrow = a.verify ? R : 1;             // query rows per sequence
  const int U = R * NC * NHG;                    // units: (row, chunk, head group)
  const int G = gridDim.x, wg = blockIdx.x;
  const int u0 = (int)(((int64_t)U * wg) / G), u1 = (int)(((int64_t)U * (wg + 1)) / G);
  const float scale = 1.0f / sqrtf((float)(ph.nope + rope));
  uint4 *Qb = reinterpret_cast<uint4 *>(smem + MlaLds::q);
  char *Cs = smem + MlaLds::c;
  float *Sc = reinterpret_cast<float *>(smem + MlaLds::s);
  uint4 *Pb = reinterpret_cast<uint4 *>(smem + MlaLds::p);
  float *mst = reinterpret_cast<float *>(smem + MlaLds::st), *lst = mst + kMlaHeads, *alp = lst + kMlaHeads;
  const float *src = part_of(a, ph.src_part);
  const float *qt = part_of(a, ph.mla_src);      // absorbed queries [R][heads * rank] (one split)
  const float2 *rt = reinterpret_cast<const float2 *>(a.rope_mla);
  uint16_t *cache = reinterpret_cast<uint16_t *>(a.lat[ph.layer]);
  const int col = lane & 15, kg = lane >> 4;
  for (int u = u0; u < u1; ++u) {
    // unit order (head group, row, chunk): the head groups of one (row, chunk) sit G/NHG apart
    const int hg = u / (R * NC), rc = u - hg * (R * NC), row = rc / NC, c = rc - row * NC;
    const int seq = a.verify ? 0 : row;
    const int pbase = pos_at(a, ph, seq);
    const int prow = pbase + (a.verify ? row : 0);  // this row attends positions 0 .. prow
    const int j0 = c * CS, j1 = min(j0 + CS, prow + 1);
    const int h0 = hg * HG;
    lds_barrier();  // the previous unit's LDS reads are done
    // ---- queries of the group's heads as the B operand (rotary part rotated at prow) ----
    for (int it = tid; it < HG * (D / 8); it += kThreads) {
      const int hl = it / (D / 8), g = it - hl * (D / 8), h = h0 + hl, d0 = g * 8;
      float y[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (h < ph.heads) {
        if (d0 < rank) {
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = ld_c(qt + (size_t)row * ph.heads * rank + (size_t)h * rank + d0 + e);
        } else {
          const int r0 = d0 - rank;  // rotary dims r0..r0+7, partner dims at +-half
          const int pr = r0 < half ? r0 + half : r0 - half;
          float x[8] = {0, 0, 0, 0, 0, 0, 0, 0}, xp[8] = {0, 0, 0, 0, 0, 0, 0, 0};
          for (int s2 = 0; s2 < ph.src_S; ++s2) {
            const float *pr_row = src + ((size_t)s2 * R + row) * ph.src_N + ph.q_off + h * ph.qk_stride + ph.nope;
            add8(x, pr_row + r0);
            add8(xp, pr_row + pr);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float2 cs = rt[(size_t)prow * half + (r0 + e) % half];
            y[e] = r0 < half ? x[e] * cs.x - xp[e] * cs.y : xp[e] * cs.y + x[e] * cs.x;
          }
        }
      }
      const int ks = g >> 2, kk = g & 3;
      Qb[(ks * 4 + kk) * 16 + hl] = pack_hi_lo(y, false);
      Qb[(ks * 4 + kk) * 16 + hl + 8] = pack_hi_lo(y, true);
    }
    if (tid < kMlaHeads) { mst[tid] = -INFINITY; lst[tid] = 0.0f; }
    f32x4 acc[8];
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int jb = j0; jb < j1; jb += kMlaSub) {
      lds_barrier();  // queries staged / the previous block's reads of Cs and Pb are done
      // ---- stage 64 latent rows (new rows computed from the projections and appended) ----
      for (int it = tid; it < kMlaSub * (D / 8); it += kThreads) {
        const int jj = it / (D / 8), g = it - jj * (D / 8), j = jb + jj, d0 = g * 8;
        uint4 v = uint4{0u, 0u, 0u, 0u};
        if (j < j1) {
          if (j < pbase) {
            v = *reinterpret_cast<const uint4 *>(cache + ((size_t)seq * a.max_ctx + j) * D + d0);
          } else {  // a row of this step: latent rank part, or the rotated key part, rounded to bf16
            const int rr = a.verify ? j - pbase : row;
            float y[8];
            if (d0 < rank) {
#pragma unroll
              for (int e = 0; e < 8; ++e) y[e] = 0.0f;
              for (int s2 = 0; s2 < ph.src_S; ++s2) add8(y, src + ((size_t)s2 * R + rr) * ph.src_N + ph.dkv_off + d0);
            } else {
              const int r0 = d0 - rank, pr = r0 < half ? r0 + half : r0 - half;
              float x[8] = {0, 0, 0, 0, 0, 0, 0, 0}, xp[8] = {0, 0, 0, 0, 0, 0, 0, 0};
              for (int s2 = 0; s2 < ph.src_S; ++s2) {
                const float *kr = src + ((size_t)s2 * R + rr) * ph.src_N + ph.kr_off;
                add8(x, kr + r0);
                add8(xp, kr + pr);
              }
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const float2 cs = rt[(size_t)j * half + (r0 + e) % half];
                y[e] = r0 < half ? x[e] * cs.x - xp[e] * cs.y : xp[e] * cs.y + x[e] * cs.x;
              }
            }
            v = pack_hi_lo(y, false);
            if (hg == 0 && (a.verify ? row == R - 1 : true))  // one unit appends each new row
              *reinterpret_cast<uint4 *>(cache + ((size_t)seq * a.max_ctx + j) * D + d0) = v;
          }
        }
        *reinterpret_cast<uint4 *>(Cs + jj * kMlaRowB + d0 * 2) = v;
      }
      lds_barrier();
      // ---- scores: wave w takes positions jb + 16 w .. +15 ----
      if (wave < kCWaves) {
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
        for (int ks = 0; ks < KS; ++ks) {
          const uint4 av = *reinterpret_cast<const uint4 *>(Cs + (wave * 16 + col) * kMlaRowB + (ks * 32 + kg * 8) * 2);
          const uint4 bv = Qb[(ks * 4 + kg) * 16 + col];
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), sacc, 0,
                                                         0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = sacc[e] + __shfl_down(sacc[e], 8);  // high + low columns
          const int pl = wave * 16 + kg * 4 + e;
          if (col < 8) Sc[pl * kMlaHeads + col] = (jb + pl < j1) ? v * scale : -INFINITY;
        }
      }
      lds_barrier();
      // ---- online softmax: 16 lanes per head, 4 positions each ----
      if (tid < HG * 16) {
        const int h = tid >> 4, q = tid & 15;
        float sv[4], bm = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sv[e] = Sc[(q * 4 + e) * kMlaHeads + h];
          bm = fmaxf(bm, sv[e]);
        }
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) bm = fmaxf(bm, __shfl_xor(bm, o));
        const float mo = mst[h], mn = fmaxf(mo, bm);
        float pv[4], ls = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pv[e] = mn == -INFINITY ? 0.0f : __expf(sv[e] - mn);
          ls += pv[e];
        }
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) ls += __shfl_xor(ls, o);
        // P as the B operand: positions q*4 .. q*4+3 of head h (two lanes make one group of 8)
        const float o4[4] = {__shfl_xor(pv[0], 1), __shfl_xor(pv[1], 1), __shfl_xor(pv[2], 1), __shfl_xor(pv[3], 1)};
        if ((q & 1) == 0) {
          const float y[8] = {pv[0], pv[1], pv[2], pv[3], o4[0], o4[1], o4[2], o4[3]};
          const int g = q >> 1, kp = g >> 2, kk = g & 3;
          Pb[(kp * 4 + kk) * 16 + h] = pack_hi_lo(y, false);
          Pb[(kp * 4 + kk) * 16 + h + 8] = pack_hi_lo(y, true);
        }
        if (q == 0) {
          const float al = mo == -INFINITY ? 0.0f : __expf(mo - mn);
          alp[h] = al;
          mst[h] = mn;
          lst[h] = lst[h] * al + ls;
        }
      }
      lds_barrier();
      // ---- out^T += C^T P: wave w takes latent dims 128 w .. +127 (8 row blocks) ----
      if (wave < kCWaves && wave * 128 < rank) {
        const float al = alp[col & 7];
#pragma unroll
        for (int rb = 0; rb < 8; ++rb)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[rb][e] *= al;
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          const uint4 bv = Pb[(kp * 4 + kg) * 16 + col];
#pragma unroll
          for (int rb = 0; rb < 8; ++rb) {
            const int dim = wave * 128 + rb * 16 + col;
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
              const uint16_t lo16 = *reinterpret_cast<const uint16_t *>(Cs + (kp * 32 + kg * 8 + i) * kMlaRowB + dim * 2);
              const uint16_t hi16 = *reinterpret_cast<const uint16_t *>(Cs + (kp * 32 + kg * 8 + i + 1) * kMlaRowB + dim * 2);
              w[i >> 1] = (uint32_t)lo16 | ((uint32_t)hi16 << 16);
            }
            acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, uint4{w[0], w[1], w[2], w[3]}),
                                                              __builtin_bit_cast(bf16x8, bv), acc[rb], 0, 0, 0);
          }
        }
      }
    }
    lds_barrier();  // final statistics visible
    // ---- partials: [row][head][chunk][rank + 2] = (m, l, sum_j p_j c_j) ----
    const int W = rank + 2;
    if (wave < kCWaves && wave * 128 < rank) {
#pragma unroll
      for (int rb = 0; rb < 8; ++rb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = acc[rb][e] + __shfl_down(acc[rb][e], 8);
          const int h = h0 + col;
          if (col < 8 && h < ph.heads) {
            const int dim = wave * 128 + rb * 16 + kg * 4 + e;
            st_c(a.attn + (((size_t)row * ph.heads + h) * NC + c) * W + 2 + dim, v);
          }
        }
    }
    if (tid < HG && h0 + tid < ph.heads) {
      float *dst = a.attn + (((size_t)row * ph.heads + h0 + tid) * NC + c) * W;
      st_c(dst, mst[tid]);
      st_c(dst + 1, lst[tid]);
    }
  }
}

// Log-sum-exp merge of split-KV partials (m, l, sum p v) over chunks, per (row, query head): grouped
// query attention (head width hd) or latent attention (latent rank).
template <bool SYNCW>  // SYNCW: the sync wave's copy (it also writes the staged outputs)
__device__ __forceinline__ void merge_phase(CArgs &a, const Phase &ph, char *smem) {
  const bool mla = ph.type == PH_MLA_MERGE;
  const int R = a.R, nq = mla ? ph.heads : a.nq, hd = mla ? ph.rank : a.hd, NC = ph.n_chunks, W = hd + 2;
  const int U = R * nq;
  const int G = gridDim.x, wg = blockIdx.x, tid = threadIdx.x;
  const int u0 = (int)(((int64_t)U * wg) / G), u1 = (int)(((int64_t)U * (wg + 1)) / G);
  float *pl = reinterpret_cast<float *>(smem);  // [NC][hd + 2]
  float *wt = pl + NC * W;                       // [NC] weights, then [1] total
  float *ov = wt + NC + 1;                       // [hd] outputs, staged by the sync wave
  for (int u = u0; u < u1; ++u) {
    const int row = u / nq, h = u % nq;
    const float *p = a.attn + ((size_t)row * nq + h) * NC * W;
    lds_barrier();
    // the chunks' partials, eight loads per thread in flight before the first is stored
    for (int i0 = tid; i0 < NC * W; i0 += 8 * kThreads) {
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = i0 + q * kThreads;
        v[q] = i < NC * W ? ld_c(p + i) : 0.0f;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = i0 + q * kThreads;
        if (i < NC * W) pl[i] = v[q];
      }
    }
    lds_barrier();
    if (tid < 64) {  // one wave: global max and normaliser over chunks, in chunk order per lane
      float M = -INFINITY;
      for (int c = tid; c < NC; c += 64)
        if (pl[c * W + 1] > 0.0f) M = fmaxf(M, pl[c * W]);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
      float L = 0.0f;
      for (int c = tid; c < NC; c += 64) {
        const float l = pl[c * W + 1];
        const float w = l > 0.0f ? __expf(pl[c * W] - M) : 0.0f;
        wt[c] = w;
        L += l * w;
      }
      L = wave_sum(L);
      if (tid == 0) wt[NC] = L;
    }
    lds_barrier();
    const float L = wt[NC];
    for (int i = tid; i < hd; i += kThreads) {
      float o = 0.0f;
      for (int c = 0; c < NC; ++c) o += pl[c * W + 2 + i] * wt[c];
      st_c(a.mix + (size_t)row * a.mix_stride + h * hd + i, o / L);
      if (ph.stg_out) ov[i] = o / L;
    }
    if (ph.stg_out) {
      lds_barrier();
      if (SYNCW)
        for (int i = tid & 63; i < hd; i += 64) stg_put(a.stg[1], R, h * hd + i, row, ov[i]);
    }
  }
}

template <bool SYNCW>  // the sync wave embeds (16 values per unit); the other waves only keep the barriers
__device__ __forceinline__ void embed_phase(CArgs &a, const Phase &ph, char *smem) {
  const int R = a.R, H = a.H, nt = H / kTileRows;
  const int U = R * nt;
  const int G = gridDim.x, wg = blockIdx.x, tid = threadIdx.x;
  const int u0 = (int)(((int64_t)U * wg) / G), u1 = (int)(((int64_t)U * (wg + 1)) / G);
  float *sq = reinterpret_cast<float *>(smem);
  const uint16_t *E = reinterpret_cast<const uint16_t *>(a.wbuf + ph.w_off);
  for (int u = u0; u < u1; ++u) {
    const int row = u / nt, t = u % nt;
    lds_barrier();
    const int ln = tid & 63;
    if (SYNCW && ln < kTileRows) {
      const int n = t * kTileRows + ln;
      float v;
      if (a.V > 0) {
        // the first step embeds the caller's tokens; a later step of a multi-step launch the token the
        // previous step emitted (written by workgroup 0 before the grid barrier)
        int tok = ph.step == 0 ? a.tokens[row] : ld_ci(a.loop_tokens + (size_t)(ph.step - 1) * a.R + row);
        if (tok < 0 || tok >= a.V) {  // out-of-range token: report, read row 0 instead of faulting
          if (ln == 0) { st_ci(a.status + 1, -2); st_ci(a.status + 0, 1 /* MK_E_ARG */); }
          tok = 0;
        }
        v = bf2f(E[(size_t)tok * H + n]);
      }
      else v = a.hidden_in[(size_t)row * H + n];
      st_c(a.x + (size_t)row * H + n, v);
      if (ph.stg_out) stg_put_x(a, ph, n, row, v);
      sq[ln] = v * v;
    }
    lds_barrier();
    if (SYNCW && ln == 0) {
      float s = 0.0f;
      for (int i = 0; i < kTileRows; ++i) s += sq[i];
      st_c(a.ss + (size_t)row * nt + t, s);
    }
  }
}

__device__ __forceinline__ void final_phase(CArgs &a, const Phase &ph, char *smem) {
  const int R = a.R, G = gridDim.x, tid = threadIdx.x;
  float *cv = reinterpret_cast<float *>(smem);
  int *ci = reinterpret_cast<int *>(cv + G * kMaxBatch);
  int *am = ci + G * kMaxBatch;
  int *acc_s = am + kMaxBatch;
  if (a.V > 0) {
    for (int idx = tid; idx < G * R; idx += kThreads) {
      cv[idx] = ld_c(a.cand + (size_t)idx * 2);
      ci[idx] = ld_ci(reinterpret_cast<const int32_t *>(a.cand) + (size_t)idx * 2 + 1);
    }
    lds_barrier();
    if (tid < R) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int w = 0; w < G; ++w) {
        const float v = cv[w * R + tid];
        const int ix = ci[w * R + tid];
        if (v > bv || (v == bv && ix < bi)) { bv = v; bi = ix; }
      }
      am[tid] = bi;
      if (blockIdx.x == 0 && a.argmax) a.argmax[tid] = bi;
      if (blockIdx.x == 0 && a.loop_tokens) st_ci(a.loop_tokens + (size_t)ph.step * R + tid, bi);
    }
    lds_barrier();
  }
  if (a.verify) {
    if (tid == 0) {
      int acc = 0;
      while (acc < R - 1 && a.tokens[acc + 1] == am[acc]) ++acc;
      acc_s[0] = acc;
      if (blockIdx.x == 0) {
        if (a.accepted) a.accepted[0] = acc;
        if (a.bonus) a.bonus[0] = am[acc];
      }
    }
    lds_barrier();
    const int acc = acc_s[0];
    // commit: live state <- snapshot after row acc, for every linear-attention layer
    const size_t per = (size_t)a.lin_heads * a.dv * a.dk;
    const size_t total4 = (size_t)a.n_lin * per / 4;
    for (size_t idx = (size_t)blockIdx.x * kThreads + tid; idx < total4; idx += (size_t)G * kThreads) {
      const size_t e = idx * 4, li = e / per, off = e % per;
      const float *sn = a.snap + ((li * kMaxRows + acc) * per) + off;
      float4 v = make_float4(ld_c(sn), ld_c(sn + 1), ld_c(sn + 2), ld_c(sn + 3));
      *reinterpret_cast<float4 *>(reinterpret_cast<float *>(a.lsl[li]) + off) = v;
    }
  }
}

__device__ __forceinline__ void hidden_out_phase(CArgs &a) {
  const size_t n = (size_t)a.R * a.H;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (size_t)gridDim.x * kThreads)
    a.hidden_out[i] = ld_c(a.x + i);
}

}  // namespace mk

using namespace mk;

// Phases that every wave runs the same way; their results are acknowledged before the grid barrier.
template <bool SYNCW>  // SYNCW: the sync wave's copy of the phase loop
__device__ __forceinline__ void common_phase(CArgs &a, const Phase &ph, char *smem) {
  switch (ph.type) {
    case PH_EMBED: embed_phase<SYNCW>(a, ph, smem); break;
    case PH_DELTA: delta_phase<SYNCW>(a, ph, smem); break;
    case PH_ATTN:
      if (a.hd == 64) attn_phase<64, SYNCW>(a, ph, smem);
      else attn_phase<128, SYNCW>(a, ph, smem);
      break;
    case PH_MERGE:
    case PH_MLA_MERGE: merge_phase<SYNCW>(a, ph, smem); break;
    case PH_MLA: mla_phase(a, ph, smem); break;
    case PH_FINAL: final_phase(a, ph, smem); break;
    case PH_HIDDEN_OUT: hidden_out_phase(a); break;
    default: break;
  }
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();
}

// The step kernel: walks phases [phase_begin, phase_end) of the schedule. As a persistent launch it
// covers the whole step with a grid barrier between phases (all workgroups co-resident: cooperative
// launch, one workgroup per compute unit); the per-op baseline launches it once per phase.
// Waves 0..kCWaves-1 stream weights (their ring is never drained at a phase end: the loads of the next
// product phase are in flight through barriers and the phases in between); wave kSyncWave reduces,
// stores cross-workgroup results and runs the grid barrier. The two kinds of wave run separate copies
// of the phase loop with the same sequence of workgroup barriers, so the weight ring is not live in
// the sync wave's code.
template <bool HAS_FP4, int RING, bool WIDE = false>
__device__ __forceinline__ void step_body(char *smem) {
  CArgs *ap = (CArgs *)__builtin_amdgcn_kernarg_segment_ptr();
  __shared__ int abort_flag;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  int route_q = -1;  // expert gate/up phase whose routing this workgroup holds in LDS
  if (wave == kSyncWave) {
    uint32_t k = ap->bar_done + (uint32_t)ap->barrier_base;
    for (int p = ap->phase_begin; p < ap->phase_end; ++p) {
      CArgs &a = *ap;
      const Phase ph = load_phase(a, p);
      if (a.trace && lane == 0) a.trace[((size_t)p * gridDim.x + blockIdx.x) * 2] = __builtin_amdgcn_s_memrealtime();
      if (ph.type == PH_GEMV) {
        if (ph.seg == SEG_EXPERT && route_q != ph.route_q) {
          compute_route(a, ph, smem);
          route_q = ph.route_q;
        }
        gemv_sync<WIDE>(a, ph, smem);
      } else {
        common_phase<true>(a, ph, smem);
      }
      __builtin_amdgcn_s_waitcnt(0);  // this wave's stores are acknowledged before the barrier
      if (lane == 0) {
        if (a.trace) a.trace[((size_t)p * gridDim.x + blockIdx.x) * 2 + 1] = __builtin_amdgcn_s_memrealtime();
        int ok = 1;
        if (p + 1 < a.phase_end) ok = grid_arrive_wait(a, k + 1, p);
        abort_flag = !ok;
      }
      ++k;
      lds_barrier();
      if (abort_flag) return;
    }
  } else {
    uint4 ring[RING];
    uint32_t sring[RING];
    Stream st;
    int head = 0;
    st.route_q = -1;
    {
      CArgs &a = *ap;
      int q = a.phase_begin;
      while (q < a.phase_end && cphase(a, q)->type != PH_GEMV) ++q;
      stream_seek(st, a, smem, wave, q < a.phase_end ? q : -1);
#pragma unroll
      for (int d = 0; d < RING; ++d) stream_take<HAS_FP4>(st, a, smem, wave, lane, ring[d], sring[d]);
    }
    for (int p = ap->phase_begin; p < ap->phase_end; ++p) {
      CArgs &a = *ap;
      const Phase ph = load_phase(a, p);
      if (ph.type == PH_GEMV) {
        if (ph.seg == SEG_EXPERT && route_q != ph.route_q) {
          compute_route(a, ph, smem);
          route_q = ph.route_q;
        }
        if (st.blocked == p) {  // the stream waited here for the routing: every ring slot is a dummy
          st.route_q = route_q;
          stream_seek(st, a, smem, wave, p);
#pragma unroll
          for (int d = 0; d < RING; ++d) stream_take<HAS_FP4>(st, a, smem, wave, lane, ring[d], sring[d]);
          head = 0;
          // the refilled slots land before the ring loop: otherwise the compiler's wait counts for the
          // loop (which joins this path) assume these loads may still be in flight and drain the ring
          __builtin_amdgcn_s_waitcnt(0);
        }
        gemv_compute<HAS_FP4, RING, WIDE>(a, ph, smem, ring, sring, st, head);
      } else {
        common_phase<false>(a, ph, smem);
      }
      lds_barrier();
      if (abort_flag) return;
    }
  }
}
