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
// Cross-workgroup data is written with agent-scope (sc1, write-through) stores and read after a
// barrier whose acquire side invalidates this XCD's L2, or with sc1 loads inside a phase.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_internal.h"

namespace mk {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

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
__device__ __forceinline__ uint32_t ld_cu(const uint32_t *p) {
  return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint4 ld_nt(const uint4 *p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return uint4{v.x, v.y, v.z, v.w};
}

// workgroup barrier that orders LDS only (global memory is ordered explicitly where needed)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }
__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + __expf(-z)); }
__device__ __forceinline__ float softplusf_(float a) { return a > 20.0f ? a : log1pf(__expf(a)); }

// ---------------------------------------------------------------------------------------------
// grid barrier: two-level counters (8 groups, then one top counter), monotone across steps.
// Run by lane 0 of the sync wave; the caller brackets it with workgroup barriers.
// ---------------------------------------------------------------------------------------------
__device__ bool grid_arrive_wait(const StepArgs &a, uint32_t k, int phase) {
  const uint32_t G = gridDim.x;
  const uint32_t groups = G < 8u ? G : 8u;
  const uint32_t g = blockIdx.x % groups;
  const uint32_t cnt = G / groups + (g < (G % groups) ? 1u : 0u);
  uint32_t old = __hip_atomic_fetch_add(a.bar + g * 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (old + 1u == k * cnt) __hip_atomic_fetch_add(a.bar + 8 * 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t tgt = k * groups;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  bool ok = true;
  while ((int32_t)(ld_cu(a.bar + 8 * 32) - tgt) < 0) {
    __builtin_amdgcn_s_sleep(2);
    if (ld_ci(a.status + 2) != 0) { ok = false; break; }
    if ((int64_t)(__builtin_amdgcn_s_memrealtime() - t0) > a.timeout_ticks) {
      st_ci(a.status + 1, phase);
      st_ci(a.status + 0, 6 /* MK_E_DEVICE_TIMEOUT */);
      st_ci(a.status + 2, 1);
      ok = false;
      break;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // drop stale L1/L2 lines before the next phase reads
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
__device__ __forceinline__ CPhase *cphase(const StepArgs &a, int q) { return (CPhase *)(a.phases + q); }
__device__ __forceinline__ Phase load_phase(const StepArgs &a, int q) {
  typedef const __attribute__((address_space(4))) int32_t cint;
  Phase p;
  cint *src = (cint *)(a.phases + q);
  int32_t *dst = reinterpret_cast<int32_t *>(&p);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(Phase) / 4); ++i) dst[i] = src[i];
  return p;
}

// Work split of a product phase: the S k-splits each get gridDim.x / S workgroups (S divides the
// workgroup count), and a split's T tiles are divided evenly over its workgroups, so every workgroup
// works inside one k-split: tiles [t0, t1) of split s.
__device__ __forceinline__ void unit_range(int T, int S, int &s, int &t0, int &t1) {
  const int per = (int)gridDim.x / S, wg = blockIdx.x;
  s = wg / per;
  const int wl = wg - s * per;
  t0 = (int)(((int64_t)T * wl) / per);
  t1 = (int)(((int64_t)T * (wl + 1)) / per);
}

struct Stream {
  const uint4 *ptr;  // next fragment of this wave (or a valid dummy address once the stream is done)
  int q, left, j, nfw, skip;  // skip: fragments from the end of one tile's run to the next tile's
};

__device__ __forceinline__ void stream_seek(Stream &st, const StepArgs &a, int wave, int q) {
  st.q = -1;
  st.left = 0;
  st.ptr = reinterpret_cast<const uint4 *>(a.wbuf);
  while (q >= 0 && q < a.phase_end) {
    CPhase *ph = cphase(a, q);
    if (ph->type == PH_GEMV) {
      int s, t0, t1;
      unit_range(ph->T, ph->S, s, t0, t1);
      if (t1 > t0) {
        const int nfw = ph->nf / kCWaves;
        st.q = q;
        st.nfw = nfw;
        st.left = (t1 - t0) * nfw;
        st.j = 0;
        st.skip = ph->KF - nfw;
        st.ptr = reinterpret_cast<const uint4 *>(a.wbuf + ph->w_off) +
                 ((int64_t)t0 * ph->KF + s * ph->nf + wave * nfw) * 64;
        return;
      }
    }
    q = ph->next_gemv;
  }
}

// Always issues a load (a dummy one once the stream is done), so a ring slot is only ever written by
// a load and its register never needs a copy that would wait for the load.
__device__ __forceinline__ uint4 stream_take(Stream &st, const StepArgs &a, int wave, int lane) {
  const uint4 v = ld_nt(st.ptr + lane);
  if (st.q >= 0) {
    st.ptr += 64;
    if (++st.j == st.nfw) {
      st.j = 0;
      st.ptr += (int64_t)st.skip * 64;
    }
    if (--st.left == 0) stream_seek(st, a, wave, cphase(a, st.q)->next_gemv);
  }
  return v;
}

// r[i] <- r[(i + head) % D]: puts the oldest in-flight fragment in slot 0 (waits for the ring to land)
template <int D>
__device__ __forceinline__ void ring_rotate(uint4 (&r)[D], int head) {
  uint4 t[D];
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
// GEMV phase: Y = W * act, W packed as [tile][fragment][lane][8] bf16
// ---------------------------------------------------------------------------------------------
constexpr int kRedSlots = 8;  // unit partials in flight between the compute waves and the sync wave
struct GemvLds {
  static constexpr int act = 0;                                                 // kActLdsBudget bytes
  static constexpr int red = kActLdsBudget;                                     // [kRedSlots][kCWaves][16][kMaxRows] f32
  static constexpr int flags = red + kRedSlots * kCWaves * 16 * kMaxRows * 4;   // posted[kRedSlots], consumed[kRedSlots]
  static constexpr int misc = flags + 2 * kRedSlots * 4;                        // rstd, finalizer flags, candidates
};

__device__ __forceinline__ uint32_t lds_ld(uint32_t *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP); }

// Bounded wait for an LDS counter written by another wave of this workgroup. On expiry the step is
// marked timed out (status word) and the wait gives up, so every wave still reaches the kernel's end.
__device__ __forceinline__ void lds_wait_ge(uint32_t *p, uint32_t v, const StepArgs &a) {
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

// Stages the activation fragments of k-split s in LDS: for each row b and column k the fp32 value y,
// split into a bf16 high part and a bf16 low part (y - high), laid out as the B operand of
// v_mfma_f32_16x16x32_bf16 (columns 0..R-1 high parts, R..2R-1 low parts). For an RMSNorm input, y is
// x * gain: the per-row factor 1/rms is applied to the product's outputs (the product is linear).
__device__ __forceinline__ void prep_act(const StepArgs &a, const Phase &ph, int s, char *smem) {
  const int R = a.R;
  const int nk = ph.nf * kFragK;
  const int k0 = s * nk;
  uint4 *act = reinterpret_cast<uint4 *>(smem + GemvLds::act);
  const int items = (nk / 8) * R;
  for (int it = threadIdx.x; it < items; it += kThreads) {
    const int b = it % R, kg = it / R, k = k0 + kg * 8;
    float y[8];
    if (ph.act == ACT_NORM) {
      const float4 *xp = reinterpret_cast<const float4 *>(a.x + (size_t)b * a.H + k);
      float4 x0 = xp[0], x1 = xp[1];
      const uint16_t *gp = reinterpret_cast<const uint16_t *>(a.wbuf + ph.gain_off) + k;
      uint4 gg = *reinterpret_cast<const uint4 *>(gp);
      float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      uint32_t gw[4] = {gg.x, gg.y, gg.z, gg.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float g = bf2f((uint16_t)(gw[e >> 1] >> ((e & 1) * 16)));
        y[e] = xs[e] * g;
      }
    } else if (ph.act == ACT_MIX) {
      const float4 *mp = reinterpret_cast<const float4 *>(a.mix + (size_t)b * a.mix_stride + k);
      float4 m0 = mp[0], m1 = mp[1];
      y[0] = m0.x; y[1] = m0.y; y[2] = m0.z; y[3] = m0.w; y[4] = m1.x; y[5] = m1.y; y[6] = m1.z; y[7] = m1.w;
    } else {
      const float *src = a.part[ph.src_part];
      float g[8] = {0, 0, 0, 0, 0, 0, 0, 0}, u[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int s2 = 0; s2 < ph.src_S; ++s2) {
        const float *row = src + ((size_t)s2 * R + b) * ph.src_N + ph.src_off + k;
        float4 p0 = reinterpret_cast<const float4 *>(row)[0], p1 = reinterpret_cast<const float4 *>(row)[1];
        g[0] += p0.x; g[1] += p0.y; g[2] += p0.z; g[3] += p0.w; g[4] += p1.x; g[5] += p1.y; g[6] += p1.z; g[7] += p1.w;
        if (ph.act == ACT_SWIGLU) {
          const float *up = row + ph.K;  // up rows follow the gate rows
          float4 q0 = reinterpret_cast<const float4 *>(up)[0], q1 = reinterpret_cast<const float4 *>(up)[1];
          u[0] += q0.x; u[1] += q0.y; u[2] += q0.z; u[3] += q0.w; u[4] += q1.x; u[5] += q1.y; u[6] += q1.z; u[7] += q1.w;
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = (ph.act == ACT_SWIGLU) ? silu(g[e]) * u[e] : g[e];
    }
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      uint16_t h0 = f2bf(y[e]), h1 = f2bf(y[e + 1]);
      uint16_t l0 = f2bf(y[e] - bf2f(h0)), l1 = f2bf(y[e + 1] - bf2f(h1));
      hi[e >> 1] = (uint32_t)h0 | ((uint32_t)h1 << 16);
      lo[e >> 1] = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
    const int f = kg >> 2, g4 = kg & 3;
    act[(f * 4 + g4) * (2 * R) + b] = uint4{hi[0], hi[1], hi[2], hi[3]};
    act[(f * 4 + g4) * (2 * R) + R + b] = uint4{lo[0], lo[1], lo[2], lo[3]};
  }
}

// compute waves: consume this phase's fragments from the ring, refilling each slot from the stream.
// A finished 16-row unit is handed to the sync wave through an LDS slot and a counter, without a
// workgroup barrier, so the four waves never wait for each other inside a phase.
template <int D>
__device__ __forceinline__ void gemv_compute(const StepArgs &a, const Phase &ph, char *smem, uint4 (&ring)[D], Stream &st, int &head) {
  const int R = a.R;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int nfw = ph.nf / kCWaves;
  int s, t0, t1;
  unit_range(ph.T, ph.S, s, t0, t1);
  const int total = (t1 - t0) * nfw;
  float *red = reinterpret_cast<float *>(smem + GemvLds::red);
  uint32_t *posted = reinterpret_cast<uint32_t *>(smem + GemvLds::flags);
  uint32_t *consumed = posted + kRedSlots;
  const uint4 *actv = reinterpret_cast<const uint4 *>(smem + GemvLds::act);
  if (head != 0) {
    ring_rotate(ring, head);
    head = 0;
  }
  if (total > 0) prep_act(a, ph, s, smem);
  lds_barrier();  // activation fragments ready, handoff counters cleared
  int c_j = 0, unit = 0;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int col = lane & 15, kgrp = lane >> 4;
  const uint4 *aw = actv + (size_t)wave * nfw * 4 * (2 * R);
  // one fragment: MFMA with the activation fragment, refill the slot from the stream, close the unit
  auto slot = [&](uint4 &r) {
    uint4 bv = uint4{0u, 0u, 0u, 0u};
    if (col < 2 * R) bv = aw[(c_j * 4 + kgrp) * (2 * R) + col];
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r), __builtin_bit_cast(bf16x8, bv), acc, 0,
                                                  0, 0);
    r = stream_take(st, a, wave, lane);  // the slot's old fragment is consumed: refill it
    if (++c_j == nfw) {  // unit done: combine hi/lo columns and post this wave's 16 x R partials
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = acc[e] + __shfl_down(acc[e], R);
      const int sl = unit % kRedSlots;
      const uint32_t use = (uint32_t)(unit / kRedSlots);
      if (lds_ld(consumed + sl) < use) lds_wait_ge(consumed + sl, use, a);  // slot free (the sync wave read it)
      float *rb = red + (sl * kCWaves + wave) * 16 * kMaxRows;
      if (col < R) {
#pragma unroll
        for (int e = 0; e < 4; ++e) rb[(kgrp * 4 + e) * kMaxRows + col] = v[e];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      if (lane == 0) __hip_atomic_fetch_add(posted + sl, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      ++unit;
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
      c_j = 0;
    }
  };
  // full turns of the ring: every slot consumed and refilled once per turn, so each fragment is waited
  // for with D - 1 younger loads still in flight
  const int turns = total / D;
  for (int it = 0; it < turns; ++it) {
#pragma unroll
    for (int d = 0; d < D; ++d) slot(ring[d]);
  }
  const int rem = total - turns * D;
#pragma unroll
  for (int d = 0; d < D - 1; ++d)
    if (d < rem) slot(ring[d]);
  head = rem;
}

// sync wave: activation staging (with the compute waves), norm statistics, per-unit reduction and
// stores, finalisation
__device__ __forceinline__ void gemv_sync(const StepArgs &a, const Phase &ph, char *smem) {
  const int R = a.R, lane = threadIdx.x & 63;
  int s, t0, t1;
  unit_range(ph.T, ph.S, s, t0, t1);
  const int nunits = t1 - t0;
  float *red = reinterpret_cast<float *>(smem + GemvLds::red);
  uint32_t *posted = reinterpret_cast<uint32_t *>(smem + GemvLds::flags);
  uint32_t *consumed = posted + kRedSlots;
  float *misc = reinterpret_cast<float *>(smem + GemvLds::misc);
  float *rstd = misc;                                        // [kMaxRows]
  int *flags = reinterpret_cast<int *>(misc + 16);           // [kMaxUnits]
  float *cval = misc + 16 + kMaxUnits;                       // [128]
  int *cidx = reinterpret_cast<int *>(cval + 128);           // [128]
  float *sq = cval + 256;                                    // [16][kMaxRows]
  const bool direct = ph.out == OUT_LOGITS && ph.S == 1;
  if (lane < 2 * kRedSlots) posted[lane] = 0u;  // posted[] and consumed[] (adjacent)
  if (nunits > 0) prep_act(a, ph, s, smem);
  lds_barrier();  // activation fragments ready, handoff counters cleared
  if (ph.act == ACT_NORM) {  // 1/rms of each row from the per-tile sums of squares (while the waves stream)
    const int nt = a.H / kTileRows;
    for (int b = 0; b < R; ++b) {
      float v = 0.0f;
      for (int t = lane; t < nt; t += 64) v += a.ss[(size_t)b * nt + t];
      v = wave_sum(v);
      if (lane == 0) rstd[b] = 1.0f / sqrtf(v / (float)a.H + a.eps);
    }
    wave_lds_sync();
  }
  float rs[2] = {1.0f, 1.0f};
#pragma unroll
  for (int k = 0; k < 2; ++k)
    if (ph.act == ACT_NORM && lane + 64 * k < 16 * R) rs[k] = rstd[(lane + 64 * k) % R];
  float best_v[2] = {-INFINITY, -INFINITY};
  int best_i[2] = {0x7fffffff, 0x7fffffff};
  for (int t = t0, unit = 0; t < t1; ++t, ++unit) {
    const int sl = unit % kRedSlots;
    const uint32_t need = (uint32_t)(kCWaves * (unit / kRedSlots + 1));
    if (lds_ld(posted + sl) < need) lds_wait_ge(posted + sl, need, a);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    const float *rb = red + sl * kCWaves * 16 * kMaxRows;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int idx = lane + 64 * k;
      if (idx < 16 * R) {
        const int row = idx / R, b = idx % R;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < kCWaves; ++w) v += rb[(w * 16 + row) * kMaxRows + b];
        v *= rs[k];
        const int n = t * kTileRows + row;
        if (direct) {
          a.logits[(size_t)b * a.V + n] = v;
          if (v > best_v[k]) { best_v[k] = v; best_i[k] = n; }
        } else {
          st_c(a.part[ph.dst_part] + ((size_t)s * R + b) * ph.N + n, v);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane == 0) __hip_atomic_store(consumed + sl, (uint32_t)(unit / kRedSlots + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  if (ph.out == OUT_RESID || (ph.out == OUT_LOGITS && !direct)) {
    // the last contributor of a tile adds the tile's k-split partials (in split order) into the
    // residual (and records its sum of squares), or into the logits
    __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are acknowledged
    for (int i = lane; i < nunits; i += 64) {
      const int t = t0 + i;
      uint32_t old = __hip_atomic_fetch_add(a.fin + ph.cnt_off + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      flags[i] = (old + 1u == a.epoch * (uint32_t)ph.S) ? t : -1;
    }
    wave_lds_sync();
    for (int i = 0; i < nunits; ++i) {
      const int t = flags[i];
      if (t < 0) continue;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int idx = lane + 64 * k;
        if (idx < 16 * R) {
          const int row = idx / R, b = idx % R, n = t * kTileRows + row;
          float v = 0.0f;
          for (int s2 = 0; s2 < ph.S; ++s2) v += ld_c(a.part[ph.dst_part] + ((size_t)s2 * R + b) * ph.N + n);
          if (ph.out == OUT_RESID) {
            const float xn = ld_c(a.x + (size_t)b * a.H + n) + v;
            st_c(a.x + (size_t)b * a.H + n, xn);
            sq[row * kMaxRows + b] = xn * xn;
          } else {
            a.logits[(size_t)b * a.V + n] = v;
            if (v > best_v[k] || (v == best_v[k] && n < best_i[k])) { best_v[k] = v; best_i[k] = n; }
          }
        }
      }
      if (ph.out == OUT_RESID) {
        wave_lds_sync();
        if (lane < R) {
          float v = 0.0f;
          for (int row = 0; row < 16; ++row) v += sq[row * kMaxRows + lane];
          st_c(a.ss + (size_t)lane * (a.H / kTileRows) + t, v);
        }
        wave_lds_sync();
      }
    }
  }
  if (ph.out == OUT_LOGITS) {  // per-workgroup argmax candidate of each row (first index on ties)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
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
// gated delta rule: per (sequence, head, 16 state rows); one wave per state row, 2 channels per lane
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void delta_phase(const StepArgs &a, const Phase &ph) {
  constexpr int kRowsPerUnit = 16;
  const int R = a.R, Hl = a.lin_heads, dk = a.dk, dv = a.dv;
  const int RB = dv / kRowsPerUnit;
  const int nseq = a.verify ? 1 : R;
  const int U = nseq * Hl * RB;
  const int G = gridDim.x, wg = blockIdx.x;
  const int u0 = (int)(((int64_t)U * wg) / G), u1 = (int)(((int64_t)U * (wg + 1)) / G);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const float *src = a.part[ph.src_part];
  const int c0 = lane * 2;
  for (int u = u0; u < u1; ++u) {
    const int b = u / (Hl * RB), h = (u / RB) % Hl, rb = u % RB;
    for (int r = rb * kRowsPerUnit + wave; r < (rb + 1) * kRowsPerUnit; r += kWavesTotal) {
      float *Srow = reinterpret_cast<float *>(a.ls[ph.layer]) + (((size_t)b * Hl + h) * dv + r) * dk;
      float2 S = *reinterpret_cast<const float2 *>(Srow + c0);
      const int j0 = a.verify ? 0 : b, j1 = a.verify ? a.R : b + 1;
      for (int j = j0; j < j1; ++j) {
        float q0 = 0, q1 = 0, k0 = 0, k1 = 0, vr = 0, av0 = 0, av1 = 0, bv = 0;
        for (int s2 = 0; s2 < ph.src_S; ++s2) {
          const float *row = src + ((size_t)s2 * R + j) * ph.src_N;
          const float2 qq = *reinterpret_cast<const float2 *>(row + ph.q_off + h * dk + c0);
          const float2 kk = *reinterpret_cast<const float2 *>(row + ph.k_off + h * dk + c0);
          q0 += qq.x; q1 += qq.y; k0 += kk.x; k1 += kk.y;
          vr += row[ph.v_off + h * dv + r];
          if (ph.per_channel_gate) {
            const float2 aa = *reinterpret_cast<const float2 *>(row + ph.a_off + h * dk + c0);
            av0 += aa.x; av1 += aa.y;
          } else {
            av0 += row[ph.a_off + h];
          }
          bv += row[ph.b_off + h];
        }
        if (!ph.per_channel_gate) av1 = av0;
        const float qn = 1.0f / sqrtf(wave_sum(q0 * q0 + q1 * q1) + 1e-6f);
        const float kn = 1.0f / sqrtf(wave_sum(k0 * k0 + k1 * k1) + 1e-6f);
        q0 *= qn; q1 *= qn; k0 *= kn; k1 *= kn;
        const float al0 = __expf(-softplusf_(av0)), al1 = ph.per_channel_gate ? __expf(-softplusf_(av1)) : al0;
        const float beta = sigmoidf_(bv);
        S.x *= al0; S.y *= al1;
        const float uu = wave_sum(S.x * k0 + S.y * k1);
        const float delta = beta * (vr - uu);
        S.x += delta * k0; S.y += delta * k1;
        const float o = wave_sum(S.x * q0 + S.y * q1);
        if (lane == 0) st_c(a.mix + (size_t)j * a.mix_stride + h * dv + r, o);
        if (a.verify) {
          float *sn = a.snap + ((((size_t)ph.lin_idx * kMaxRows + j) * Hl + h) * dv + r) * dk + c0;
          st_c(sn, S.x);
          st_c(sn + 1, S.y);
        }
      }
      if (!a.verify) *reinterpret_cast<float2 *>(Srow + c0) = S;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// split-KV grouped-query attention: per (sequence, kv head, chunk of positions)
// ---------------------------------------------------------------------------------------------
template <int HD>
__device__ __forceinline__ void attn_phase(const StepArgs &a, const Phase &ph, char *smem) {
  const int R = a.R, nq = a.nq, nkv = a.nkv, grp = nq / nkv;
  const int CS = ph.chunk, NC = ph.n_chunks;
  const int nseq = a.verify ? 1 : R;
  const int nrow = a.verify ? R : 1;  // query rows per unit
  const int Q = grp * nrow;
  const int U = nseq * nkv * NC;
  const int G = gridDim.x, wg = blockIdx.x, tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int u0 = (int)(((int64_t)U * wg) / G), u1 = (int)(((int64_t)U * (wg + 1)) / G);
  const float scale = 1.0f / sqrtf((float)HD);
  constexpr int half = HD / 2;
  float *qs = reinterpret_cast<float *>(smem);                        // [Q][HD]       <= 32 KiB
  uint16_t *Ks = reinterpret_cast<uint16_t *>(qs + kAttnMaxQ * 128);  // [CS][HD] bf16 <= 32 KiB
  uint16_t *Vs = Ks + kAttnMaxChunk * 128;                            // [CS][HD] bf16 <= 32 KiB
  float *sc = reinterpret_cast<float *>(Vs + kAttnMaxChunk * 128);    // [Q][CS]       <= 32 KiB
  float *ml = sc + kAttnMaxQ * kAttnMaxChunk;                         // [Q][2]
  int *rpos = reinterpret_cast<int *>(ml + kAttnMaxQ * 2);            // [nrow]
  const float *src = a.part[ph.src_part];
  uint16_t *kc = reinterpret_cast<uint16_t *>(a.kc[ph.layer]);
  uint16_t *vc = reinterpret_cast<uint16_t *>(a.vc[ph.layer]);

  for (int u = u0; u < u1; ++u) {
    const int b = u / (nkv * NC), g = (u / NC) % nkv, c = u % NC;
    const int seq = a.verify ? 0 : b;
    const int pbase = a.pos[seq];
    const int maxpos = pbase + nrow - 1;
    const int c0 = c * CS;
    const int c1 = min(c0 + CS, min(a.max_ctx, maxpos + 1));  // positions [c0, c1) are read
    const int npos = max(c1 - c0, 0);
    lds_barrier();
    if (tid < nrow) rpos[tid] = pbase + tid;
    // queries (sum of k-split partials)
    for (int idx = tid; idx < Q * HD; idx += kThreads) {
      const int qi = idx / HD, i = idx % HD, rr = qi / grp, hh = qi % grp;
      const int row = a.verify ? rr : b;
      const int h = g * grp + hh;
      float s = 0.0f;
      for (int s2 = 0; s2 < ph.src_S; ++s2) s += src[((size_t)s2 * R + row) * ph.src_N + ph.q_off + h * HD + i];
      qs[qi * HD + i] = s;
    }
    // cached K/V rows of the chunk
    for (int idx = tid; idx < npos * (HD / 8); idx += kThreads) {
      const int jj = idx / (HD / 8), i8 = (idx % (HD / 8)) * 8, j = c0 + jj;
      if (j < pbase) {
        const size_t off = (((size_t)seq * nkv + g) * a.max_ctx + j) * HD + i8;
        *reinterpret_cast<uint4 *>(Ks + jj * HD + i8) = *reinterpret_cast<const uint4 *>(kc + off);
        *reinterpret_cast<uint4 *>(Vs + jj * HD + i8) = *reinterpret_cast<const uint4 *>(vc + off);
      }
    }
    // this step's new rows: rotated K and V rounded to bf16, appended to the cache
    for (int idx = tid; idx < npos * half; idx += kThreads) {
      const int jj = idx / half, i = idx % half, j = c0 + jj;
      if (j >= pbase) {
        const int row = a.verify ? (j - pbase) : b;
        float k0 = 0, k1 = 0, v0 = 0, v1 = 0;
        for (int s2 = 0; s2 < ph.src_S; ++s2) {
          const float *pr = src + ((size_t)s2 * R + row) * ph.src_N;
          k0 += pr[ph.k_off + g * HD + i];
          k1 += pr[ph.k_off + g * HD + i + half];
          v0 += pr[ph.v_off + g * HD + i];
          v1 += pr[ph.v_off + g * HD + i + half];
        }
        const float2 cs = reinterpret_cast<const float2 *>(a.rope)[(size_t)j * half + i];
        const uint16_t kr0 = f2bf(k0 * cs.x - k1 * cs.y), kr1 = f2bf(k0 * cs.y + k1 * cs.x);
        const uint16_t vb0 = f2bf(v0), vb1 = f2bf(v1);
        Ks[jj * HD + i] = kr0;
        Ks[jj * HD + i + half] = kr1;
        Vs[jj * HD + i] = vb0;
        Vs[jj * HD + i + half] = vb1;
        const size_t off = (((size_t)seq * nkv + g) * a.max_ctx + j) * HD;
        kc[off + i] = kr0;
        kc[off + i + half] = kr1;
        vc[off + i] = vb0;
        vc[off + i + half] = vb1;
      }
    }
    lds_barrier();
    for (int idx = tid; idx < Q * half; idx += kThreads) {  // rotate the queries
      const int qi = idx / half, i = idx % half, rr = qi / grp;
      const float2 cs = reinterpret_cast<const float2 *>(a.rope)[(size_t)rpos[rr] * half + i];
      const float x0 = qs[qi * HD + i], x1 = qs[qi * HD + i + half];
      qs[qi * HD + i] = x0 * cs.x - x1 * cs.y;
      qs[qi * HD + i + half] = x0 * cs.y + x1 * cs.x;
    }
    lds_barrier();
    // scores: one thread per (query, position), the HD-long dot product fully unrolled
    for (int idx = tid; idx < Q * CS; idx += kThreads) {
      const int qi = idx / CS, jj = idx % CS, j = c0 + jj;
      float s = -INFINITY;
      if (jj < npos && j <= rpos[qi / grp]) {
        const float4 *qv = reinterpret_cast<const float4 *>(qs + qi * HD);
        const uint4 *kv = reinterpret_cast<const uint4 *>(Ks + jj * HD);
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < HD / 8; ++i) {
          const uint4 kk = kv[i];
          const float4 qa = qv[2 * i], qb = qv[2 * i + 1];
          acc += qa.x * bf2f((uint16_t)kk.x) + qa.y * bf2f((uint16_t)(kk.x >> 16)) + qa.z * bf2f((uint16_t)kk.y) +
                 qa.w * bf2f((uint16_t)(kk.y >> 16)) + qb.x * bf2f((uint16_t)kk.z) + qb.y * bf2f((uint16_t)(kk.z >> 16)) +
                 qb.z * bf2f((uint16_t)kk.w) + qb.w * bf2f((uint16_t)(kk.w >> 16));
        }
        s = acc * scale;
      }
      sc[qi * CS + jj] = s;
    }
    lds_barrier();
    // softmax statistics: one wave per query, lanes over positions
    for (int qi = wave; qi < Q; qi += kWavesTotal) {
      float m = -INFINITY;
      for (int jj = lane; jj < CS; jj += 64) m = fmaxf(m, sc[qi * CS + jj]);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      float l = 0.0f;
      for (int jj = lane; jj < CS; jj += 64) {
        const float p = (m == -INFINITY) ? 0.0f : __expf(sc[qi * CS + jj] - m);
        sc[qi * CS + jj] = p;
        l += p;
      }
      l = wave_sum(l);
      if (lane == 0) { ml[qi * 2] = m; ml[qi * 2 + 1] = l; }
    }
    lds_barrier();
    // weighted values: one thread per (query, output dim)
    for (int idx = tid; idx < Q * HD; idx += kThreads) {
      const int qi = idx / HD, i = idx % HD, rr = qi / grp, hh = qi % grp;
      float acc = 0.0f;
      const float *pr = sc + qi * CS;
#pragma unroll 8
      for (int jj = 0; jj < npos; ++jj) acc += pr[jj] * bf2f(Vs[jj * HD + i]);
      const int row = a.verify ? rr : b, h = g * grp + hh;
      float *dst = a.attn + (((size_t)row * nq + h) * NC + c) * (HD + 2);
      st_c(dst + 2 + i, acc);
      if (i == 0) { st_c(dst, ml[qi * 2]); st_c(dst + 1, ml[qi * 2 + 1]); }
    }
  }
}

__device__ __forceinline__ void merge_phase(const StepArgs &a, const Phase &ph, char *smem) {
  const int R = a.R, nq = a.nq, hd = a.hd, NC = ph.n_chunks, W = hd + 2;
  const int U = R * nq;
  const int G = gridDim.x, wg = blockIdx.x, tid = threadIdx.x;
  const int u0 = (int)(((int64_t)U * wg) / G), u1 = (int)(((int64_t)U * (wg + 1)) / G);
  float *pl = reinterpret_cast<float *>(smem);  // [NC][hd + 2]
  float *wt = pl + NC * W;                       // [NC] weights, then [1] total
  for (int u = u0; u < u1; ++u) {
    const int row = u / nq, h = u % nq;
    const float *p = a.attn + ((size_t)row * nq + h) * NC * W;
    lds_barrier();
    for (int i = tid; i < NC * W; i += kThreads) pl[i] = p[i];
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
    }
  }
}

__device__ __forceinline__ void embed_phase(const StepArgs &a, const Phase &ph, char *smem) {
  const int R = a.R, H = a.H, nt = H / kTileRows;
  const int U = R * nt;
  const int G = gridDim.x, wg = blockIdx.x, tid = threadIdx.x;
  const int u0 = (int)(((int64_t)U * wg) / G), u1 = (int)(((int64_t)U * (wg + 1)) / G);
  float *sq = reinterpret_cast<float *>(smem);
  const uint16_t *E = reinterpret_cast<const uint16_t *>(a.wbuf + ph.w_off);
  for (int u = u0; u < u1; ++u) {
    const int row = u / nt, t = u % nt;
    lds_barrier();
    if (tid < kTileRows) {
      const int n = t * kTileRows + tid;
      float v;
      if (a.V > 0) {
        int tok = a.tokens[row];
        if (tok < 0 || tok >= a.V) {  // out-of-range token: report, read row 0 instead of faulting
          if (tid == 0) { st_ci(a.status + 1, -2); st_ci(a.status + 0, 1 /* MK_E_ARG */); }
          tok = 0;
        }
        v = bf2f(E[(size_t)tok * H + n]);
      }
      else v = a.hidden_in[(size_t)row * H + n];
      st_c(a.x + (size_t)row * H + n, v);
      sq[tid] = v * v;
    }
    lds_barrier();
    if (tid == 0) {
      float s = 0.0f;
      for (int i = 0; i < kTileRows; ++i) s += sq[i];
      st_c(a.ss + (size_t)row * nt + t, s);
    }
  }
}

__device__ __forceinline__ void final_phase(const StepArgs &a, char *smem) {
  const int R = a.R, G = gridDim.x, tid = threadIdx.x;
  float *cv = reinterpret_cast<float *>(smem);
  int *ci = reinterpret_cast<int *>(cv + G * kMaxRows);
  int *am = ci + G * kMaxRows;
  int *acc_s = am + kMaxRows;
  if (a.V > 0) {
    for (int idx = tid; idx < G * R; idx += kThreads) {
      cv[idx] = a.cand[(size_t)idx * 2];
      ci[idx] = reinterpret_cast<const int32_t *>(a.cand)[(size_t)idx * 2 + 1];
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

__device__ __forceinline__ void hidden_out_phase(const StepArgs &a) {
  const size_t n = (size_t)a.R * a.H;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (size_t)gridDim.x * kThreads)
    a.hidden_out[i] = ld_c(a.x + i);
}

}  // namespace mk

using namespace mk;

// The step kernel: walks phases [phase_begin, phase_end) of the schedule. As a persistent launch it
// covers the whole step with a grid barrier between phases (all workgroups co-resident: cooperative
// launch, one workgroup per compute unit); the per-op baseline launches it once per phase.
// Waves 0..kCWaves-1 stream weights (their ring is never drained at a phase end: the loads of the next
// product phase are in flight through barriers and the phases in between); wave kSyncWave reduces,
// stores cross-workgroup results and runs the grid barrier.
extern "C" __global__ void __launch_bounds__(kThreads) mk_step_kernel(StepArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int abort_flag;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const bool is_sync = wave == kSyncWave;
  uint32_t k = (a.epoch - 1u) * (uint32_t)a.n_barriers + (uint32_t)a.barrier_base;
  uint4 ring[kRing];
  Stream st;
  int head = 0;
  st.q = -1;
  st.left = 0;
  if (!is_sync) {
    int q = a.phase_begin;
    while (q < a.phase_end && cphase(a, q)->type != PH_GEMV) ++q;
    stream_seek(st, a, wave, q < a.phase_end ? q : -1);
#pragma unroll
    for (int d = 0; d < kRing; ++d) ring[d] = stream_take(st, a, wave, lane);
  }
  for (int p = a.phase_begin; p < a.phase_end; ++p) {
    const Phase ph = load_phase(a, p);
    if (a.trace && is_sync && lane == 0) a.trace[((size_t)p * gridDim.x + blockIdx.x) * 2] = __builtin_amdgcn_s_memrealtime();
    const bool gemv = ph.type == PH_GEMV;
    switch (ph.type) {
      case PH_EMBED: embed_phase(a, ph, smem); break;
      case PH_GEMV:
        if (is_sync) gemv_sync(a, ph, smem);
        else gemv_compute<kRing>(a, ph, smem, ring, st, head);
        break;
      case PH_DELTA: delta_phase(a, ph); break;
      case PH_ATTN:
        if (a.hd == 64) attn_phase<64>(a, ph, smem);
        else attn_phase<128>(a, ph, smem);
        break;
      case PH_MERGE: merge_phase(a, ph, smem); break;
      case PH_FINAL: final_phase(a, smem); break;
      case PH_HIDDEN_OUT: hidden_out_phase(a); break;
      default: break;
    }
    // phase end: results stored by a wave are acknowledged before the grid barrier. In product phases
    // only the sync wave stores; the compute waves keep their weight loads in flight.
    if (!gemv) {
      __builtin_amdgcn_s_waitcnt(0);
      lds_barrier();
    }
    if (is_sync) {
      __builtin_amdgcn_s_waitcnt(0);
      if (lane == 0) {
        if (a.trace) a.trace[((size_t)p * gridDim.x + blockIdx.x) * 2 + 1] = __builtin_amdgcn_s_memrealtime();
        int ok = 1;
        if (p + 1 < a.phase_end) ok = grid_arrive_wait(a, k + 1, p);
        abort_flag = !ok;
      }
    }
    ++k;
    lds_barrier();
    if (abort_flag) return;
  }
}

// Weight repacking: natural bf16 [rows][cols] -> tile-major MFMA fragments. Fragment (t, f) holds, for
// lane l, the 8 columns f*32 + 8*(l/16) .. +7 of row t*16 + l%16; rows land at row_off + r of the
// destination matrix (row_off a multiple of 16; padding rows stay as the caller zeroed them).
extern "C" __global__ void mk_repack_bf16(const uint16_t *__restrict__ src, int64_t rows, int64_t cols,
                                          uint4 *__restrict__ dst, int64_t row_off, int64_t KF) {
  const int64_t nfr_rows = (rows + 15) / 16;
  const int64_t total = nfr_rows * KF * 64;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * blockDim.x) {
    const int lane = (int)(idx & 63);
    const int64_t fr = idx >> 6;
    const int64_t t = fr / KF, f = fr % KF;
    const int64_t r = t * 16 + (lane & 15);
    if (r >= rows) continue;
    const int64_t c = f * 32 + 8 * (lane >> 4);
    const uint4 v = *reinterpret_cast<const uint4 *>(src + r * cols + c);
    const int64_t dr = row_off + r;
    dst[((dr / 16) * KF + f) * 64 + (dr % 16) + 16 * (lane >> 4)] = v;
  }
}
