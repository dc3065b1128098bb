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
// grid barrier: two-level counters (8 groups, then one top counter), monotone across steps
// ---------------------------------------------------------------------------------------------
__device__ bool grid_barrier(const StepArgs &a, uint32_t k, int phase, int *abort_flag) {
  __builtin_amdgcn_s_waitcnt(0);  // this wave's stores are acknowledged (sc1 stores are write-through)
  lds_barrier();
  if (threadIdx.x == 0) {
    int ok = 1;
    const uint32_t G = gridDim.x;
    const uint32_t groups = G < 8u ? G : 8u;
    const uint32_t g = blockIdx.x % groups;
    const uint32_t cnt = G / groups + (g < (G % groups) ? 1u : 0u);
    uint32_t old = __hip_atomic_fetch_add(a.bar + g * 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1u == k * cnt) __hip_atomic_fetch_add(a.bar + 8 * 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t tgt = k * groups;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while ((int32_t)(ld_cu(a.bar + 8 * 32) - tgt) < 0) {
      __builtin_amdgcn_s_sleep(2);
      if (ld_ci(a.status + 2) != 0) { ok = 0; break; }
      if ((int64_t)(__builtin_amdgcn_s_memrealtime() - t0) > a.timeout_ticks) {
        st_ci(a.status + 1, phase);
        st_ci(a.status + 0, 6 /* MK_E_DEVICE_TIMEOUT */);
        st_ci(a.status + 2, 1);
        ok = 0;
        break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // drop stale L1/L2 lines before reading
    *abort_flag = !ok;
  }
  lds_barrier();
  return *abort_flag == 0;
}

// ---------------------------------------------------------------------------------------------
// GEMV phase: Y = W * act, W packed as [tile][fragment][lane][8] bf16
// ---------------------------------------------------------------------------------------------
// LDS carve-up for GEMV
struct GemvLds {
  static constexpr int act = 0;                                    // kActLdsBudget bytes
  static constexpr int red = kActLdsBudget;                        // [2][kWaves][16][kMaxRows] f32
  static constexpr int misc = red + 2 * kWaves * 16 * kMaxRows * 4;  // rstd, flags, candidates
};

__device__ void prep_act(const StepArgs &a, const Phase &ph, int s, char *smem, const float *rstd) {
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
      const float r = rstd[b];
      float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      uint32_t gw[4] = {gg.x, gg.y, gg.z, gg.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float g = bf2f((uint16_t)(gw[e >> 1] >> ((e & 1) * 16)));
        y[e] = (xs[e] * r) * g;
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

template <int D>
__device__ void gemv_phase(const StepArgs &a, const Phase &ph, char *smem) {
  const int R = a.R;
  const int G = gridDim.x, wg = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int T = ph.T, nf = ph.nf, KF = ph.KF;
  const int U = T * ph.S;
  const int u0 = (int)(((int64_t)U * wg) / G), u1 = (int)(((int64_t)U * (wg + 1)) / G);
  float *red = reinterpret_cast<float *>(smem + GemvLds::red);
  float *misc = reinterpret_cast<float *>(smem + GemvLds::misc);
  float *rstd = misc;                                      // [kMaxRows]
  int *flags = reinterpret_cast<int *>(misc + 16);          // [kMaxUnits] finalizer tile flags
  float *cval = misc + 16 + kMaxUnits;                      // [16][kMaxRows] candidate values
  int *cidx = reinterpret_cast<int *>(misc + 16 + kMaxUnits + 16 * kMaxRows);
  const uint4 *actv = reinterpret_cast<const uint4 *>(smem + GemvLds::act);

  float best_v = -INFINITY;
  int best_i = 0x7fffffff;

  if (ph.act == ACT_NORM && tid < R) {  // rstd from per-tile sums of squares, tiles in order
    const int nt = a.H / kTileRows;
    float s = 0.0f;
    for (int t = 0; t < nt; ++t) s += a.ss[(size_t)tid * nt + t];
    rstd[tid] = 1.0f / sqrtf(s / (float)a.H + a.eps);
  }

  const int nunits = u1 - u0;
  const int nfw = nf / kWaves;
  const bool direct = ph.out == OUT_LOGITS && ph.S == 1;  // one k-split: unit results are final logits
  const int total = nunits > 0 ? nunits * nfw : 0;
  const uint4 *W = reinterpret_cast<const uint4 *>(a.wbuf + ph.w_off);

  // prefetch cursor over this wave's fragment sequence
  int p_j = 0, p_t = u0 % T, p_s = u0 / T;
  uint4 ring[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    if (d < total) {
      ring[d] = ld_nt(W + ((int64_t)p_t * KF + p_s * nf + wave * nfw + p_j) * 64 + lane);
      if (++p_j == nfw) { p_j = 0; if (++p_t == T) { p_t = 0; ++p_s; } }
    }
  }
  int c_j = 0, c_t = u0 % T, c_s = u0 / T, act_s = -1, buf = 0;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int col = lane & 15, kgrp = lane >> 4;

  for (int i0 = 0; i0 < total; i0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int i = i0 + d;
      if (i < total) {
        if (c_j == 0 && c_s != act_s) {  // new k-split: rebuild the activation fragments
          lds_barrier();
          prep_act(a, ph, c_s, smem, rstd);
          lds_barrier();
          act_s = c_s;
        }
        const uint4 wv = ring[d];
        if (i + D < total) {
          ring[d] = ld_nt(W + ((int64_t)p_t * KF + p_s * nf + wave * nfw + p_j) * 64 + lane);
          if (++p_j == nfw) { p_j = 0; if (++p_t == T) { p_t = 0; ++p_s; } }
        }
        uint4 bv = uint4{0u, 0u, 0u, 0u};
        if (col < 2 * R) bv = actv[((wave * nfw + c_j) * 4 + kgrp) * (2 * R) + col];
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wv), __builtin_bit_cast(bf16x8, bv),
                                                      acc, 0, 0, 0);
        if (++c_j == nfw) {  // unit done: combine hi/lo columns, reduce the 8 waves, emit 16 x R values
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[e] + __shfl_down(acc[e], R);
          float *rb = red + buf * (kWaves * 16 * kMaxRows);
          if (col < R) {
#pragma unroll
            for (int e = 0; e < 4; ++e) rb[(wave * 16 + kgrp * 4 + e) * kMaxRows + col] = v[e];
          }
          lds_barrier();
          if (tid < 16 * R) {
            const int row = tid / R, b = tid % R;
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) s += rb[(w * 16 + row) * kMaxRows + b];
            const int n = c_t * kTileRows + row;
            if (direct) {
              a.logits[(size_t)b * a.V + n] = s;
              if (s > best_v) { best_v = s; best_i = n; }
            } else {
              st_c(a.part[ph.dst_part] + ((size_t)c_s * R + b) * ph.N + n, s);
            }
          }
          buf ^= 1;
          acc = f32x4{0.f, 0.f, 0.f, 0.f};
          c_j = 0;
          if (++c_t == T) { c_t = 0; ++c_s; }
        }
      }
    }
  }

  if (ph.out == OUT_RESID || (ph.out == OUT_LOGITS && !direct)) {
    // every partial of this workgroup is stored; the last contributor of a tile adds the tile's
    // partials (k-split order): into the residual (and its sum of squares), or into the logits
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    if (tid < nunits) {
      const int u = u0 + tid, t = u % T;
      uint32_t old = __hip_atomic_fetch_add(a.fin + ph.cnt_off + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      flags[tid] = (old + 1u == a.epoch * (uint32_t)ph.S) ? t : -1;
    }
    lds_barrier();
    float *sq = red;  // reuse
    for (int i = 0; i < nunits; ++i) {
      const int t = flags[i];
      if (t < 0) continue;
      if (tid < 16 * R) {
        const int row = tid / R, b = tid % R, n = t * kTileRows + row;
        float s = 0.0f;
        for (int s2 = 0; s2 < ph.S; ++s2) s += ld_c(a.part[ph.dst_part] + ((size_t)s2 * R + b) * ph.N + n);
        if (ph.out == OUT_RESID) {
          const float xn = ld_c(a.x + (size_t)b * a.H + n) + s;
          st_c(a.x + (size_t)b * a.H + n, xn);
          sq[row * kMaxRows + b] = xn * xn;
        } else {
          a.logits[(size_t)b * a.V + n] = s;
          if (s > best_v || (s == best_v && n < best_i)) { best_v = s; best_i = n; }
        }
      }
      if (ph.out == OUT_RESID) {
        lds_barrier();
        if (tid < R) {
          float s = 0.0f;
          for (int row = 0; row < 16; ++row) s += sq[row * kMaxRows + tid];
          st_c(a.ss + (size_t)tid * (a.H / kTileRows) + t, s);
        }
        lds_barrier();
      }
    }
  }
  if (ph.out == OUT_LOGITS) {
    if (tid < 16 * R) {
      cval[(tid / R) * kMaxRows + tid % R] = best_v;
      cidx[(tid / R) * kMaxRows + tid % R] = best_i;
    }
    lds_barrier();
    if (tid < R) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int row = 0; row < 16; ++row) {
        float v = cval[row * kMaxRows + tid];
        int ix = cidx[row * kMaxRows + tid];
        if (v > bv || (v == bv && ix < bi)) { bv = v; bi = ix; }
      }
      st_c(a.cand + ((size_t)wg * R + tid) * 2, bv);
      st_ci(reinterpret_cast<int32_t *>(a.cand) + ((size_t)wg * R + tid) * 2 + 1, bi);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// gated delta rule: per (sequence, head, 8 state rows); one wave per state row, 2 channels per lane
// ---------------------------------------------------------------------------------------------
__device__ void delta_phase(const StepArgs &a, const Phase &ph) {
  const int R = a.R, Hl = a.lin_heads, dk = a.dk, dv = a.dv;
  const int RB = dv / kWaves;  // row blocks of 8 rows
  const int nseq = a.verify ? 1 : R;
  const int U = nseq * Hl * RB;
  const int G = gridDim.x, wg = blockIdx.x;
  const int u0 = (int)(((int64_t)U * wg) / G), u1 = (int)(((int64_t)U * (wg + 1)) / G);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float *src = a.part[ph.src_part];
  for (int u = u0; u < u1; ++u) {
    const int b = u / (Hl * RB), h = (u / RB) % Hl, rb = u % RB;
    const int r = rb * kWaves + wave;
    const int c0 = lane * 2;
    float *Srow = reinterpret_cast<float *>(a.ls[ph.layer]) + (((size_t)b * Hl + h) * dv + r) * dk;
    float2 S = *reinterpret_cast<const float2 *>(Srow + c0);
    const int j0 = a.verify ? 0 : b, j1 = a.verify ? a.R : b + 1;
    for (int j = j0; j < j1; ++j) {
      float q0 = 0, q1 = 0, k0 = 0, k1 = 0, vr = 0, av0 = 0, av1 = 0, bv = 0;
      for (int s2 = 0; s2 < ph.src_S; ++s2) {
        const float *row = src + ((size_t)s2 * R + j) * ph.src_N;
        float2 qq = *reinterpret_cast<const float2 *>(row + ph.q_off + h * dk + c0);
        float2 kk = *reinterpret_cast<const float2 *>(row + ph.k_off + h * dk + c0);
        q0 += qq.x; q1 += qq.y; k0 += kk.x; k1 += kk.y;
        vr += row[ph.v_off + h * dv + r];
        if (ph.per_channel_gate) {
          float2 aa = *reinterpret_cast<const float2 *>(row + ph.a_off + h * dk + c0);
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

// ---------------------------------------------------------------------------------------------
// split-KV grouped-query attention: per (sequence, kv head, chunk of positions)
// ---------------------------------------------------------------------------------------------
__device__ void attn_phase(const StepArgs &a, const Phase &ph, char *smem) {
  const int R = a.R, nq = a.nq, nkv = a.nkv, hd = a.hd, grp = nq / nkv;
  const int CS = ph.chunk, NC = ph.n_chunks;
  const int nseq = a.verify ? 1 : R;
  const int nrow = a.verify ? R : 1;  // query rows per unit
  const int Q = grp * nrow;
  const int U = nseq * nkv * NC;
  const int G = gridDim.x, wg = blockIdx.x, tid = threadIdx.x;
  const int u0 = (int)(((int64_t)U * wg) / G), u1 = (int)(((int64_t)U * (wg + 1)) / G);
  const float scale = 1.0f / sqrtf((float)hd);
  const int half = hd / 2;
  float *qs = reinterpret_cast<float *>(smem);                       // [Q][hd]       32 KiB
  uint16_t *Ks = reinterpret_cast<uint16_t *>(qs + kAttnMaxQ * 128);   // [CS][hd] bf16 32 KiB
  uint16_t *Vs = Ks + kAttnMaxChunk * 128;                             // [CS][hd] bf16 32 KiB
  float *sc = reinterpret_cast<float *>(Vs + kAttnMaxChunk * 128);     // [Q][CS]       32 KiB
  float *ml = sc + kAttnMaxQ * kAttnMaxChunk;                          // [Q][2]
  int *rpos = reinterpret_cast<int *>(ml + kAttnMaxQ * 2);             // [nrow]
  const float *src = a.part[ph.src_part];
  uint16_t *kc = reinterpret_cast<uint16_t *>(a.kc[ph.layer]);
  uint16_t *vc = reinterpret_cast<uint16_t *>(a.vc[ph.layer]);

  for (int u = u0; u < u1; ++u) {
    const int b = u / (nkv * NC), g = (u / NC) % nkv, c = u % NC;
    const int seq = a.verify ? 0 : b;
    const int pbase = a.pos[seq];
    lds_barrier();
    if (tid < nrow) rpos[tid] = pbase + tid;
    const int maxpos = pbase + nrow - 1;
    const int c0 = c * CS;
    const int c1 = min(c0 + CS, min(a.max_ctx, maxpos + 1));  // positions [c0, c1) are read
    // queries (sum of k-split partials), rotated
    for (int idx = tid; idx < Q * hd; idx += kThreads) {
      const int qi = idx / hd, i = idx % hd, rr = qi / grp, hh = qi % grp;
      const int row = a.verify ? rr : b;
      const int h = g * grp + hh;
      float s = 0.0f;
      for (int s2 = 0; s2 < ph.src_S; ++s2) s += src[((size_t)s2 * R + row) * ph.src_N + ph.q_off + h * hd + i];
      qs[qi * hd + i] = s;
    }
    lds_barrier();
    for (int idx = tid; idx < Q * half; idx += kThreads) {
      const int qi = idx / half, i = idx % half, rr = qi / grp;
      const float2 cs = reinterpret_cast<const float2 *>(a.rope)[(size_t)rpos[rr] * half + i];
      const float x0 = qs[qi * hd + i], x1 = qs[qi * hd + i + half];
      qs[qi * hd + i] = x0 * cs.x - x1 * cs.y;
      qs[qi * hd + i + half] = x0 * cs.y + x1 * cs.x;
    }
    // K and V of the chunk: cached rows from memory, new rows from this step's projections
    const int npos = max(c1 - c0, 0);
    for (int idx = tid; idx < npos * (hd / 8); idx += kThreads) {
      const int jj = idx / (hd / 8), i8 = (idx % (hd / 8)) * 8, j = c0 + jj;
      if (j < pbase) {
        const size_t off = (((size_t)seq * nkv + g) * a.max_ctx + j) * hd + i8;
        *reinterpret_cast<uint4 *>(Ks + jj * hd + i8) = *reinterpret_cast<const uint4 *>(kc + off);
        *reinterpret_cast<uint4 *>(Vs + jj * hd + i8) = *reinterpret_cast<const uint4 *>(vc + off);
      }
    }
    for (int idx = tid; idx < npos * half; idx += kThreads) {
      const int jj = idx / half, i = idx % half, j = c0 + jj;
      if (j >= pbase) {  // a new row of this step
        const int row = a.verify ? (j - pbase) : b;
        float k0 = 0, k1 = 0, v0 = 0, v1 = 0;
        for (int s2 = 0; s2 < ph.src_S; ++s2) {
          const float *pr = src + ((size_t)s2 * R + row) * ph.src_N;
          k0 += pr[ph.k_off + g * hd + i];
          k1 += pr[ph.k_off + g * hd + i + half];
          v0 += pr[ph.v_off + g * hd + i];
          v1 += pr[ph.v_off + g * hd + i + half];
        }
        const float2 cs = reinterpret_cast<const float2 *>(a.rope)[(size_t)j * half + i];
        const uint16_t kr0 = f2bf(k0 * cs.x - k1 * cs.y), kr1 = f2bf(k0 * cs.y + k1 * cs.x);
        const uint16_t vb0 = f2bf(v0), vb1 = f2bf(v1);
        Ks[jj * hd + i] = kr0; Ks[jj * hd + i + half] = kr1;
        Vs[jj * hd + i] = vb0; Vs[jj * hd + i + half] = vb1;
        const size_t off = (((size_t)seq * nkv + g) * a.max_ctx + j) * hd;
        kc[off + i] = kr0; kc[off + i + half] = kr1;
        vc[off + i] = vb0; vc[off + i + half] = vb1;
      }
    }
    lds_barrier();
    // scores
    for (int idx = tid; idx < Q * CS; idx += kThreads) {
      const int qi = idx / CS, jj = idx % CS, j = c0 + jj;
      float s = -INFINITY;
      if (jj < npos && j <= rpos[qi / grp]) {
        float acc = 0.0f;
        const float *qv = qs + qi * hd;
        const uint16_t *kv = Ks + jj * hd;
        for (int i = 0; i < hd; i += 8) {
          uint4 kk = *reinterpret_cast<const uint4 *>(kv + i);
          uint32_t kw[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) acc += qv[i + e] * bf2f((uint16_t)(kw[e >> 1] >> ((e & 1) * 16)));
        }
        s = acc * scale;
      }
      sc[qi * CS + jj] = s;
    }
    lds_barrier();
    if (tid < Q) {
      float m = -INFINITY;
      for (int jj = 0; jj < CS; ++jj) m = fmaxf(m, sc[tid * CS + jj]);
      float l = 0.0f;
      for (int jj = 0; jj < CS; ++jj) {
        const float p = (m == -INFINITY) ? 0.0f : __expf(sc[tid * CS + jj] - m);
        sc[tid * CS + jj] = p;
        l += p;
      }
      ml[tid * 2] = m;
      ml[tid * 2 + 1] = l;
    }
    lds_barrier();
    for (int idx = tid; idx < Q * hd; idx += kThreads) {
      const int qi = idx / hd, i = idx % hd, rr = qi / grp, hh = qi % grp;
      float acc = 0.0f;
      for (int jj = 0; jj < npos; ++jj) acc += sc[qi * CS + jj] * bf2f(Vs[jj * hd + i]);
      const int row = a.verify ? rr : b, h = g * grp + hh;
      float *dst = a.attn + (((size_t)row * nq + h) * NC + c) * (hd + 2);
      st_c(dst + 2 + i, acc);
      if (i == 0) { st_c(dst, ml[qi * 2]); st_c(dst + 1, ml[qi * 2 + 1]); }
    }
  }
}

__device__ void merge_phase(const StepArgs &a, const Phase &ph) {
  const int R = a.R, nq = a.nq, hd = a.hd, NC = ph.n_chunks;
  const int U = R * nq;
  const int G = gridDim.x, wg = blockIdx.x, tid = threadIdx.x;
  const int u0 = (int)(((int64_t)U * wg) / G), u1 = (int)(((int64_t)U * (wg + 1)) / G);
  for (int u = u0; u < u1; ++u) {
    const int row = u / nq, h = u % nq;
    const float *p = a.attn + ((size_t)row * nq + h) * NC * (hd + 2);
    for (int i = tid; i < hd; i += kThreads) {
      float M = -INFINITY;
      for (int c = 0; c < NC; ++c)
        if (p[c * (hd + 2) + 1] > 0.0f) M = fmaxf(M, p[c * (hd + 2)]);
      float L = 0.0f, o = 0.0f;
      for (int c = 0; c < NC; ++c) {
        const float l = p[c * (hd + 2) + 1];
        if (l > 0.0f) {
          const float w = __expf(p[c * (hd + 2)] - M);
          L += l * w;
          o += p[c * (hd + 2) + 2 + i] * w;
        }
      }
      st_c(a.mix + (size_t)row * a.mix_stride + h * hd + i, o / L);
    }
  }
}

__device__ void embed_phase(const StepArgs &a, const Phase &ph, char *smem) {
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

__device__ void final_phase(const StepArgs &a, char *smem) {
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

__device__ void hidden_out_phase(const StepArgs &a) {
  const size_t n = (size_t)a.R * a.H;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (size_t)gridDim.x * kThreads)
    a.hidden_out[i] = ld_c(a.x + i);
}

}  // namespace mk

using namespace mk;

// The step kernel: walks phases [phase_begin, phase_end) of the schedule. As a persistent launch it
// covers the whole step with a grid barrier between phases (all workgroups co-resident: cooperative
// launch, one workgroup per compute unit); the per-op baseline launches it once per phase.
extern "C" __global__ void __launch_bounds__(kThreads) mk_step_kernel(StepArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int abort_flag;
  uint32_t k = (a.epoch - 1u) * (uint32_t)a.n_barriers + (uint32_t)a.barrier_base;
  for (int p = a.phase_begin; p < a.phase_end; ++p) {
    const Phase ph = a.phases[p];
    switch (ph.type) {
      case PH_EMBED: embed_phase(a, ph, smem); break;
      case PH_GEMV: gemv_phase<8>(a, ph, smem); break;
      case PH_DELTA: delta_phase(a, ph); break;
      case PH_ATTN: attn_phase(a, ph, smem); break;
      case PH_MERGE: merge_phase(a, ph); break;
      case PH_FINAL: final_phase(a, smem); break;
      case PH_HIDDEN_OUT: hidden_out_phase(a); break;
      default: break;
    }
    if (p + 1 < a.phase_end) {
      ++k;
      if (!grid_barrier(a, k, p, &abort_flag)) return;
    }
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
