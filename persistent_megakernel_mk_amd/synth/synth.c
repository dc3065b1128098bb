/*
 * Seeded, counter-based synthetic inputs for the decode-step workloads (host side).
 *
 * This file holds input generation only: no step of the decoder is computed here.
 * The same definitions are implemented for the GPU in synth_gpu.hip; both sides
 * produce bit-identical values because every operation below is an integer
 * operation or a single correctly rounded IEEE fp32 operation (built with
 * -ffp-contract=off so no multiply-add is fused).
 *
 * Generator definition
 *   mix(z)     : the SplitMix64 output function (Steele, Lea, Flood, "Fast
 *                splittable pseudorandom number generators", OOPSLA 2014):
 *                z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
 *                z *= 0x94D049BB133111EB; z ^= z >> 31.
 *   G          : the golden-ratio increment 0x9E3779B97F4A7C15.
 *   key(s, t)  : mix(s * G + mix(t * G + 1))   -- one stream per (seed s, tensor id t)
 *   draw(k, j) : mix(k + (j + 1) * G)          -- 64 random bits, counter j
 *   normal(k,i): twelve 16-bit uniforms U_0..U_11 taken from draw(k, 3i), draw(k, 3i+1),
 *                draw(k, 3i+2) (four 16-bit fields each, low bits first);
 *                S = sum(U) - 393210 (an integer, mean 0, standard deviation ~65536);
 *                z = (float)S * (sigma / 65536) + mean, each step rounded to fp32.
 *                The centred sum of twelve uniforms is the classical Irwin-Hall
 *                approximation of a normal deviate: mean and variance match N(0,1)
 *                exactly (up to the 16-bit discreteness) and tails stop at 6 sigma.
 *   uniform_int(k, i, n): ((draw(k, i) >> 32) * n) >> 32, in [0, n).
 *   bf16 output: round-to-nearest-even of the fp32 value.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

#define SYN_G 0x9E3779B97F4A7C15ULL

static inline uint64_t syn_mix(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ULL;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t tensor_id) {
  return syn_mix(seed * SYN_G + syn_mix(tensor_id * SYN_G + 1ULL));
}

static inline uint64_t syn_draw(uint64_t key, uint64_t j) { return syn_mix(key + (j + 1ULL) * SYN_G); }

static inline int32_t syn_irwin12(uint64_t key, uint64_t i) {
  int64_t s = 0;
  for (int j = 0; j < 3; ++j) {
    uint64_t h = syn_draw(key, 3ULL * i + (uint64_t)j);
    s += (int64_t)(h & 0xffffULL) + (int64_t)((h >> 16) & 0xffffULL) + (int64_t)((h >> 32) & 0xffffULL) +
         (int64_t)(h >> 48);
  }
  return (int32_t)(s - 393210);
}

static inline float syn_normal(uint64_t key, uint64_t i, float scale, float mean) {
  float z = (float)syn_irwin12(key, i) * scale;
  return z + mean;
}

static inline uint16_t syn_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* out[i] = bf16(normal(key(seed,tid), offset + i)) for i < n. sigma/mean as documented above. */
void synth_normal_bf16(uint64_t seed, uint64_t tid, uint64_t offset, int64_t n, float sigma, float mean,
                       uint16_t *out) {
  const uint64_t key = synth_key(seed, tid);
  const float scale = sigma / 65536.0f;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = syn_bf16_rne(syn_normal(key, offset + (uint64_t)i, scale, mean));
}

void synth_normal_f32(uint64_t seed, uint64_t tid, uint64_t offset, int64_t n, float sigma, float mean, float *out) {
  const uint64_t key = synth_key(seed, tid);
  const float scale = sigma / 65536.0f;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = syn_normal(key, offset + (uint64_t)i, scale, mean);
}

void synth_uniform_int(uint64_t seed, uint64_t tid, uint64_t offset, int64_t n, uint32_t bound, int32_t *out) {
  const uint64_t key = synth_key(seed, tid);
  for (int64_t i = 0; i < n; ++i) {
    uint64_t h = syn_draw(key, offset + (uint64_t)i);
    out[i] = (int32_t)(((h >> 32) * (uint64_t)bound) >> 32);
  }
}

/* ---- NVFP4 encoding of synthetic weights (input preparation only) ----------------------------
 * Encodes a [rows][k] fp32 matrix as FP4 E2M1 codes (two per byte, element 2i in the low nibble),
 * one FP8 E4M3 (OCP e4m3fn) scale per 16 consecutive elements of a row, and one fp32 tensor scale:
 *   s_tensor = amax / (6 * 448); scale_blk = e4m3_rne(amax_blk / (6 * s_tensor));
 *   code = e2m1_rne(w / (decode(scale_blk) * s_tensor)).
 * The decode side of this format is part of the method and is not implemented here.            */

static const float syn_e2m1_mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

static uint8_t syn_e2m1_rne(float x) {
  uint8_t sign = x < 0.0f ? 8u : 0u;
  float a = fabsf(x);
  if (a >= 6.0f) return sign | 7u;
  /* nearest grid point; ties go to the even code (lowest mantissa bit 0) */
  int best = 0;
  for (int c = 1; c < 8; ++c) {
    float dc = fabsf(a - syn_e2m1_mag[c]), db = fabsf(a - syn_e2m1_mag[best]);
    if (dc < db || (dc == db && (c & 1) == 0)) best = c;
  }
  return sign | (uint8_t)best;
}

static float syn_e4m3_value(uint8_t c) {
  int e = (c >> 3) & 15, m = c & 7;
  float v = (e == 0) ? ldexpf((float)m / 8.0f, -6) : ldexpf(1.0f + (float)m / 8.0f, e - 7);
  return (c & 0x80) ? -v : v;
}

static uint8_t syn_e4m3_rne_pos(float a) {
  /* a >= 0: nearest finite E4M3 code, ties to even mantissa, saturating at 448 (code 0x7e) */
  if (!(a > 0.0f)) return 0;
  if (a >= 448.0f) return 0x7e;
  if (a < ldexpf(1.0f, -6)) {                /* subnormal range: units of 2^-9 */
    float m = nearbyintf(a * 512.0f);
    return (uint8_t)m;                         /* m == 8 is exactly the smallest normal, code 0x08 */
  }
  int e;
  float f = frexpf(a, &e);                     /* a = f * 2^e, f in [0.5, 1) */
  e -= 1;                                      /* a = (2f) * 2^e, 2f in [1, 2) */
  float m = nearbyintf((2.0f * f - 1.0f) * 8.0f);
  if (m >= 8.0f) { m = 0.0f; e += 1; }
  int E = e + 7;
  if (E > 15 || (E == 15 && m >= 7.0f)) return 0x7e;
  return (uint8_t)((E << 3) | (int)m);
}

/* MXFP4 encoding of seeded weights (Open Compute Project "OCP Microscaling Formats (MX) v1.0",
 * the MXFP4 element format with its conversion recipe): per block of 32 consecutive values along a row,
 * the shared E8M0 scale is X = 2^(floor(log2(amax)) - 2) (2 = the largest exponent of E2M1), and each
 * element becomes the E2M1 code of v / X rounded to nearest even, saturating at 6. An all-zero block
 * takes X = 2^-127 (code 0). Codes are packed as for NVFP4 (element 2i in the low nibble of byte i). */
void synth_mxfp4_encode(const float *w, int64_t rows, int64_t k, uint8_t *codes, uint8_t *scales) {
  const int64_t nb = k / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const float *blk = w + r * k + b * 32;
      float amax = 0.0f;
      for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(blk[e]));
      int ex = 0;
      if (amax > 0.0f) {
        int e2;
        frexpf(amax, &e2);                      /* amax = f * 2^e2, f in [0.5, 1): floor(log2 amax) = e2 - 1 */
        ex = (e2 - 1) - 2 + 127;
        if (ex < 0) ex = 0;
        if (ex > 254) ex = 254;
      }
      scales[r * nb + b] = (uint8_t)ex;
      const float X = ldexpf(1.0f, ex - 127);
      for (int e = 0; e < 32; e += 2) {
        uint8_t lo = amax > 0.0f ? syn_e2m1_rne(blk[e] / X) : 0;
        uint8_t hi = amax > 0.0f ? syn_e2m1_rne(blk[e + 1] / X) : 0;
        codes[r * (k / 2) + (b * 32 + e) / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}

void synth_nvfp4_encode(const float *w, int64_t rows, int64_t k, uint8_t *codes, uint8_t *scales, float *tensor_scale) {
  float amax = 0.0f;
  for (int64_t i = 0; i < rows * k; ++i) amax = fmaxf(amax, fabsf(w[i]));
  const float st = amax > 0.0f ? amax / (6.0f * 448.0f) : 1.0f;
  *tensor_scale = st;
  const int64_t nb = k / 16;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const float *blk = w + r * k + b * 16;
      float bmax = 0.0f;
      for (int e = 0; e < 16; ++e) bmax = fmaxf(bmax, fabsf(blk[e]));
      uint8_t sc = syn_e4m3_rne_pos(bmax / (6.0f * st));
      scales[r * nb + b] = sc;
      float denom = syn_e4m3_value(sc) * st;
      for (int e = 0; e < 16; e += 2) {
        uint8_t lo = denom > 0.0f ? syn_e2m1_rne(blk[e] / denom) : 0;
        uint8_t hi = denom > 0.0f ? syn_e2m1_rne(blk[e + 1] / denom) : 0;
        codes[r * (k / 2) + (b * 16 + e) / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}
