// CPU oracle for the persistent decode megakernel: the operations of one decode step, fp32.
//
// TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call this file; only the
// tests, the smoke check and the CPU-baseline leg of the benchmark do. It shares no code, header or
// table with the HIP path.
//
// What it computes. The pages ("Kimi K3's TPU megakernel: 92 layers in one Pallas call, and what 709
// tokens a second measures", sections "What a megakernel is, and what it fixes on a TPU" and "How it
// maps onto a TPU v7") describe a megakernel as the plain decoder step with op boundaries removed: the
// arithmetic is unchanged, only the timing of weight loads moves. So the oracle is the plain step:
// every function below is the textbook definition of one op, written as straight loops.
//
// Precision. The same page, section "How it maps onto a TPU v7", has the matrix units accumulate in
// FP32 with bf16 weights; here every weight or cache element is widened exactly from bf16 to fp32,
// every product is rounded to fp32 and every sum is accumulated sequentially in index order in fp32
// (built with -ffp-contract=off, so no multiply-add is fused). OpenMP splits only independent output
// rows, so results are identical for any thread count.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

extern "C" {

// ---- bf16 <-> fp32 ---------------------------------------------------------------------------
float orc_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// round to nearest, ties to even (used where the step stores a value in a bf16 cache)
uint16_t orc_f32_to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

void orc_widen_bf16(const uint16_t* src, int64_t n, float* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = orc_bf16_to_f32(src[i]);
}

void orc_round_bf16(const float* src, int64_t n, uint16_t* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = orc_f32_to_bf16(src[i]);
}

// ---- matrix-vector product -------------------------------------------------------------------
// Y[b][n] = sum_k W[n][k] * X[b][k], W bf16 row-major [N][K], X and Y fp32.
void orc_gemv_bf16(const uint16_t* W, int64_t N, int64_t K, const float* X, int B, float* Y) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    const uint16_t* w = W + n * K;
    for (int b = 0; b < B; ++b) {
      const float* x = X + (int64_t)b * K;
      float acc = 0.0f;
      for (int64_t k = 0; k < K; ++k) acc += orc_bf16_to_f32(w[k]) * x[k];
      Y[(int64_t)b * N + n] = acc;
    }
  }
}

// ---- NVFP4 (FP4 E2M1 values, FP8 E4M3 scale per 16 elements, fp32 tensor scale) --------------
// E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa; exponent 0 is subnormal (m * 0.5).
float orc_e2m1_value(uint8_t nib) {
  int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
  float v = (e == 0) ? 0.5f * (float)m : std::ldexp(1.0f + 0.5f * (float)m, e - 1);
  return s ? -v : v;
}

// E4M3 as OCP e4m3fn: bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa; no infinities;
// S.1111.111 is NaN; exponent 0 is subnormal (2^-6 * m/8).
float orc_e4m3_value(uint8_t c) {
  int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return std::nanf("");
  float v = (e == 0) ? std::ldexp((float)m / 8.0f, -6) : std::ldexp(1.0f + (float)m / 8.0f, e - 7);
  return s ? -v : v;
}

// One row of K weights: element j = e2m1(code_j) * e4m3(scale_{j/16}) * tensor_scale, where code_j
// is the low nibble of byte j/2 for even j and the high nibble for odd j. The product of the two
// narrow values is exact in fp32; the tensor scale is the one rounded multiply.
void orc_nvfp4_dequant_row(const uint8_t* codes, const uint8_t* scales, float tensor_scale, int64_t K, float* out) {
  for (int64_t j = 0; j < K; ++j) {
    uint8_t byte = codes[j / 2];
    uint8_t nib = (j & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
    out[j] = (orc_e2m1_value(nib) * orc_e4m3_value(scales[j / 16])) * tensor_scale;
  }
}

void orc_gemv_nvfp4(const uint8_t* codes, const uint8_t* scales, float tensor_scale, int64_t N, int64_t K,
                    const float* X, int B, float* Y) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    std::vector<float> w((size_t)K);
    orc_nvfp4_dequant_row(codes + n * (K / 2), scales + n * (K / 16), tensor_scale, K, w.data());
    for (int b = 0; b < B; ++b) {
      const float* x = X + (int64_t)b * K;
      float acc = 0.0f;
      for (int64_t k = 0; k < K; ++k) acc += w[(size_t)k] * x[k];
      Y[(int64_t)b * N + n] = acc;
    }
  }
}

// ---- MXFP4 (FP4 E2M1 values, E8M0 scale per 32 elements) and its FP8 re-encoding ---------------
// E8M0: an 8-bit biased exponent, value 2^(e - 127); 0xFF is NaN (OCP Microscaling Formats v1.0).
float orc_e8m0_value(uint8_t e) {
  if (e == 0xFF) return std::nanf("");
  return std::ldexp(1.0f, (int)e - 127);
}

// One row of K weights: element j = e2m1(code_j) * 2^(e_{j/32} - 127), exact in fp32.
void orc_mxfp4_dequant_row(const uint8_t* codes, const uint8_t* scales, int64_t K, float* out) {
  for (int64_t j = 0; j < K; ++j) {
    uint8_t byte = codes[j / 2];
    uint8_t nib = (j & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
    out[j] = orc_e2m1_value(nib) * orc_e8m0_value(scales[j / 32]);
  }
}

void orc_gemv_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K, const float* X, int B, float* Y) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    std::vector<float> w((size_t)K);
    orc_mxfp4_dequant_row(codes + n * (K / 2), scales + n * (K / 32), K, w.data());
    for (int b = 0; b < B; ++b) {
      const float* x = X + (int64_t)b * K;
      float acc = 0.0f;
      for (int64_t k = 0; k < K; ++k) acc += w[(size_t)k] * x[k];
      Y[(int64_t)b * N + n] = acc;
    }
  }
}

// E4M3 (OCP e4m3fn) code of a value that the format holds exactly, else of its nearest (ties to even,
// saturating at 448); the caller checks exactness by decoding.
static uint8_t orc_e4m3_encode(float v) {
  const uint8_t sign = std::signbit(v) ? 0x80 : 0;
  const float a = std::fabs(v);
  if (a == 0.0f) return sign;
  if (a >= 448.0f) return sign | 0x7E;
  if (a < std::ldexp(1.0f, -6)) {  // subnormals: multiples of 2^-9 (8 * 2^-9 is the smallest normal)
    return sign | (uint8_t)std::nearbyint(a * 512.0f);
  }
  int e;
  const float f = std::frexp(a, &e);  // a = f * 2^e, f in [0.5, 1)
  e -= 1;                              // a = (2 f) * 2^e
  float q = std::nearbyint((2.0f * f - 1.0f) * 8.0f);  // three mantissa bits, ties to even
  if (q == 8.0f) { q = 0.0f; e += 1; }
  const int E = e + 7;
  if (E > 15 || (E == 15 && q == 7.0f)) return sign | 0x7E;
  return sign | (uint8_t)((E << 3) | (int)q);
}

// The loader's re-encoding of an MXFP4 gate or up matrix [N][K] into FP8 E4M3 values with one bf16
// scale per 256 consecutive elements of a row (page "Kimi K3's TPU megakernel ...", section "How it maps
// onto a TPU v7", the precision paragraph). Per (row, 256-block) the scale is the power of two
// S = 2^(m - 133), m the largest E8M0 exponent among the block's 32-blocks that hold a nonzero code
// (S = 1 for an all-zero block), so every element becomes e2m1 * 2^(e - m + 6) with |value| <= 6 * 2^6
// = 384 <= 448. The re-encoding is lossless when decode(fp8) * S equals the MXFP4 value bit for bit for
// every element; returns the number of elements where it does not (0: lossless).
int64_t orc_fp8_reencode(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K, uint8_t* fp8,
                         uint16_t* bscale) {
  int64_t bad = 0;
  const int64_t KB = K / 256;
#pragma omp parallel for schedule(static) reduction(+ : bad)
  for (int64_t n = 0; n < N; ++n) {
    std::vector<float> w((size_t)K);
    orc_mxfp4_dequant_row(codes + n * (K / 2), scales + n * (K / 32), K, w.data());
    for (int64_t kb = 0; kb < KB; ++kb) {
      int m = -1;
      for (int j = 0; j < 8; ++j) {
        bool nz = false;
        for (int e = 0; e < 32; ++e) nz |= w[(size_t)(kb * 256 + j * 32 + e)] != 0.0f;
        if (nz) m = std::max(m, (int)scales[n * (K / 32) + kb * 8 + j]);
      }
      const float S = m < 0 ? 1.0f : std::ldexp(1.0f, m - 133);
      const uint16_t sb = orc_f32_to_bf16(S);  // a power of two: exact in bf16
      bscale[n * KB + kb] = sb;
      const float Sd = orc_bf16_to_f32(sb);
      for (int e = 0; e < 256; ++e) {
        const int64_t j = kb * 256 + e;
        const float v = w[(size_t)j];
        const uint8_t c = orc_e4m3_encode(v / Sd);
        fp8[n * K + j] = c;
        const float back = orc_e4m3_value(c) * Sd;
        uint32_t ub, uv;
        std::memcpy(&ub, &back, 4);
        std::memcpy(&uv, &v, 4);
        if (ub != uv) ++bad;
      }
    }
  }
  return bad;
}

// Y[b][n] = sum_k (e4m3(fp8[n][k]) * bscale[n][k / 256]) * X[b][k]
void orc_gemv_fp8r(const uint8_t* fp8, const uint16_t* bscale, int64_t N, int64_t K, const float* X, int B, float* Y) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    std::vector<float> w((size_t)K);
    for (int64_t k = 0; k < K; ++k) w[(size_t)k] = orc_e4m3_value(fp8[n * K + k]) * orc_bf16_to_f32(bscale[n * (K / 256) + k / 256]);
    for (int b = 0; b < B; ++b) {
      const float* x = X + (int64_t)b * K;
      float acc = 0.0f;
      for (int64_t k = 0; k < K; ++k) acc += w[(size_t)k] * x[k];
      Y[(int64_t)b * N + n] = acc;
    }
  }
}

// ---- normalisations --------------------------------------------------------------------------
// RMSNorm: y_i = x_i * (1 / sqrt(mean_j x_j^2 + eps)) * g_i
void orc_rmsnorm(const float* X, const uint16_t* g, int B, int64_t H, float eps, float* Y) {
  for (int b = 0; b < B; ++b) {
    const float* x = X + (int64_t)b * H;
    float ss = 0.0f;
    for (int64_t i = 0; i < H; ++i) ss += x[i] * x[i];
    float r = 1.0f / std::sqrt(ss / (float)H + eps);
    for (int64_t i = 0; i < H; ++i) Y[(int64_t)b * H + i] = (x[i] * r) * orc_bf16_to_f32(g[i]);
  }
}

// L2 normalisation of n_vec vectors of length d: v <- v / sqrt(sum v^2 + eps)
void orc_l2norm(float* v, int n_vec, int d, float eps) {
  for (int h = 0; h < n_vec; ++h) {
    float* x = v + (int64_t)h * d;
    float ss = 0.0f;
    for (int i = 0; i < d; ++i) ss += x[i] * x[i];
    float r = 1.0f / std::sqrt(ss + eps);
    for (int i = 0; i < d; ++i) x[i] = x[i] * r;
  }
}

// ---- rotary position embedding ---------------------------------------------------------------
// For each of n_vec vectors (start at v + h*stride + offset), rotate the pairs (i, i + rot/2),
// i < rot/2, by the angle pos * theta^(-2i/rot). Angles and their sine/cosine in double, rounded
// to fp32 before use.
void orc_rope(float* v, int n_vec, int stride, int offset, int rot, int64_t pos, double theta) {
  const int half = rot / 2;
  for (int h = 0; h < n_vec; ++h) {
    float* x = v + (int64_t)h * stride + offset;
    for (int i = 0; i < half; ++i) {
      double ang = (double)pos * std::pow(theta, -2.0 * (double)i / (double)rot);
      float c = (float)std::cos(ang), s = (float)std::sin(ang);
      float a = x[i], b = x[i + half];
      x[i] = a * c - b * s;
      x[i + half] = a * s + b * c;
    }
  }
}

// ---- softmax attention over a bf16 cache (grouped-query) -------------------------------------
// q: [nq][d] fp32 (already rotated). Kc, Vc: this sequence's caches, [nkv][head_stride/d][d] bf16.
// Query head h reads kv head h / (nq / nkv). Positions 0..L-1 are attended.
// s_j = (q . k_j) * (1/sqrt(d)); p = softmax(s) with max subtraction; o = sum_j p_j v_j.
void orc_attention(const float* q, int nq, int d, const uint16_t* Kc, const uint16_t* Vc, int nkv,
                   int64_t head_stride, int64_t L, float* o) {
  const int group = nq / nkv;
  const float scale = 1.0f / std::sqrt((float)d);
  std::vector<float> s((size_t)L);
  for (int h = 0; h < nq; ++h) {
    const int g = h / group;
    const float* qh = q + (int64_t)h * d;
    const uint16_t* K = Kc + (int64_t)g * head_stride;
    const uint16_t* V = Vc + (int64_t)g * head_stride;
    float m = -INFINITY;
    for (int64_t j = 0; j < L; ++j) {
      float acc = 0.0f;
      for (int i = 0; i < d; ++i) acc += qh[i] * orc_bf16_to_f32(K[j * d + i]);
      s[(size_t)j] = acc * scale;
      if (s[(size_t)j] > m) m = s[(size_t)j];
    }
    float l = 0.0f;
    for (int64_t j = 0; j < L; ++j) {
      s[(size_t)j] = std::exp(s[(size_t)j] - m);
      l += s[(size_t)j];
    }
    for (int i = 0; i < d; ++i) {
      float acc = 0.0f;
      for (int64_t j = 0; j < L; ++j) acc += s[(size_t)j] * orc_bf16_to_f32(V[j * d + i]);
      o[(int64_t)h * d + i] = acc / l;
    }
  }
}

// ---- gates -----------------------------------------------------------------------------------
float orc_sigmoid(float z) { return 1.0f / (1.0f + std::exp(-z)); }

float orc_softplus(float a) { return a > 20.0f ? a : std::log1p(std::exp(a)); }

// decay alpha = exp(-softplus(a)) in (0, 1); write strength beta = sigmoid(b)
void orc_decay_gates(const float* a, int n, float* alpha) {
  for (int i = 0; i < n; ++i) alpha[i] = std::exp(-orc_softplus(a[i]));
}

void orc_sigmoid_vec(const float* z, int n, float* out) {
  for (int i = 0; i < n; ++i) out[i] = orc_sigmoid(z[i]);
}

// ---- gated delta rule: one token, one head ---------------------------------------------------
// State S is d_v x d_k (row r holds the d_k-vector that maps keys to output channel r).
//   S <- S Diag(alpha) (I - beta k k^T) + beta v k^T,   o = S q
// evaluated row by row: S_r <- S_r * alpha (per column); u = S_r . k; S_r <- S_r + beta (v_r - u) k;
// o_r = S_r . q. A scalar gate (gated DeltaNet) passes alpha with all d_k entries equal; a
// per-channel gate (Kimi delta attention) passes d_k different entries.
void orc_delta_step(float* S, int dk, int dv, const float* q, const float* k, const float* v, const float* alpha,
                    float beta, float* o) {
  for (int r = 0; r < dv; ++r) {
    float* row = S + (int64_t)r * dk;
    for (int c = 0; c < dk; ++c) row[c] = row[c] * alpha[c];
    float u = 0.0f;
    for (int c = 0; c < dk; ++c) u += row[c] * k[c];
    float delta = beta * (v[r] - u);
    for (int c = 0; c < dk; ++c) row[c] = row[c] + delta * k[c];
    float acc = 0.0f;
    for (int c = 0; c < dk; ++c) acc += row[c] * q[c];
    o[r] = acc;
  }
}

// ---- multi-head latent attention, absorbed form, one sequence --------------------------------
// q: [heads][nope + rope] (nope part first; rope part already rotated). cache: [L'][rank + rope]
// bf16, each position holding the latent c_j (rank) then its rotated key k_r,j (rope), positions
// 0..L-1 attended. wuk: [heads*nope][rank] (maps a latent to per-head keys), wuv: [heads*vdim][rank].
//   q~_h = W_uk,h^T q_nope,h;  s_j = (q~_h . c_j + q_rope,h . k_r,j) / sqrt(nope + rope)
//   p = softmax(s);  obar_h = sum_j p_j c_j;  out_h = W_uv,h obar_h
void orc_mla_attend(const float* q, int heads, int nope, int rope, const uint16_t* wuk, const uint16_t* wuv, int rank,
                    int vdim, const uint16_t* cache, int64_t L, float* out) {
  const int row = rank + rope;
  const float scale = 1.0f / std::sqrt((float)(nope + rope));
  std::vector<float> qt((size_t)rank), s((size_t)L), ob((size_t)rank);
  for (int h = 0; h < heads; ++h) {
    const float* qn = q + (int64_t)h * (nope + rope);
    const float* qr = qn + nope;
    for (int c = 0; c < rank; ++c) {
      float acc = 0.0f;
      for (int n = 0; n < nope; ++n) acc += orc_bf16_to_f32(wuk[((int64_t)h * nope + n) * rank + c]) * qn[n];
      qt[(size_t)c] = acc;
    }
    float m = -INFINITY;
    for (int64_t j = 0; j < L; ++j) {
      const uint16_t* cj = cache + j * row;
      float a = 0.0f;
      for (int c = 0; c < rank; ++c) a += qt[(size_t)c] * orc_bf16_to_f32(cj[c]);
      float b = 0.0f;
      for (int r = 0; r < rope; ++r) b += qr[r] * orc_bf16_to_f32(cj[rank + r]);
      s[(size_t)j] = (a + b) * scale;
      if (s[(size_t)j] > m) m = s[(size_t)j];
    }
    float l = 0.0f;
    for (int64_t j = 0; j < L; ++j) {
      s[(size_t)j] = std::exp(s[(size_t)j] - m);
      l += s[(size_t)j];
    }
    for (int c = 0; c < rank; ++c) {
      float acc = 0.0f;
      for (int64_t j = 0; j < L; ++j) acc += s[(size_t)j] * orc_bf16_to_f32(cache[j * row + c]);
      ob[(size_t)c] = acc / l;
    }
    for (int vv = 0; vv < vdim; ++vv) {
      float acc = 0.0f;
      for (int c = 0; c < rank; ++c) acc += orc_bf16_to_f32(wuv[((int64_t)h * vdim + vv) * rank + c]) * ob[(size_t)c];
      out[(int64_t)h * vdim + vv] = acc;
    }
  }
}

// ---- router: top-k as k sequential argmax passes ---------------------------------------------
// The page "Kimi K3's TPU megakernel ...", section "How it maps onto a TPU v7", computes the router's
// top-16 as sixteen sequential argmax passes; an argmax keeps the first maximum, so ties go to the
// lowest expert index. Selection is on the router logit z (sigmoid is monotone, so the set equals
// the top-k of the sigmoid scores); gates are the selected sigmoid scores normalised to sum to 1.
void orc_topk(const float* z, int E, int k, int* idx, float* gates) {
  std::vector<char> taken((size_t)E, 0);
  float total = 0.0f;
  for (int t = 0; t < k; ++t) {
    int best = -1;
    for (int e = 0; e < E; ++e) {
      if (taken[(size_t)e]) continue;
      if (best < 0 || z[e] > z[best]) best = e;
    }
    taken[(size_t)best] = 1;
    idx[t] = best;
    gates[t] = orc_sigmoid(z[best]);
    total += gates[t];
  }
  for (int t = 0; t < k; ++t) gates[t] = gates[t] / total;
}

// ---- residual add and expert combine ---------------------------------------------------------
// x <- x + o (one residual block's output added to the residual stream; page "Kimi K3's TPU
// megakernel ...", section "How it maps onto a TPU v7": mixer then residual, FFN then residual)
void orc_residual_add(float* x, const float* o, int64_t n) {
  for (int64_t i = 0; i < n; ++i) x[i] = x[i] + o[i];
}

// acc <- acc + w * y: one expert's output added with its gate weight (shared experts pass w = 1,
// routed experts their normalised score; same page and section: shared expert, then routed experts)
void orc_moe_accumulate(float* acc, const float* y, float w, int64_t n) {
  for (int64_t i = 0; i < n; ++i) acc[i] = acc[i] + w * y[i];
}

// ---- SwiGLU activation and argmax ------------------------------------------------------------
// h = silu(g) * u with silu(t) = t / (1 + exp(-t))
void orc_silu_mul(const float* g, const float* u, int64_t n, float* h) {
  for (int64_t i = 0; i < n; ++i) h[i] = (g[i] / (1.0f + std::exp(-g[i]))) * u[i];
}

// first index of the maximum
int64_t orc_argmax(const float* x, int64_t n) {
  int64_t best = 0;
  for (int64_t i = 1; i < n; ++i)
    if (x[i] > x[best]) best = i;
  return best;
}

}  // extern "C"
