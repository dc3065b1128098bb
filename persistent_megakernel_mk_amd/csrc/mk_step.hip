// The step kernel for weights in bf16 only, and the kernels that repack weights into the layouts the
// step streams. The step's device code is in mk_device.h.
#include "mk_device.h"

extern "C" __global__ void __launch_bounds__(kThreads) mk_step_kernel(StepArgs args) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  (void)args;
  step_body<false, kRing>(smem);
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

// NVFP4 repacking: codes uint8 [rows][cols/2] (element 2i in the low nibble of byte i) and E4M3 scales
// uint8 [rows][cols/16] -> the stream layout of a dst_rows x cols matrix whose rows row_off.. this
// tensor fills (row_off a multiple of 16). Per 16-row tile t and 128-column group g, 1 KiB of codes:
// lane l holds row l%16, columns g*128 + 32f + 8*(l/16) .. +7 in bytes 4f..4f+3 (f = 0..3, the four
// MFMA fragments of the group). After all tiles' codes come the scales, 128 B per (t, g): word
// r + 16h holds in byte f the scale of row r, 16-column block 8g + 2f + h (the block the lanes with
// l/16 in {2h, 2h+1} use for fragment f).
extern "C" __global__ void mk_repack_nvfp4(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales, int64_t rows,
                                           int64_t cols, uint8_t *__restrict__ dst, int64_t row_off, int64_t dst_rows) {
  const int64_t NG = cols / 128, T = rows / 16;
  const int64_t total = T * NG * 64;
  uint8_t *sdst = dst + (dst_rows / 16) * NG * 1024;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * blockDim.x) {
    const int lane = (int)(idx & 63);
    const int64_t tg = idx >> 6, t = tg / NG, g = tg - t * NG;
    const int64_t dtg = (row_off / 16 + t) * NG + g;  // destination (tile, group)
    const int64_t r = t * 16 + (lane & 15);
    const int kg = lane >> 4;
    uint32_t w[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) w[f] = *reinterpret_cast<const uint32_t *>(codes + r * (cols / 2) + g * 64 + f * 16 + kg * 4);
    *reinterpret_cast<uint4 *>(dst + (dtg * 64 + lane) * 16) = uint4{w[0], w[1], w[2], w[3]};
    if (lane < 32) {
      const int64_t r2 = t * 16 + (lane & 15);
      const int h = lane >> 4;
      uint32_t v = 0;
#pragma unroll
      for (int f = 0; f < 4; ++f) v |= (uint32_t)scales[r2 * (cols / 16) + g * 8 + 2 * f + h] << (8 * f);
      *reinterpret_cast<uint32_t *>(sdst + (dtg * 32 + lane) * 4) = v;
    }
  }
}

// MXFP4 repacking: codes uint8 [rows][cols/2] (element 2i in the low nibble of byte i) and E8M0 scales
// uint8 [rows][cols/32] -> the stream layout of a dst_rows x cols matrix whose rows row_off.. this tensor
// fills. The codes of a (tile, 128-column group) are laid out as for NVFP4; after all codes come the
// scales, 64 B per (tile, group): word r holds in byte f the scale of row r, 32-column block 4g + f (the
// block of the group's fragment f, shared by all four lane groups).
extern "C" __global__ void mk_repack_mxfp4(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales, int64_t rows,
                                           int64_t cols, uint8_t *__restrict__ dst, int64_t row_off, int64_t dst_rows) {
  const int64_t NG = cols / 128, T = rows / 16;
  const int64_t total = T * NG * 64;
  uint8_t *sdst = dst + (dst_rows / 16) * NG * 1024;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * blockDim.x) {
    const int lane = (int)(idx & 63);
    const int64_t tg = idx >> 6, t = tg / NG, g = tg - t * NG;
    const int64_t dtg = (row_off / 16 + t) * NG + g;  // destination (tile, group)
    const int64_t r = t * 16 + (lane & 15);
    const int kg = lane >> 4;
    uint32_t w[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) w[f] = *reinterpret_cast<const uint32_t *>(codes + r * (cols / 2) + g * 64 + f * 16 + kg * 4);
    *reinterpret_cast<uint4 *>(dst + (dtg * 64 + lane) * 16) = uint4{w[0], w[1], w[2], w[3]};
    if (lane < 16) {
      const uint32_t v = *reinterpret_cast<const uint32_t *>(scales + r * (cols / 32) + g * 4);  // blocks 4g .. 4g+3
      *reinterpret_cast<uint32_t *>(sdst + (dtg * 16 + lane) * 4) = v;
    }
  }
}

// FP8 re-encoding of an MXFP4 gate or up matrix [rows][cols] (codes and E8M0 scales as above) into rows
// row_off.. of a dst_rows x cols FP8 E4M3 matrix with one bf16 scale per 256 consecutive elements of a row
// (the loader step of page "Kimi K3's TPU megakernel: 92 layers in one Pallas call, and what 709 tokens a
// second measures", section "How it maps onto a TPU v7", the precision paragraph). One thread per (row,
// 256-column block): the scale is 2^(m - 133), m the largest E8M0 exponent among the block's 32-blocks with
// a nonzero code (1 for an all-zero block), so an element E2M1 * 2^(e - 127) becomes M * 2^E with
// M in {1, 1.5} and E = (its E2M1 exponent) + e - m + 6 <= 8. That value has an E4M3 code exactly when
// E >= -6 (normal) or M * 2^(E + 9) is a whole number (subnormal); every element without one is counted
// in *inexact (the loader then refuses the tensor). Stream layout: codes [tile][64-column item][lane][16 B]
// (lane l: row l % 16, columns 32 f + 8 (l / 16) .. +7 of the item in bytes 8 f .. 8 f + 7), then the
// scales [tile][256-column block][16 rows] bf16.
extern "C" __global__ void mk_reencode_fp8(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales, int64_t rows,
                                           int64_t cols, uint8_t *__restrict__ dst, int64_t row_off, int64_t dst_rows,
                                           uint32_t *inexact) {
  const int64_t KB = cols / 256, total = rows * KB, NI = cols / 64;
  uint16_t *sdst = reinterpret_cast<uint16_t *>(dst + dst_rows * cols);
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = idx / KB, kb = idx - r * KB;
    const uint8_t *cr = codes + r * (cols / 2) + kb * 128;
    const uint8_t *sr = scales + r * (cols / 32) + kb * 8;
    int m = -1;
    for (int j = 0; j < 8; ++j) {  // 32-blocks holding a nonzero code (a code other than +-0)
      bool nz = false;
      for (int b = 0; b < 16; ++b) nz |= (cr[j * 16 + b] & 0x77) != 0;
      if (nz) m = max(m, (int)sr[j]);
    }
    const uint16_t sb = m < 0 ? (uint16_t)0x3F80 : (m > 6 ? (uint16_t)((m - 6) << 7) : (uint16_t)(1u << m));
    const int64_t dr = row_off + r, t = dr / 16, rr = dr % 16;
    sdst[(t * KB + kb) * 16 + rr] = sb;
    uint32_t bad = 0;
    for (int e0 = 0; e0 < 256; e0 += 8) {  // eight consecutive elements: one lane's half of an item
      uint32_t word[2] = {0u, 0u};
      for (int e = 0; e < 8; ++e) {
        const int k = e0 + e, j = k / 32;
        const uint32_t nib = (cr[k / 2] >> ((k & 1) * 4)) & 15u;
        const uint32_t c = nib & 7u;
        uint32_t code = 0;
        if (c != 0) {
          const bool m15 = (c & 1u) && c > 1;                  // magnitudes 1.5, 3, 6: 1.5 * 2^p
          const int p = c == 1 ? -1 : (int)((c - 2) >> 1);     // 0.5 = 2^-1; 1, 1.5: p 0; 2, 3: 1; 4, 6: 2
          const int E = p + (int)sr[j] - m + 6;
          if (E >= -6) {
            code = ((uint32_t)(E + 7) << 3) | (m15 ? 4u : 0u);
          } else if (!m15 && E >= -9) {
            code = 1u << (E + 9);
          } else if (m15 && E >= -8) {
            code = 3u << (E + 8);
          } else {
            ++bad;
          }
        }
        code |= (nib & 8u) << 4;  // sign
        word[e >> 2] |= code << (8 * (e & 3));
      }
      const int64_t kk = kb * 256 + e0;
      const int64_t item = kk / 64;
      const int f = (int)((kk % 64) / 32), kg = (int)((kk % 32) / 8);
      const int lane = (int)rr + 16 * kg;
      *reinterpret_cast<uint2 *>(dst + ((t * NI + item) * 64 + lane) * 16 + 8 * f) = uint2{word[0], word[1]};
    }
    if (bad) atomicAdd(inexact, bad);
  }
}

extern "C" __global__ void mk_store_f32(float *dst, float v) { *dst = v; }

// Per-head transposed repack of the key up-projection W_uk [heads * nope][rank] into the packed matrix
// [heads * rank][nope]: row h * rank + c, column n holds W_uk[h * nope + n][c], so one product with the
// per-head query slice gives q~_h = W_uk,h^T q_nope,h.
extern "C" __global__ void mk_repack_bf16_headT(const uint16_t *__restrict__ src, int64_t heads, int64_t nope, int64_t rank,
                                                uint4 *__restrict__ dst) {
  const int64_t KF = nope / 32, rows = heads * rank;
  const int64_t total = (rows / 16) * KF * 64;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * blockDim.x) {
    const int lane = (int)(idx & 63);
    const int64_t fr = idx >> 6, t = fr / KF, f = fr % KF;
    const int64_t r = t * 16 + (lane & 15), h = r / rank, cc = r % rank;
    const int64_t n0 = f * 32 + 8 * (lane >> 4);
    uint16_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = src[(h * nope + n0 + i) * rank + cc];
    dst[(t * KF + f) * 64 + (lane & 15) + 16 * (lane >> 4)] =
        uint4{(uint32_t)v[0] | ((uint32_t)v[1] << 16), (uint32_t)v[2] | ((uint32_t)v[3] << 16),
              (uint32_t)v[4] | ((uint32_t)v[5] << 16), (uint32_t)v[6] | ((uint32_t)v[7] << 16)};
  }
}
