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
