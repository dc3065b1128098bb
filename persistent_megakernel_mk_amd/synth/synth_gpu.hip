// Device-side twin of synth.c: the same counter-based generator (SplitMix64 output function over
// (seed, tensor id, counter), twelve 16-bit uniforms summed into an Irwin-Hall normal deviate), so
// large synthetic workloads are generated in device memory. Input generation only; the values are
// bit-identical to the host generator's (integer arithmetic, then one fp32 multiply and one fp32 add,
// each correctly rounded and never fused, then round-to-nearest-even to bf16).
#include <hip/hip_runtime.h>
#include <stdint.h>

#define SYN_G 0x9E3779B97F4A7C15ULL

__device__ __forceinline__ uint64_t syn_mix(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ULL;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float syn_normal(uint64_t key, uint64_t i, float scale, float mean) {
  int64_t s = 0;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const uint64_t h = syn_mix(key + (3ULL * i + (uint64_t)j + 1ULL) * SYN_G);
    s += (int64_t)(h & 0xffffULL) + (int64_t)((h >> 16) & 0xffffULL) + (int64_t)((h >> 32) & 0xffffULL) +
         (int64_t)(h >> 48);
  }
  const float z = __fmul_rn((float)(int32_t)(s - 393210), scale);
  return __fadd_rn(z, mean);
}

__device__ __forceinline__ uint16_t syn_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// out[i] for i < n: element (offset + i) of the stream; for caches, elements whose position index
// ((offset + i) / inner) % positions >= valid are zero (valid < 0: no masking).
extern "C" __global__ void synth_normal_bf16_kernel(uint64_t key, uint64_t offset, int64_t n, float scale, float mean,
                                                    int64_t inner, int64_t positions, int64_t valid, uint16_t *out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const uint64_t e = offset + (uint64_t)i;
    if (valid >= 0 && (int64_t)((e / (uint64_t)inner) % (uint64_t)positions) >= valid) {
      out[i] = 0;
      continue;
    }
    out[i] = syn_bf16_rne(syn_normal(key, e, scale, mean));
  }
}

extern "C" __global__ void synth_normal_f32_kernel(uint64_t key, uint64_t offset, int64_t n, float scale, float mean,
                                                   float *out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = syn_normal(key, offset + (uint64_t)i, scale, mean);
}

extern "C" int synth_gpu_normal_bf16(uint64_t key, uint64_t offset, int64_t n, float sigma, float mean, int64_t inner,
                                     int64_t positions, int64_t valid, void *out, void *stream) {
  const float scale = sigma / 65536.0f;
  const int blocks = (int)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536);
  if (n <= 0) return 0;
  hipLaunchKernelGGL(synth_normal_bf16_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, key, offset, n, scale,
                     mean, inner > 0 ? inner : 1, positions > 0 ? positions : 1, valid, (uint16_t *)out);
  return (int)hipGetLastError();
}

extern "C" int synth_gpu_normal_f32(uint64_t key, uint64_t offset, int64_t n, float sigma, float mean, void *out,
                                    void *stream) {
  const float scale = sigma / 65536.0f;
  const int blocks = (int)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536);
  if (n <= 0) return 0;
  hipLaunchKernelGGL(synth_normal_f32_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, key, offset, n, scale,
                     mean, (float *)out);
  return (int)hipGetLastError();
}
