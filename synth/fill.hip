// Device fill of the synthetic affine-Q4 weight banks (input generation only).
//
// Implements the counter-based definition in synth/counter.py on the GPU so
// that banks of tens of GB are generated in HBM instead of on the host:
//   rand64(key, ctr) = mix64(key + (ctr + 1) * GAMMA)   (SplitMix64 output)
//   code word w      = 32-bit half (w & 1) of rand64(key, w >> 1)
//   affine bf16 i    = bf16_rne(lo + span * u), u = (rand64(key, i) >> 40) * 2^-24,
//                      evaluated in fp32 as t = span * u, then lo + t.
// Built with -ffp-contract=off so the two fp32 operations round separately,
// as numpy does.  Holds no verification arithmetic.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t rand64(uint64_t key, uint64_t ctr) {
  return mix64(key + (ctr + 1) * kGamma);
}

// Two code words per thread step: one 64-bit draw gives words 2m and 2m+1.
__global__ void fill_codes_kernel(uint32_t* dst, uint64_t key, uint64_t first_word, uint64_t n_words) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words; i += stride) {
    const uint64_t w = first_word + i;
    const uint64_t r = rand64(key, w >> 1);
    dst[i] = (w & 1) ? (uint32_t)(r >> 32) : (uint32_t)(r & 0xFFFFFFFFu);
  }
}

__global__ void fill_affine_kernel(uint16_t* dst, uint64_t key, uint64_t first, uint64_t n,
                                   float lo, float span) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint64_t r = rand64(key, first + i);
    const float u = (float)(uint32_t)(r >> 40) * 5.9604644775390625e-8f;  // 2^-24
    const float t = span * u;
    const float v = lo + t;
    uint32_t b = __float_as_uint(v);
    b += 0x7FFFu + ((b >> 16) & 1u);
    dst[i] = (uint16_t)(b >> 16);
  }
}

unsigned grid_for(uint64_t n) {
  uint64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks == 0) blocks = 1;
  return (unsigned)blocks;
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) int sdvsynth_fill_codes(uint32_t* dst, uint64_t key,
                                                               uint64_t first_word, uint64_t n_words,
                                                               void* stream) {
  if (!dst || n_words == 0) return -1;
  hipLaunchKernelGGL(fill_codes_kernel, dim3(grid_for(n_words)), dim3(256), 0, (hipStream_t)stream, dst,
                     key, first_word, n_words);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

__attribute__((visibility("default"))) int sdvsynth_fill_affine_bf16(uint16_t* dst, uint64_t key,
                                                                     uint64_t first, uint64_t n, float lo,
                                                                     float span, void* stream) {
  if (!dst || n == 0) return -1;
  hipLaunchKernelGGL(fill_affine_kernel, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, dst, key,
                     first, n, lo, span);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
