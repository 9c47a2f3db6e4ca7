// Internal helpers shared by the libsdv kernels and host wrappers (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sdv.h"

namespace sdv {

// Compute units of the current device (host; cached per device).
int device_cus();

// Rows of one pass of the Q4 kernels: a 32-row MFMA operand holds 9
// activation rows (as three bf16 parts each for fp32 activations).  Wider
// calls run a unit or launch per pass of at most kPassRows rows.
constexpr int kPassRows = 9;
// Row capacity of the wide instantiations of the row-indexed kernels.
constexpr int kWideRows = SDV_MAX_ROWS;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming loads for data read once per call (weights, the input state):
// nontemporal, so they do not displace data that is read again.
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
  const u32x4v w = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
  return make_uint4(w.x, w.y, w.z, w.w);
}
__device__ __forceinline__ uint32_t load_nt(const uint32_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ float4 load_nt(const float4* p) {
  const f32x4 w = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(w.x, w.y, w.z, w.w);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return b >> 16;
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }

// x * sigmoid(x), written as x / (1 + exp(-x)).
__device__ __forceinline__ float siluf_(float x) { return x / (1.0f + expf(-x)); }

// DPP lane move within a 16-lane row.  Controls used: quad_perm [1,0,3,2]
// (0xB1), quad_perm [2,3,0,1] (0x4E), row_ror:8 (0x128), row_ror:4 (0x124).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row.  The pairing (xor 1, xor 2, then
// rotations by 8 and 4) leaves the bit-identical total in all 16 lanes,
// because each step adds two values that every lane of the pair sees in the
// same two-operand sum.
__device__ __forceinline__ float row16_sum(float x) {
  x = x + dpp_f32<0xB1>(x);
  x = x + dpp_f32<0x4E>(x);
  x = x + dpp_f32<0x128>(x);
  x = x + dpp_f32<0x124>(x);
  return x;
}

}  // namespace sdv
