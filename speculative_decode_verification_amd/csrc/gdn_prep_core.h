// Per-channel and per-head pieces of the GDN preparation, shared by the
// stand-alone preparation kernel and the recurrence kernel that prepares its
// own inputs, so both compute every value with the same instructions.
//
// Flash-Next plan, "2.1 Gated DeltaNet": a per-channel filter along time over
// the q, k and v channels (current and earlier inputs only, the earlier ones
// carried between calls), q and k scaled to unit L2 norm per head, decay
// gate exp(-exp(A_log) softplus(a + dt_bias)), beta = sigmoid(b); "5.1 Gated
// DeltaNet": 4 taps.
#pragma once

#include "common.h"

namespace sdv {

constexpr int kConvTaps = 4;
constexpr int kConvHist = kConvTaps - 1;
// history plus the rows of one call, for a kernel of row capacity R
template <int R>
constexpr int kConvWin = kConvHist + R;

// Sum over the 64 lanes of a wave, in every lane: a 16-lane DPP sum, then the
// four row totals in row order.
__device__ __forceinline__ float gdn_wave_sum(float x) {
  const float r = row16_sum(x);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 48));
  return (r0 + r1) + (r2 + r3);
}

// log(1 + e^x) = max(x, 0) + log1p(e^-|x|)
__device__ __forceinline__ float gdn_softplus(float x) { return fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x))); }

__device__ __forceinline__ float gdn_decay(float a, float A_log, float dt_bias) {
  return expf(-expf(A_log) * gdn_softplus(a + dt_bias));
}

__device__ __forceinline__ float gdn_beta(float b) { return 1.0f / (1.0f + expf(-b)); }

// Channel c's history (3 inputs) and the inputs of rows 0..k-1 into x, in
// time order; slots past row k-1 repeat row k-1 (loads always issued, values
// unused).
template <int R>
__device__ __forceinline__ void gdn_conv_load(const float* qkv, const float* hist, int C, int c, int k,
                                              float (&x)[kConvWin<R>]) {
#pragma unroll
  for (int j = 0; j < kConvHist; ++j) x[j] = hist[(size_t)j * C + c];
#pragma unroll
  for (int t = 0; t < R; ++t) x[kConvHist + t] = qkv[(size_t)min(t, k - 1) * C + c];
}

// The conv outputs of every row slot t: taps applied oldest input first (tap
// 3 multiplies the current input), then the optional silu.
template <int R>
__device__ __forceinline__ void gdn_conv_rows(const float4 w, const float (&x)[kConvWin<R>], int act,
                                              float (&o)[R]) {
#pragma unroll
  for (int t = 0; t < R; ++t) {
    float acc = w.x * x[t];
    acc = fmaf(w.y, x[t + 1], acc);
    acc = fmaf(w.z, x[t + 2], acc);
    o[t] = fmaf(w.w, x[t + 3], acc);
  }
  if (act == SDV_CONV_SILU) {
#pragma unroll
    for (int t = 0; t < R; ++t) o[t] = siluf_(o[t]);
  }
}

// gdn_wave_sum(o[t] * o[t]) for every row slot, the rows' DPP stages
// interleaved (each row's sum has the same order as gdn_wave_sum).
template <int R>
__device__ __forceinline__ void gdn_wave_sq_sums(const float (&o)[R], float (&s)[R]) {
  float r[R];
#pragma unroll
  for (int t = 0; t < R; ++t) r[t] = o[t] * o[t];
#pragma unroll
  for (int t = 0; t < R; ++t) r[t] = r[t] + dpp_f32<0xB1>(r[t]);
#pragma unroll
  for (int t = 0; t < R; ++t) r[t] = r[t] + dpp_f32<0x4E>(r[t]);
#pragma unroll
  for (int t = 0; t < R; ++t) r[t] = r[t] + dpp_f32<0x128>(r[t]);
#pragma unroll
  for (int t = 0; t < R; ++t) r[t] = r[t] + dpp_f32<0x124>(r[t]);
#pragma unroll
  for (int t = 0; t < R; ++t) {
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r[t]), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r[t]), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r[t]), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r[t]), 48));
    s[t] = (r0 + r1) + (r2 + r3);
  }
}

// The L2 normalisation factor of a head from its sum of squares: one
// reciprocal square root, so a normalised value is o * gdn_inv_norm(ss, eps).
__device__ __forceinline__ float gdn_inv_norm(float ss, float eps) { return rsqrtf(ss + eps); }

}  // namespace sdv
