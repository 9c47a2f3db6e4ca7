// k-row Gated DeltaNet preparation and output norm (gfx950).
//
// Flash-Next plan, "2.1 Gated DeltaNet": before the recurrence, every q, k
// and v channel passes its own short filter along time (current and earlier
// inputs only; the earlier inputs are kept between calls), q and k are
// scaled to unit L2 norm per head, g comes from A_log and dt_bias through
// softplus and exp, and beta = sigmoid(b); after it, y is RMS-normalised and
// multiplied by the weight and act(gate).  "5.1 Gated DeltaNet": 4 taps, sigmoid gate
// for this model.  Red Lite dev45, "What it is", runs these per row pair
// (dn_conv_shift2, dn_qk_l2_2, dn_ba_params2, dn_tail_norm2).
//
// Preparation.  The conv of row t reads inputs only (the history and rows
// 0..t), so all k rows are independent: one workgroup per head block of
// D channels (q heads, then k heads, then v heads), one thread per channel,
// all rows.  A thread loads its channel's 3 + k inputs and 4 taps, applies
// the taps in order (fma chain from the oldest input), and writes the window
// [history; rows] that rollback selects from.  q and k are multiplied per
// (row, head) by rsqrt(sum of squares + eps); the sum is a fixed 16-lane DPP sum,
// the four row totals of a wave in row order, then the waves in order, so
// every row is computed the same way at every width.  The workgroup of v
// head h also forms g and beta of head h for every row (thread t, row t).
//
// Output norm.  One workgroup per (row, v head) of Dv threads: the mean of
// squares in the same fixed order, then y / sqrt(mean + eps) * w * act(z).

#include "gdn_prep_core.h"

namespace sdv {

namespace {

struct PrepArgs {
  const float* qkv;      // [k][C]
  const float* hist;     // [3][C]
  const float* conv_w;   // [C][4]
  const float* a;        // [k][Hv]
  const float* b;        // [k][Hv]
  const float* A_log;    // [Hv]
  const float* dt_bias;  // [Hv]
  int k, Hv, Hk, Dk, Dv, C, conv_act;
  float eps;
  float* q;       // [k][Hk][Dk]
  float* kk;      // [k][Hk][Dk]
  float* v;       // [k][Hv][Dv]
  float* g;       // [k][Hv]
  float* beta;    // [k][Hv]
  float* window;  // [k + 3][C]
};

// Block of D (64 or 128) channels, all k rows (k <= R).
template <int D, int R>
__global__ __launch_bounds__(D) void gdn_prepare_kernel(PrepArgs a) {
  __shared__ float s_part[D / 64][R];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int nq = a.Hk, nqk = 2 * a.Hk;
  const int blk = blockIdx.x;
  const bool is_q = blk < nq, is_k = !is_q && blk < nqk;
  const int hv = max(blk - nqk, 0);
  const int c = is_q ? blk * a.Dk + tid : (is_k ? nq * a.Dk + (blk - nq) * a.Dk + tid
                                                : nqk * a.Dk + hv * a.Dv + tid);
  const int C = a.C, k = a.k;
  // every load first: the channel's history and rows, its taps, and the gate
  // inputs of (row tid, head hv) (clamped; used by the v blocks only)
  float x[kConvWin<R>];
  gdn_conv_load<R>(a.qkv, a.hist, C, c, k, x);
  const float4 w = reinterpret_cast<const float4*>(a.conv_w)[c];
  const int tg = min(tid, k - 1);
  const float ga = a.a[tg * a.Hv + hv], gb = a.b[tg * a.Hv + hv];
  const float al = a.A_log[hv], db = a.dt_bias[hv];
  // the window [history; rows] for rollback by selection
#pragma unroll
  for (int j = 0; j < kConvWin<R>; ++j)
    if (j < kConvHist + k) a.window[(size_t)j * C + c] = x[j];
  float o[R];
  gdn_conv_rows<R>(w, x, a.conv_act, o);
  if (!is_q && !is_k) {
#pragma unroll
    for (int t = 0; t < R; ++t)
      if (t < k) a.v[((size_t)t * a.Hv + hv) * a.Dv + tid] = o[t];
    if (tid < k) {
      a.g[tid * a.Hv + hv] = gdn_decay(ga, al, db);
      a.beta[tid * a.Hv + hv] = gdn_beta(gb);
    }
    return;
  }
  // per-row L2 norm over the head's D channels
  {
    float ws[R];
    gdn_wave_sq_sums<R>(o, ws);
    if ((tid & 63) == 0) {
#pragma unroll
      for (int t = 0; t < R; ++t) s_part[wave][t] = ws[t];
    }
  }
  __syncthreads();
  const int h = is_q ? blk : blk - nq;
  float* dst = is_q ? a.q : a.kk;
#pragma unroll
  for (int t = 0; t < R; ++t) {
    if (t < k) {
      float ss = s_part[0][t];
#pragma unroll
      for (int w2 = 1; w2 < D / 64; ++w2) ss = ss + s_part[w2][t];
      dst[((size_t)t * a.Hk + h) * a.Dk + tid] = o[t] * gdn_inv_norm(ss, a.eps);
    }
  }
}

struct NormArgs {
  const float* y;  // [k][Hv][Dv]
  const float* z;  // [k][Hv][Dv]
  const float* w;  // [Dv]
  int Dv, gate_act;
  float eps;
  float* out;
};

template <int D>
__global__ __launch_bounds__(D) void gdn_gated_norm_kernel(NormArgs a) {
  __shared__ float s_part[D / 64];
  const int tid = threadIdx.x, wave = tid >> 6;
  const size_t base = (size_t)blockIdx.x * D;  // (row, v head)
  const float y = a.y[base + tid];
  const float z = a.z[base + tid];
  const float ws = gdn_wave_sum(y * y);
  if ((tid & 63) == 0) s_part[wave] = ws;
  __syncthreads();
  float ss = s_part[0];
#pragma unroll
  for (int w2 = 1; w2 < D / 64; ++w2) ss = ss + s_part[w2];
  const float n = y / sqrtf(ss / (float)D + a.eps);
  const float gate = a.gate_act == SDV_GATE_SILU ? siluf_(z) : sigmoidf_(z);
  a.out[base + tid] = n * a.w[tid] * gate;
}

}  // namespace

hipError_t gdn_prepare_launch(const float* qkv, const float* hist, const float* conv_w, const float* ga,
                              const float* gb, const float* A_log, const float* dt_bias, int k, int Hv, int Hk,
                              int Dk, int Dv, int conv_act, float eps, float* q, float* kk, float* v, float* g,
                              float* beta, float* window, hipStream_t st) {
  PrepArgs a{qkv, hist, conv_w, ga, gb, A_log, dt_bias, k, Hv, Hk, Dk, Dv, 2 * Hk * Dk + Hv * Dv, conv_act,
             eps, q, kk, v, g, beta, window};
  const dim3 grid((unsigned)(2 * Hk + Hv));
  const bool wide = k > kPassRows;
  if (Dk == 64 && !wide)
    hipLaunchKernelGGL((gdn_prepare_kernel<64, kPassRows>), grid, dim3(64), 0, st, a);
  else if (Dk == 64)
    hipLaunchKernelGGL((gdn_prepare_kernel<64, kWideRows>), grid, dim3(64), 0, st, a);
  else if (Dk == 128 && !wide)
    hipLaunchKernelGGL((gdn_prepare_kernel<128, kPassRows>), grid, dim3(128), 0, st, a);
  else if (Dk == 128)
    hipLaunchKernelGGL((gdn_prepare_kernel<128, kWideRows>), grid, dim3(128), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t gdn_gated_norm_launch(const float* y, const float* z, const float* w, int k, int Hv, int Dv,
                                 int gate_act, float eps, float* out, hipStream_t st) {
  NormArgs a{y, z, w, Dv, gate_act, eps, out};
  const dim3 grid((unsigned)(k * Hv));
  if (Dv == 64)
    hipLaunchKernelGGL(gdn_gated_norm_kernel<64>, grid, dim3(64), 0, st, a);
  else if (Dv == 128)
    hipLaunchKernelGGL(gdn_gated_norm_kernel<128>, grid, dim3(128), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sdv
