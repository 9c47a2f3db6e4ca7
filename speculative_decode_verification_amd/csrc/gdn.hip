// k-row Gated DeltaNet verification with in-kernel snapshots (gfx950).
//
// Flash-Next plan, "2.1 Gated DeltaNet": per v head h the fp32 state S_h
// [Dv, Dk] takes, for every row t, decay S <- g S, kv_mem m = S k, delta
// d = beta (v - m), rank-1 update S += d k^T, readout y = S q.  "3.1": g and
// beta are per-head scalars and each qk head serves Hv/Hk consecutive v heads.
// Red Lite dev45, "What it is": row t runs from row t-1's state and the state
// after each row is written to a snapshot from inside the kernel, so a
// rejected draft is undone by selecting a snapshot.
//
// Every value row S_h[i, :] is independent; only t is serial.  A value row
// lives in registers of 16 lanes (one DPP row) for all k rows of the call:
// lane p holds elements 4p + 64j .. +3 (j < Dk/64), so each float4 access of
// the 16 lanes covers 256 contiguous bytes.  Dot products are an in-lane fma
// chain followed by a fixed 16-lane DPP sum, the same instructions for every
// t, so row t of a width-k call equals a width-1 call fed the snapshot after
// row t-1, bit for bit.  HBM traffic per layer: the state once in, k
// snapshots out, plus the small per-row vectors.

#include "common.h"

namespace sdv {

namespace {

struct GdnArgs {
  const float* S_in;
  const float* q;
  const float* kk;
  const float* v;
  const float* g;
  const float* beta;
  int k, Hv, Hk, Dv;
  float* y;
  float* snaps[SDV_MAX_ROWS];
};

constexpr int kRowsPerBlock = 16;  // 16 value rows x 16 lanes = 256 threads

// LDS_KQ: the block's 16 value rows belong to one v head (Dv % 16 == 0), so
// the per-row vectors k_t, q_t (for that head's qk head), v_t, g_t, beta_t of
// all k rows are staged in LDS once and the serial t loop reads only LDS and
// registers.  Otherwise they are read from global memory inside the loop.
template <int DK, bool LDS_KQ>
__global__ __launch_bounds__(256) void gdn_verify_kernel(GdnArgs a) {
  constexpr int NV4 = DK / 64;  // float4 per lane
  __shared__ float4 s_k[LDS_KQ ? SDV_MAX_ROWS * DK / 4 : 1];
  __shared__ float4 s_q[LDS_KQ ? SDV_MAX_ROWS * DK / 4 : 1];
  __shared__ float s_v[LDS_KQ ? SDV_MAX_ROWS * kRowsPerBlock : 1];
  __shared__ float s_g[SDV_MAX_ROWS], s_b[SDV_MAX_ROWS];

  const int sub = threadIdx.x & 15;
  const int lrow = threadIdx.x >> 4;
  const long row = (long)blockIdx.x * kRowsPerBlock + lrow;  // h * Dv + i
  const long nrows = (long)a.Hv * a.Dv;
  const bool active = row < nrows;
  const int h = active ? (int)(row / a.Dv) : 0;
  const int i = active ? (int)(row - (long)h * a.Dv) : 0;
  const int c = h / (a.Hv / a.Hk);

  // Every load is issued before any is used: first the per-row vectors of
  // the staging (at most two float4 of k and of q, one v and one g, beta per
  // thread), then the state.  Loads complete in issue order, so the LDS
  // writes wait only for the staging loads and overlap the state's arrival.
  static_assert(kRowsPerBlock * 16 == 256, "staging assumes 256 threads");
  float4 S[NV4];
  constexpr int KQ_PER_THREAD = (SDV_MAX_ROWS * DK / 4 + 255) / 256;
  float4 ck[KQ_PER_THREAD], cq[KQ_PER_THREAD];
#pragma unroll
  for (int u = 0; u < KQ_PER_THREAD; ++u) ck[u] = cq[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float cv = 0.0f, cg = 0.0f, cb = 0.0f;
  const long row0 = (long)blockIdx.x * kRowsPerBlock;
  const int h0 = (int)(row0 / a.Dv);
  const int i0 = (int)(row0 - (long)h0 * a.Dv);
  const int c0 = h0 / (a.Hv / a.Hk);
  const int n4 = a.k * DK / 4;
  if (LDS_KQ) {
    // every row of the block is in head h0 (and qk head c0).  The loads are
    // unconditional (indices past the data are clamped and the values
    // discarded), so the compiler can count them exactly in its waits.
#pragma unroll
    for (int u = 0; u < KQ_PER_THREAD; ++u) {
      const int t = min((int)threadIdx.x + 256 * u, n4 - 1);
      const int tt = t / (DK / 4), jj = t - tt * (DK / 4);
      ck[u] = reinterpret_cast<const float4*>(a.kk + ((long)tt * a.Hk + c0) * DK)[jj];
      cq[u] = reinterpret_cast<const float4*>(a.q + ((long)tt * a.Hk + c0) * DK)[jj];
    }
    const int tv = min((int)threadIdx.x, a.k * kRowsPerBlock - 1);
    const int tt = tv / kRowsPerBlock, r = min(tv - tt * kRowsPerBlock, (int)(nrows - 1 - row0));
    cv = a.v[((long)tt * a.Hv + h0) * a.Dv + i0 + r];
    const int tg = min((int)threadIdx.x, a.k - 1);
    cg = a.g[tg * a.Hv + h0];
    cb = a.beta[tg * a.Hv + h0];
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the staging loads ahead of the state loads
  {
    const float4* sin4 = reinterpret_cast<const float4*>(a.S_in + (active ? row : nrows - 1) * DK);
#pragma unroll
    for (int j = 0; j < NV4; ++j) S[j] = load_nt(sin4 + sub + 16 * j);  // the state: read once per call
  }
  __builtin_amdgcn_sched_barrier(0);
  if (LDS_KQ) {
#pragma unroll
    for (int u = 0; u < KQ_PER_THREAD; ++u) {
      const int t = threadIdx.x + 256 * u;
      if (t < n4) {
        s_k[t] = ck[u];
        s_q[t] = cq[u];
      }
    }
    if (threadIdx.x < a.k * kRowsPerBlock) s_v[threadIdx.x] = (row0 + threadIdx.x % kRowsPerBlock < nrows) ? cv : 0.0f;
    if (threadIdx.x < a.k) {
      s_g[threadIdx.x] = cg;
      s_b[threadIdx.x] = cb;
    }
    __syncthreads();
  }
  if (!active) return;  // whole 16-lane groups leave together

  for (int t = 0; t < a.k; ++t) {
    float gt, bt, vt;
    float4 kt[NV4], qt[NV4];
    if (LDS_KQ) {
      gt = s_g[t];
      bt = s_b[t];
      vt = s_v[t * kRowsPerBlock + lrow];
#pragma unroll
      for (int j = 0; j < NV4; ++j) {
        kt[j] = s_k[t * (DK / 4) + sub + 16 * j];
        qt[j] = s_q[t * (DK / 4) + sub + 16 * j];
      }
    } else {
      gt = a.g[t * a.Hv + h];
      bt = a.beta[t * a.Hv + h];
      vt = a.v[((long)t * a.Hv + h) * a.Dv + i];
      const float4* k4 = reinterpret_cast<const float4*>(a.kk + ((long)t * a.Hk + c) * DK);
      const float4* q4 = reinterpret_cast<const float4*>(a.q + ((long)t * a.Hk + c) * DK);
#pragma unroll
      for (int j = 0; j < NV4; ++j) {
        kt[j] = k4[sub + 16 * j];
        qt[j] = q4[sub + 16 * j];
      }
    }
    // decay, then kv_mem on the decayed state
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < NV4; ++j) {
      S[j].x = gt * S[j].x;
      S[j].y = gt * S[j].y;
      S[j].z = gt * S[j].z;
      S[j].w = gt * S[j].w;
      m = fmaf(S[j].x, kt[j].x, m);
      m = fmaf(S[j].y, kt[j].y, m);
      m = fmaf(S[j].z, kt[j].z, m);
      m = fmaf(S[j].w, kt[j].w, m);
    }
    m = row16_sum(m);
    const float d = bt * (vt - m);
    // rank-1 update and readout
    float o = 0.0f;
#pragma unroll
    for (int j = 0; j < NV4; ++j) {
      S[j].x = fmaf(d, kt[j].x, S[j].x);
      S[j].y = fmaf(d, kt[j].y, S[j].y);
      S[j].z = fmaf(d, kt[j].z, S[j].z);
      S[j].w = fmaf(d, kt[j].w, S[j].w);
      o = fmaf(S[j].x, qt[j].x, o);
      o = fmaf(S[j].y, qt[j].y, o);
      o = fmaf(S[j].z, qt[j].z, o);
      o = fmaf(S[j].w, qt[j].w, o);
    }
    o = row16_sum(o);
    if (sub == 0) a.y[((long)t * a.Hv + h) * a.Dv + i] = o;
    // snapshots are written once and read back at most once, after the call:
    // streaming (nontemporal) stores keep them from displacing cached data
    f32x4* dst = reinterpret_cast<f32x4*>(a.snaps[t] + row * DK);
#pragma unroll
    for (int j = 0; j < NV4; ++j) __builtin_nontemporal_store(f32x4{S[j].x, S[j].y, S[j].z, S[j].w}, dst + sub + 16 * j);
  }
}

}  // namespace

hipError_t gdn_launch(const float* S_in, const float* q, const float* kk, const float* v,
                      const float* g, const float* beta, int k, int Hv, int Hk, int Dk, int Dv,
                      float* y, float* const* snaps, hipStream_t st) {
  GdnArgs a;
  a.S_in = S_in;
  a.q = q;
  a.kk = kk;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.k = k;
  a.Hv = Hv;
  a.Hk = Hk;
  a.Dv = Dv;
  a.y = y;
  for (int t = 0; t < SDV_MAX_ROWS; ++t) a.snaps[t] = t < k ? snaps[t] : nullptr;
  const long blocks = ((long)Hv * Dv + kRowsPerBlock - 1) / kRowsPerBlock;
  const bool lds = (Dv % kRowsPerBlock) == 0;
  const dim3 grid((unsigned)blocks), block(kRowsPerBlock * 16);
  if (Dk == 64 && lds)
    hipLaunchKernelGGL((gdn_verify_kernel<64, true>), grid, block, 0, st, a);
  else if (Dk == 64)
    hipLaunchKernelGGL((gdn_verify_kernel<64, false>), grid, block, 0, st, a);
  else if (Dk == 128 && lds)
    hipLaunchKernelGGL((gdn_verify_kernel<128, true>), grid, block, 0, st, a);
  else if (Dk == 128)
    hipLaunchKernelGGL((gdn_verify_kernel<128, false>), grid, block, 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sdv
