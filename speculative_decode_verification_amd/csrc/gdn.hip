// k-row Gated DeltaNet verification with in-kernel snapshots (gfx950).
//
// Flash-Next plan, "2.1 Gated DeltaNet": per v head h the fp32 state S_h
// [Dv, Dk] takes, for every row t, decay S <- g S, kv_mem m = S k, delta
// d = beta (v - m), rank-1 update S += d k^T, readout y = S q.  "3.1": g and
// beta are per-head scalars and each qk head serves Hv/Hk consecutive v heads.
// Red Lite dev45, "What it is": row t runs from row t-1's state and the state
// after each row is written to a snapshot from inside the kernel; rolling
// back after a rejection is the choice of one snapshot as the live state.
//
// Every value row S_h[i, :] is independent; only t is serial.  A value row
// lives in registers of 16 lanes (one DPP row) for all k rows of the call:
// lane p holds elements 4p + 64j .. +3 (j < Dk/64), so each float4 access of
// the 16 lanes covers 256 contiguous bytes.  Dot products are an in-lane fma
// chain followed by a fixed 16-lane DPP sum, the same instructions for every
// t, so row t of a width-k call equals a width-1 call fed the snapshot after
// row t-1, bit for bit.  HBM traffic per layer: the state once in, k
// snapshots out, plus the small per-row vectors.

#include <utility>

#include "gdn_prep_core.h"

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
  // with the preparation in the kernel: the projections instead of q, kk, v,
  // g, beta, and the conv window out
  const float* qkv;      // [k][C]
  const float* hist;     // [3][C]
  const float* conv_w;   // [C][4]
  const float* ga;       // [k][Hv]
  const float* gb;       // [k][Hv]
  const float* A_log;    // [Hv]
  const float* dt_bias;  // [Hv]
  int C, conv_act;
  float eps;
  float* window;  // [k + 3][C]
  // with the gated output norm in the kernel (NORM)
  const float* nz;  // gate input [k][Hv][Dv]
  const float* nw;  // norm weight [Dv]
  int gate_act;
  float neps;
  float* out;       // [k][Hv][Dv]
  int32_t* cnt;     // [Hv], zero between calls
  // several layers in one launch (LAYERS): layer blockIdx.y's buffers replace
  // S_in, qkv, hist, conv_w, ga, gb, A_log, dt_bias, window, y and snaps
  const sdv_gdn_layer* layers;
};

// Value rows per workgroup (16 lanes each): 16 (256 threads), or 32 (512
// threads) for the one-launch preparation at Dk = 128, where every workgroup
// repeats the conv and norms of its qk head's 2Dk channels: four workgroups
// per head instead of eight halve that repeated work.
constexpr int kRowsPerBlock = 16;
constexpr int kRowsPerBlockPrep = 32;

// f(integral_constant<int, t>) for t = 0, 1, ... while t < k, in order.
template <int... T, class F>
__device__ __forceinline__ void for_rows(std::integer_sequence<int, T...>, int k, F&& f) {
  (void)((T < k ? (f(std::integral_constant<int, T>{}), true) : false) && ...);
}

// LDS_KQ: the block's RB value rows belong to one v head (Dv % RB == 0), so
// the per-row vectors k_t, q_t (for that head's qk head), v_t, g_t, beta_t of
// all k rows are staged in LDS once and the serial t loop reads only LDS and
// registers.  Otherwise they are read from global memory inside the loop.
//
// PREP (Dk = Dv, LDS_KQ): the block prepares its own inputs from the
// projections with the instructions of the stand-alone preparation, so its
// rows equal preparation followed by the recurrence, bit for bit.  Threads
// 0..2Dk-1 take the q then k channels of the block's qk head (conv, per-wave
// sums of squares; the factor rsqrt(sum of the waves in order + eps) is
// applied as row t is read), RB threads the block's RB v channels, k threads
// the gates of its v head; one barrier.  The waves' sums are the same at
// either block size, so every output is too.  The qk columns of the window
// are written by the first block of each qk head, the v columns by their
// block.  Blocks of one qk head are placed on one XCD when the block count
// allows, so its repeated q/k inputs are L2 hits.
//
// NORM (with PREP): the gated output norm of each head is applied by the
// last of the head's Dv / RB workgroups to finish.  Every workgroup stores
// its y rows with agent-scope coherent stores, and every thread issues an
// agent-scope release fence before the workgroup counts itself in on the
// head's counter (an acquire-release add); the workgroup
// that brings the count to Dv / RB resets it to zero, issues an acquire
// fence, reads the head's y rows back (coherent loads) and runs the same arithmetic as
// gdn_gated_norm_kernel, in the same order, so the output equals the
// separate launch's bit for bit.  No workgroup waits for another.
//
// LAYERS (with PREP): blockIdx.y picks one of several independent layers of
// one shape; each runs exactly as its own launch would.
template <int DK, bool LDS_KQ, bool PREP, int R, bool NORM = false, int RB = kRowsPerBlock, bool LAYERS = false>
__global__ __launch_bounds__(RB * 16) void gdn_verify_kernel(GdnArgs a_in) {
  static_assert(!LAYERS || (PREP && !NORM), "the layer form is built for the preparation + recurrence");
  GdnArgs a = a_in;
  if constexpr (LAYERS) {
    const sdv_gdn_layer& l = a_in.layers[blockIdx.y];
    a.S_in = l.S_in;
    a.qkv = l.qkv;
    a.hist = l.hist;
    a.conv_w = l.conv_w;
    a.ga = l.a;
    a.gb = l.b;
    a.A_log = l.A_log;
    a.dt_bias = l.dt_bias;
    a.window = l.window;
    a.y = l.y;
#pragma unroll
    for (int t = 0; t < R; ++t) a.snaps[t] = l.snaps[t];
  }
  static_assert(!PREP || LDS_KQ, "the in-kernel preparation stages through LDS");
  static_assert(!NORM || PREP, "the output norm needs whole heads per workgroup group (Dv = Dk)");
  static_assert(RB == 16 || (RB == 32 && DK == 128 && PREP), "32-row blocks are built for the preparation at Dk = 128");
  constexpr int NT = RB * 16;  // threads: at least 2 DK, one q or k channel each
  if (blockDim.x != NT) return;  // a launch of another block size would index past its rows
  constexpr int NV4 = DK / 64;  // float4 per lane
  __shared__ float4 s_k[LDS_KQ ? R * DK / 4 : 1];
  __shared__ float4 s_q[LDS_KQ ? R * DK / 4 : 1];
  __shared__ float s_v[LDS_KQ ? R * RB : 1];
  __shared__ float s_g[R], s_b[R];
  __shared__ float s_part[PREP ? 4 : 1][R];

  // blocks dealt round-robin over the 8 XCDs; with PREP and a multiple of 8
  // blocks, XCD x takes the consecutive logical blocks x*n/8 .. (x+1)*n/8-1
  int lblk = blockIdx.x;
  if (PREP && (gridDim.x & 7) == 0) lblk = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int sub = threadIdx.x & 15;
  const int lrow = threadIdx.x >> 4;
  // value rows fit in int (Hv * Dv <= 2^26); with PREP, Dv = DK is known
  const int Dv = PREP ? DK : a.Dv;
  const int row = lblk * RB + lrow;  // h * Dv + i
  const int nrows = a.Hv * Dv;
  const bool active = row < nrows;
  const int h = active ? row / Dv : 0;
  const int i = active ? row - h * Dv : 0;
  const int c = h / (a.Hv / a.Hk);

  // Every load is issued before any is used: first the per-row vectors of
  // the staging (KQ_PER_THREAD float4 of k and of q, V_PER_THREAD values of
  // v, one g and beta per thread), then the state.  Loads complete in issue order, so the LDS
  // writes wait only for the staging loads and overlap the state's arrival.
  float4 S[NV4];
  constexpr int KQ_PER_THREAD = (R * DK / 4 + NT - 1) / NT;
  float4 ck[KQ_PER_THREAD], cq[KQ_PER_THREAD];
#pragma unroll
  for (int u = 0; u < KQ_PER_THREAD; ++u) ck[u] = cq[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  constexpr int V_PER_THREAD = (R * RB + NT - 1) / NT;  // v values staged per thread
  float cv[V_PER_THREAD], cg = 0.0f, cb = 0.0f;
#pragma unroll
  for (int u = 0; u < V_PER_THREAD; ++u) cv[u] = 0.0f;
  const int row0 = lblk * RB;
  const int h0 = row0 / Dv;
  const int i0 = row0 - h0 * Dv;
  const int c0 = h0 / (a.Hv / a.Hk);
  const int n4 = a.k * DK / 4;
  // PREP: the inputs of the block's q/k channel (threads 0..2Dk-1), of its v
  // channel (threads VB..VB+RB-1) and of its gates (threads GB..GB+k-1); every
  // thread issues all of them, clamped, so the waits are static
  constexpr int VB = DK == 128 ? 0 : 128, GB = NT - 64;
  static_assert(2 * DK <= NT && GB + SDV_MAX_ROWS <= NT && (DK == 128 || VB + RB <= GB), "preparation thread roles");
  float xq[PREP ? kConvWin<R> : 1], xv[PREP ? kConvWin<R> : 1];
  float4 wq = make_float4(0.0f, 0.0f, 0.0f, 0.0f), wv = wq;
  float pa = 0.0f, pb = 0.0f, pal = 0.0f, pdb = 0.0f;
  const int ratio = a.Hv / a.Hk;
  const int cq_ch = min((int)threadIdx.x, 2 * DK - 1);
  const int c_qk = cq_ch < DK ? c0 * DK + cq_ch : (a.Hk + c0) * DK + cq_ch - DK;
  const int rv = min(max((int)threadIdx.x - VB, 0), RB - 1);
  const int c_v = 2 * a.Hk * DK + h0 * DK + i0 + rv;
  if constexpr (PREP) {
    // gate inputs first: their wave forms the gates while the rest arrives
    const int tg = min(max((int)threadIdx.x - GB, 0), a.k - 1);
    pa = a.ga[tg * a.Hv + h0];
    pb = a.gb[tg * a.Hv + h0];
    pal = a.A_log[h0];
    pdb = a.dt_bias[h0];
    __builtin_amdgcn_sched_barrier(0);
    gdn_conv_load<R>(a.qkv, a.hist, a.C, c_qk, a.k, xq);
    gdn_conv_load<R>(a.qkv, a.hist, a.C, c_v, a.k, xv);
    wq = reinterpret_cast<const float4*>(a.conv_w)[c_qk];
    wv = reinterpret_cast<const float4*>(a.conv_w)[c_v];
  }
  if (LDS_KQ && !PREP) {
    // every row of the block is in head h0 (and qk head c0).  The loads are
    // unconditional (indices past the data are clamped and the values
    // discarded), so the compiler can count them exactly in its waits.
#pragma unroll
    for (int u = 0; u < KQ_PER_THREAD; ++u) {
      const int t = min((int)threadIdx.x + NT * u, n4 - 1);
      const int tt = t / (DK / 4), jj = t - tt * (DK / 4);
      ck[u] = reinterpret_cast<const float4*>(a.kk + ((long)tt * a.Hk + c0) * DK)[jj];
      cq[u] = reinterpret_cast<const float4*>(a.q + ((long)tt * a.Hk + c0) * DK)[jj];
    }
#pragma unroll
    for (int u = 0; u < V_PER_THREAD; ++u) {
      const int tv = min((int)threadIdx.x + NT * u, a.k * RB - 1);
      const int tt = tv / RB, r = min(tv - tt * RB, (int)(nrows - 1 - row0));
      cv[u] = a.v[((long)tt * a.Hv + h0) * Dv + i0 + r];
    }
    const int tg = min((int)threadIdx.x, a.k - 1);
    cg = a.g[tg * a.Hv + h0];
    cb = a.beta[tg * a.Hv + h0];
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the staging loads ahead of the state loads
  {
    const float4* sin4 = reinterpret_cast<const float4*>(a.S_in + (size_t)(active ? row : nrows - 1) * DK);
#pragma unroll
    for (int j = 0; j < NV4; ++j) S[j] = load_nt(sin4 + sub + 16 * j);  // the state: read once per call
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (PREP) {
    // conv of the q/k channel and the per-wave sums of squares; the conv
    // outputs go to LDS unnormalised, each row's factor is applied as it is
    // read in the row loop
    const int tid = threadIdx.x, wave = tid >> 6, k = a.k;
    if (tid >= GB && tid < GB + k) {
      s_g[tid - GB] = gdn_decay(pa, pal, pdb);
      s_b[tid - GB] = gdn_beta(pb);
    }
    float o[R];
    gdn_conv_rows<R>(wq, xq, a.conv_act, o);
    if (tid < 2 * DK) {  // whole waves: q, then k
      float ws[R];
      gdn_wave_sq_sums<R>(o, ws);
      if ((tid & 63) == 0) {
#pragma unroll
        for (int t = 0; t < R; ++t) s_part[wave][t] = ws[t];
      }
      float* dst = reinterpret_cast<float*>(tid < DK ? s_q : s_k);
      const int ch = tid < DK ? tid : tid - DK;
#pragma unroll
      for (int t = 0; t < R; ++t)
        if (t < k) dst[t * DK + ch] = o[t];
    }
    if (tid >= VB && tid < VB + RB) {
      float ov[R];
      gdn_conv_rows<R>(wv, xv, a.conv_act, ov);
#pragma unroll
      for (int t = 0; t < R; ++t)
        if (t < k) s_v[t * RB + rv] = ov[t];
    }
    __syncthreads();
  } else if (LDS_KQ) {
#pragma unroll
    for (int u = 0; u < KQ_PER_THREAD; ++u) {
      const int t = threadIdx.x + NT * u;
      if (t < n4) {
        s_k[t] = ck[u];
        s_q[t] = cq[u];
      }
    }
#pragma unroll
    for (int u = 0; u < V_PER_THREAD; ++u) {
      const int tv = threadIdx.x + NT * u;
      if (tv < a.k * RB) s_v[tv] = (row0 + tv % RB < nrows) ? cv[u] : 0.0f;
    }
    if (threadIdx.x < a.k) {
      s_g[threadIdx.x] = cg;
      s_b[threadIdx.x] = cb;
    }
    __syncthreads();
  }
  if (!active) return;  // whole 16-lane groups leave together

  // PREP: the window [history; rows] of the block's channels, stored once
  // the state has arrived (stores issued earlier would be counted in the
  // waits for it): the v columns by their block, the q/k columns by the first
  // block of the qk head
  auto window_out = [&]() {
    const int tid = threadIdx.x, k = a.k;
    if (tid >= VB && tid < VB + RB) {
#pragma unroll
      for (int j = 0; j < kConvWin<R>; ++j)
        if (j < kConvHist + k) a.window[(size_t)j * a.C + c_v] = xv[j];
    }
    if (tid < 2 * DK && h0 % ratio == 0 && i0 == 0) {
#pragma unroll
      for (int j = 0; j < kConvWin<R>; ++j)
        if (j < kConvHist + k) a.window[(size_t)j * a.C + c_qk] = xq[j];
    }
  };
  // one row of the recurrence; the rows are expanded with t a constant, so
  // the LDS reads of a row, which need nothing of the previous row, can be
  // issued ahead of it
  auto row_step = [&](auto tc) __attribute__((always_inline)) {
    constexpr int t = decltype(tc)::value;
    {
      float gt, bt, vt;
      float4 kt[NV4], qt[NV4];
      if (LDS_KQ) {
        gt = s_g[t];
        bt = s_b[t];
        vt = s_v[t * RB + lrow];
  #pragma unroll
        for (int j = 0; j < NV4; ++j) {
          kt[j] = s_k[t * (DK / 4) + sub + 16 * j];
          qt[j] = s_q[t * (DK / 4) + sub + 16 * j];
        }
        if constexpr (PREP) {
          // the L2 norm of row t: the q waves' sums in wave order, then the k waves'
          float sq = s_part[0][t], sk = s_part[DK / 64][t];
  #pragma unroll
          for (int w2 = 1; w2 < DK / 64; ++w2) {
            sq = sq + s_part[w2][t];
            sk = sk + s_part[DK / 64 + w2][t];
          }
          const float iq = gdn_inv_norm(sq, a.eps), ik = gdn_inv_norm(sk, a.eps);
  #pragma unroll
          for (int j = 0; j < NV4; ++j) {
            kt[j].x = kt[j].x * ik;
            kt[j].y = kt[j].y * ik;
            kt[j].z = kt[j].z * ik;
            kt[j].w = kt[j].w * ik;
            qt[j].x = qt[j].x * iq;
            qt[j].y = qt[j].y * iq;
            qt[j].z = qt[j].z * iq;
            qt[j].w = qt[j].w * iq;
          }
        }
      } else {
        gt = a.g[t * a.Hv + h];
        bt = a.beta[t * a.Hv + h];
        vt = a.v[((long)t * a.Hv + h) * Dv + i];
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
      if (sub == 0) {
        if constexpr (NORM)
          __hip_atomic_store(a.y + ((long)t * a.Hv + h) * Dv + i, o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          a.y[((long)t * a.Hv + h) * Dv + i] = o;
      }
      // snapshots are written once and read back at most once, after the call:
      // streaming (nontemporal) stores keep them from displacing cached data
      f32x4* dst = reinterpret_cast<f32x4*>(a.snaps[t] + (size_t)row * DK);
  #pragma unroll
      for (int j = 0; j < NV4; ++j) __builtin_nontemporal_store(f32x4{S[j].x, S[j].y, S[j].z, S[j].w}, dst + sub + 16 * j);
      if constexpr (PREP) {
        if (t == 0) window_out();
      }
    }
  };
  for_rows(std::make_integer_sequence<int, R>{}, a.k, row_step);

  if constexpr (NORM) {
    __shared__ int s_last;
    __shared__ float s_np[NT / 64];
    // Release: every thread's y stores are visible at agent scope before its
    // workgroup counts itself in; the counter update is acquire-release, and
    // the last workgroup acquires before it reads the other workgroups' y.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (threadIdx.x == 0) {
      const int n = __hip_atomic_fetch_add(a.cnt + h0, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      const int last = n == DK / RB - 1;
      if (last) __hip_atomic_store(a.cnt + h0, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = last;
    }
    __syncthreads();
    if (s_last) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      // NT / DK rows of the head at a time, DK threads per row; wave w of
      // a row sums the squares of elements 64 w .. 64 w + 63
      constexpr int kRowsAtOnce = NT / DK, kWavesPerRow = DK / 64;
      const int d = threadIdx.x % DK, rsub = threadIdx.x / DK, wave = threadIdx.x >> 6;
      const float wd = a.nw[d];
      for (int t0 = 0; t0 < a.k; t0 += kRowsAtOnce) {
        const int t = min(t0 + rsub, a.k - 1);
        const size_t base = ((size_t)t * a.Hv + h0) * DK;
        const float yv = __hip_atomic_load(a.y + base + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float z = a.nz[base + d];
        const float ws = gdn_wave_sum(yv * yv);
        if ((threadIdx.x & 63) == 0) s_np[wave] = ws;
        __syncthreads();
        float ss = s_np[rsub * kWavesPerRow];
#pragma unroll
        for (int w2 = 1; w2 < kWavesPerRow; ++w2) ss = ss + s_np[rsub * kWavesPerRow + w2];
        const float nv = yv / sqrtf(ss / (float)DK + a.neps);
        const float gate = a.gate_act == SDV_GATE_SILU ? siluf_(z) : sigmoidf_(z);
        if (t0 + rsub < a.k) a.out[base + d] = nv * wd * gate;
        __syncthreads();  // s_np is rewritten by the next rows
      }
    }
  }
}

}  // namespace

hipError_t gdn_launch(const float* S_in, const float* q, const float* kk, const float* v,
                      const float* g, const float* beta, int k, int Hv, int Hk, int Dk, int Dv,
                      float* y, float* const* snaps, hipStream_t st) {
  GdnArgs a{};
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
  if (Dk != 64 && Dk != 128) return hipErrorInvalidValue;
  const bool wide = k > kPassRows;
  auto kern = Dk == 64 ? (lds ? (wide ? gdn_verify_kernel<64, true, false, kWideRows>
                                      : gdn_verify_kernel<64, true, false, kPassRows>)
                              : (wide ? gdn_verify_kernel<64, false, false, kWideRows>
                                      : gdn_verify_kernel<64, false, false, kPassRows>))
                       : (lds ? (wide ? gdn_verify_kernel<128, true, false, kWideRows>
                                      : gdn_verify_kernel<128, true, false, kPassRows>)
                              : (wide ? gdn_verify_kernel<128, false, false, kWideRows>
                                      : gdn_verify_kernel<128, false, false, kPassRows>));
  hipLaunchKernelGGL(kern, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t gdn_verify_prep_launch(const float* S_in, const float* qkv, const float* hist, const float* conv_w,
                                  const float* ga, const float* gb, const float* A_log, const float* dt_bias, int k,
                                  int Hv, int Hk, int D, int conv_act, float eps, float* window, float* y,
                                  float* const* snaps, hipStream_t st, const float* nz, const float* nw,
                                  int gate_act, float neps, float* out, int32_t* cnt) {
  GdnArgs a{};
  a.nz = nz;
  a.nw = nw;
  a.gate_act = gate_act;
  a.neps = neps;
  a.out = out;
  a.cnt = cnt;
  a.S_in = S_in;
  a.k = k;
  a.Hv = Hv;
  a.Hk = Hk;
  a.Dv = D;
  a.y = y;
  for (int t = 0; t < SDV_MAX_ROWS; ++t) a.snaps[t] = t < k ? snaps[t] : nullptr;
  a.qkv = qkv;
  a.hist = hist;
  a.conv_w = conv_w;
  a.ga = ga;
  a.gb = gb;
  a.A_log = A_log;
  a.dt_bias = dt_bias;
  a.C = 2 * Hk * D + Hv * D;
  a.conv_act = conv_act;
  a.eps = eps;
  a.window = window;
  if (D != 64 && D != 128) return hipErrorInvalidValue;
  const bool wide = k > kPassRows;
  // 32-row blocks for Dk = 128; 16-row blocks otherwise
  const int rb = D == 128 ? kRowsPerBlockPrep : kRowsPerBlock;
  const dim3 grid((unsigned)((long)Hv * D / rb)), block(rb * 16);
  auto kern = D == 64 ? (wide ? gdn_verify_kernel<64, true, true, kWideRows> : gdn_verify_kernel<64, true, true, kPassRows>)
                      : (wide ? gdn_verify_kernel<128, true, true, kWideRows, false, kRowsPerBlockPrep>
                              : gdn_verify_kernel<128, true, true, kPassRows, false, kRowsPerBlockPrep>);
  if (out)
    kern = D == 64 ? (wide ? gdn_verify_kernel<64, true, true, kWideRows, true>
                           : gdn_verify_kernel<64, true, true, kPassRows, true>)
                   : (wide ? gdn_verify_kernel<128, true, true, kWideRows, true, kRowsPerBlockPrep>
                           : gdn_verify_kernel<128, true, true, kPassRows, true, kRowsPerBlockPrep>);
  hipLaunchKernelGGL(kern, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t gdn_verify_prep_layers_launch(const sdv_gdn_layer* table, int L, int k, int Hv, int Hk, int D,
                                         int conv_act, float eps, hipStream_t st) {
  GdnArgs a{};
  a.layers = table;
  a.k = k;
  a.Hv = Hv;
  a.Hk = Hk;
  a.Dv = D;
  a.C = 2 * Hk * D + Hv * D;
  a.conv_act = conv_act;
  a.eps = eps;
  if (D != 64 && D != 128) return hipErrorInvalidValue;
  const bool wide = k > kPassRows;
  const int rb = D == 128 ? kRowsPerBlockPrep : kRowsPerBlock;
  const dim3 grid((unsigned)((long)Hv * D / rb), (unsigned)L), block(rb * 16);
  auto kern = D == 64 ? (wide ? gdn_verify_kernel<64, true, true, kWideRows, false, kRowsPerBlock, true>
                              : gdn_verify_kernel<64, true, true, kPassRows, false, kRowsPerBlock, true>)
                      : (wide ? gdn_verify_kernel<128, true, true, kWideRows, false, kRowsPerBlockPrep, true>
                              : gdn_verify_kernel<128, true, true, kPassRows, false, kRowsPerBlockPrep, true>);
  hipLaunchKernelGGL(kern, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace sdv
