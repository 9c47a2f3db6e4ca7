// One router dispatch for all k rows: per-row top-k, routing weights, the
// union of the rows' experts and the (expert, row, slot) pair lists
// (Red Lite dev45, "What it is": one router dispatch for both rows and the
// (expert, row) pairs of their union; Flash-Next plan "2.3 MoE").
//
// One workgroup of 16 waves.  Wave r selects row r's top-k by repeated
// argmax: each lane scans its own logits, the 16 lanes of a DPP row reduce
// with DPP moves, and the four row winners are read into scalar registers.
// Selection compares the raw fp32 logits (higher first, ties to the lower
// index), so it is exact and independent of how the scores are rounded.
// The union and the pair order come from per-row expert bitmaps, per-expert
// counts and one prefix scan over the experts, all integer and independent
// of thread timing.

#include "common.h"

namespace sdv {

namespace {

constexpr int kRouteThreads = 1024;
constexpr int kMaxPerLane = SDV_MAX_EXPERTS / 64;
constexpr int kWords = SDV_MAX_EXPERTS / 32;

struct RouteArgs {
  const float* logits;
  int k, E, topk, mode, renorm;
  int32_t* idx;
  float* w;
  int32_t* union_ids;
  int32_t* n_union;
  int32_t* pair_off;
  int32_t* pair_row;
  int32_t* pair_slot;
};

// (value, index) order: larger value first, then smaller index.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return (v > bv) || (v == bv && i < bi);
}

template <int CTRL>
__device__ __forceinline__ void dpp_best(float& bv, int& bi) {
  const float ov = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(bv), CTRL, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_mov_dpp(bi, CTRL, 0xF, 0xF, false);
  if (better(ov, oi, bv, bi)) {
    bv = ov;
    bi = oi;
  }
}

// Best (value, index) of the wave, returned in every lane (scalar registers).
__device__ __forceinline__ void wave_best(float& bv, int& bi) {
  dpp_best<0xB1>(bv, bi);   // quad_perm [1,0,3,2]
  dpp_best<0x4E>(bv, bi);   // quad_perm [2,3,0,1]
  dpp_best<0x124>(bv, bi);  // row_ror:4
  dpp_best<0x128>(bv, bi);  // row_ror:8   (every lane now holds its row's best)
  float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
  int i = __builtin_amdgcn_readlane(bi, 0);
#pragma unroll
  for (int row = 1; row < 4; ++row) {
    const float rv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 16 * row));
    const int ri = __builtin_amdgcn_readlane(bi, 16 * row);
    if (better(rv, ri, v, i)) {
      v = rv;
      i = ri;
    }
  }
  bv = v;
  bi = i;
}

__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteArgs a) {
  __shared__ int32_t s_idx[SDV_MAX_ROWS * SDV_MAX_TOPK];
  __shared__ uint32_t s_rowbits[SDV_MAX_ROWS][kWords];
  __shared__ int32_t s_cnt[SDV_MAX_EXPERTS];
  __shared__ int32_t s_wave[kRouteThreads / 64];
  __shared__ int32_t s_total;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int E = a.E, topk = a.topk;
  const int per_lane = (E + 63) >> 6;

  for (int t = tid; t < SDV_MAX_ROWS * kWords; t += kRouteThreads) (&s_rowbits[0][0])[t] = 0u;
  for (int t = tid; t < SDV_MAX_EXPERTS; t += kRouteThreads) s_cnt[t] = 0;

  if (wave < a.k) {
    const int r = wave;
    const float* l = a.logits + (size_t)r * E;
    float val[kMaxPerLane];
    bool taken[kMaxPerLane];
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
      const int e = lane + 64 * j;
      const bool in = (j < per_lane) && (e < E);
      val[j] = in ? l[e] : 0.0f;
      taken[j] = !in;
    }
    float sel_val[SDV_MAX_TOPK];
    int sel_idx[SDV_MAX_TOPK];
    for (int s = 0; s < topk; ++s) {
      float bv = -__builtin_inff();
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int j = 0; j < kMaxPerLane; ++j) {
        const int e = lane + 64 * j;
        if (!taken[j] && better(val[j], e, bv, bi)) {
          bv = val[j];
          bi = e;
        }
      }
      wave_best(bv, bi);
      sel_val[s] = bv;
      sel_idx[s] = bi < E ? bi : -1;  // no candidate left (only NaN logits remain)
      if ((bi & 63) == lane) {
#pragma unroll
        for (int j = 0; j < kMaxPerLane; ++j)
          if (j == (bi >> 6)) taken[j] = true;
      }
    }
    // scores of the selected slots
    float p[SDV_MAX_TOPK];
    if (a.mode == SDV_ROUTE_SOFTMAX) {
      const float m = sel_val[0];  // the largest logit of the row
      float part = 0.0f;
#pragma unroll
      for (int j = 0; j < kMaxPerLane; ++j) {
        const int e = lane + 64 * j;
        if (j < per_lane && e < E) part = part + expf(val[j] - m);
      }
#pragma unroll
      for (int off = 1; off <= 32; off <<= 1) part = part + __shfl_xor(part, off);
      for (int s = 0; s < topk; ++s) p[s] = expf(sel_val[s] - m) / part;
    } else {
      for (int s = 0; s < topk; ++s) p[s] = 1.0f / (1.0f + expf(-sel_val[s]));
    }
    if (a.renorm) {
      float den = 0.0f;
      for (int s = 0; s < topk; ++s) den = den + p[s];
      for (int s = 0; s < topk; ++s) p[s] = p[s] / den;
    }
    // every lane holds the same scores; lane s writes slot s
    if (lane < topk) {
      float pv = 0.0f;
      int iv = 0;
      for (int s = 0; s < topk; ++s)
        if (s == lane) {
          pv = p[s];
          iv = sel_idx[s];
        }
      a.w[r * topk + lane] = pv;
      a.idx[r * topk + lane] = iv;
      s_idx[r * topk + lane] = iv;
    }
  }
  __syncthreads();

  // ---- union and pairs
  const int total = a.k * topk;
  if (tid < total) {
    const int e = s_idx[tid];
    if (e >= 0 && e < E) {
      atomicOr(&s_rowbits[tid / topk][e >> 5], 1u << (e & 31));
      atomicAdd(&s_cnt[e], 1);
    }
  }
  __syncthreads();
  // exclusive scan over experts of (present << 16 | count): the high half
  // counts the distinct experts below e, the low half the pairs below e
  int32_t packed = 0;
  if (tid < E) packed = (s_cnt[tid] > 0 ? (1 << 16) : 0) | s_cnt[tid];
  int32_t incl = packed;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int32_t base = 0;
  for (int w2 = 0; w2 < wave; ++w2) base += s_wave[w2];
  if (tid == kRouteThreads - 1) s_total = base + incl;
  __syncthreads();
  if (tid < E) s_cnt[tid] = base + incl - packed;  // exclusive prefix of expert tid
  __syncthreads();
  if (tid < total) {
    const int r = tid / topk, s = tid - r * topk;
    const int e = s_idx[tid];
    if (e >= 0 && e < E) {
      const int32_t pre = s_cnt[e];
      const int less = pre & 0xFFFF, distinct_less = pre >> 16;
      int same_before = 0;
      bool first = true;
      for (int r2 = 0; r2 < r; ++r2) {
        const bool has = (s_rowbits[r2][e >> 5] >> (e & 31)) & 1u;
        same_before += has;
        first = first && !has;
      }
      const int pos = less + same_before;  // pairs ordered by (expert, row)
      a.pair_row[pos] = r;
      a.pair_slot[pos] = s;
      if (first) {
        a.union_ids[distinct_less] = e;
        a.pair_off[distinct_less] = less;
      }
    }
  }
  if (tid == 0) {
    const int nu = s_total >> 16, npairs = s_total & 0xFFFF;
    *a.n_union = nu;
    // entries past n_union are unused; keep them defined (the last union
    // entry's pair range ends at the number of pairs written)
    for (int u = nu; u <= total; ++u) a.pair_off[u] = npairs;
    for (int u = nu; u < total; ++u) a.union_ids[u] = -1;
  }
}

}  // namespace

hipError_t route_launch(const float* logits, int k, int E, int topk, int mode, int renorm,
                        int32_t* idx, float* w, int32_t* union_ids, int32_t* n_union,
                        int32_t* pair_off, int32_t* pair_row, int32_t* pair_slot, hipStream_t st) {
  RouteArgs a{logits, k, E, topk, mode, renorm, idx, w, union_ids, n_union, pair_off, pair_row, pair_slot};
  hipLaunchKernelGGL(route_kernel, dim3(1), dim3(kRouteThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace sdv
