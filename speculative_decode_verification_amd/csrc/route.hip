// One router dispatch for all k rows: per-row top-k, routing weights, the
// union of the rows' experts and the (expert, row, slot) pair lists
// (Red Lite dev45, "What it is": one router dispatch for both rows and the
// (expert, row) pairs of their union; Flash-Next plan "2.3 MoE").
//
// One workgroup of 16 waves; wave r handles row r.  Selection compares the raw
// fp32 logits (higher first, ties to the lower index), so it is exact and
// independent of how the scores are later rounded.  Union and pair order are
// computed by counting, one thread per (row, slot) entry, so the result does
// not depend on thread timing.

#include "common.h"

namespace sdv {

namespace {

constexpr int kRouteThreads = 1024;
constexpr int kMaxPerLane = SDV_MAX_EXPERTS / 64;

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

__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteArgs a) {
  __shared__ int32_t s_idx[SDV_MAX_ROWS * SDV_MAX_TOPK];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int E = a.E, topk = a.topk;
  const int per_lane = (E + 63) >> 6;

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
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (better(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      sel_val[s] = bv;
      sel_idx[s] = bi;
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

  // union and pairs: one thread per (row, slot) entry
  const int total = a.k * topk;
  if (tid < total) {
    const int r = tid / topk;
    const int e = s_idx[tid];
    int first = 1, less = 0, distinct_less = 0, same_before = 0;
    for (int t = 0; t < total; ++t) {
      const int et = s_idx[t];
      if (et < e) {
        ++less;
        // et is a first occurrence if no earlier entry has the same id
        int dup = 0;
        for (int u = 0; u < t; ++u) dup |= (s_idx[u] == et);
        distinct_less += !dup;
      } else if (et == e) {
        if (t < tid) first = 0;
        if (t / topk < r) ++same_before;
      }
    }
    const int pos = less + same_before;
    a.pair_row[pos] = r;
    a.pair_slot[pos] = tid - r * topk;
    if (first) {
      a.union_ids[distinct_less] = e;
      a.pair_off[distinct_less] = less;
    }
  }
  if (tid == 0) {
    int nu = 0;
    for (int t = 0; t < total; ++t) {
      int dup = 0;
      for (int u = 0; u < t; ++u) dup |= (s_idx[u] == s_idx[t]);
      nu += !dup;
    }
    *a.n_union = nu;
    a.pair_off[nu] = total;
    // entries past n_union are unused; keep them defined
    for (int u = nu + 1; u <= total; ++u) a.pair_off[u] = total;
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
