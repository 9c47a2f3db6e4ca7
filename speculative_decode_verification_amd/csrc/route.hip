// One router dispatch for all k rows: per-row top-k, routing weights, the
// union of the rows' experts and the (expert, row, slot) pair lists
// (Red Lite dev45, "What it is": one router dispatch for both rows and the
// (expert, row) pairs of their union; Flash-Next plan "2.3 MoE").
//
// One workgroup of 16 waves.  Wave w selects the top-k of rows w and w + 16
// on an order word of each fp32 logit (monotone in the value, -0 equal to
// +0, NaN lowest):
// the topk-th largest word T is found bit by bit from the top, each bit one
// round of wave ballots counting the candidates at or above the trial value;
// the candidates above T and the lowest-index ones equal to T are compacted,
// and each takes its slot by counting the selected keys (word, then lower
// index) that beat it.  Selection compares the raw logits, so it is exact and
// independent of how the scores are rounded.
// The union and the pair order come from per-expert row masks, per-expert
// counts and one prefix scan over the experts, all integer and independent
// of thread timing.

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

// Selection key of (value, index): larger value first, then smaller index.
// The high word maps the fp32 value onto an unsigned order (-0 taken as +0,
// so the two zeros tie); the low word is the complement of the index.  NaN
// and empty candidates get key 0, which never wins.
__device__ __forceinline__ uint64_t sel_key(float v, int e) {
  const float c = v + 0.0f;  // -0 + +0 = +0 under round-to-nearest
  const uint32_t b = __float_as_uint(c);
  const uint32_t hi = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  const uint64_t key = ((uint64_t)hi << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
  return (c != c) ? 0ull : key;
}

// The order word alone (0 for NaN, never selected), and its value.
__device__ __forceinline__ uint32_t sel_ord(float v) { return (uint32_t)(sel_key(v, 0) >> 32); }

__device__ __forceinline__ uint64_t key_of(uint32_t ord, int e) {
  return ((uint64_t)ord << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ float ord_value(uint32_t hi) {
  return __uint_as_float((hi & 0x80000000u) ? (hi & 0x7FFFFFFFu) : ~hi);
}

__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t hi = (uint32_t)(key >> 32);
  return __uint_as_float((hi & 0x80000000u) ? (hi & 0x7FFFFFFFu) : ~hi);
}

__device__ __forceinline__ int key_index(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t x) {
  const uint32_t o = __builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, false);
  return o > x ? o : x;
}

// Largest 32-bit value of the wave, in every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = dpp_max_u32<0xB1>(x);
  x = dpp_max_u32<0x4E>(x);
  x = dpp_max_u32<0x124>(x);
  x = dpp_max_u32<0x128>(x);
  uint32_t m = __builtin_amdgcn_readlane((int)x, 0);
  m = max(m, (uint32_t)__builtin_amdgcn_readlane((int)x, 16));
  m = max(m, (uint32_t)__builtin_amdgcn_readlane((int)x, 32));
  m = max(m, (uint32_t)__builtin_amdgcn_readlane((int)x, 48));
  return m;
}

// DPP move with zero fill: lanes whose source is outside the row (or whose
// row is masked off) read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int32_t dpp_or_zero(int32_t x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xF, true);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts by
// 1, 2, 4, 8 within each 16-lane row, then row 0's total into row 1 and row
// 2's into row 3 (row_bcast:15), then rows 0-1's total into rows 2-3
// (row_bcast:31).  Integer adds, so the order does not matter.
__device__ __forceinline__ int32_t wave_incl_scan(int32_t x) {
  x += dpp_or_zero<0x111, 0xF>(x);  // row_shr:1
  x += dpp_or_zero<0x112, 0xF>(x);  // row_shr:2
  x += dpp_or_zero<0x114, 0xF>(x);  // row_shr:4
  x += dpp_or_zero<0x118, 0xF>(x);  // row_shr:8
  x += dpp_or_zero<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_or_zero<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

// Wave r < k selects row r's top-k: each lane holds PL candidates (expert
// lane + 64 j); a round takes the wave's largest key and clears it.
template <int PL>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteArgs a) {
  __shared__ int32_t s_idx[SDV_MAX_ROWS * SDV_MAX_TOPK];
  __shared__ uint32_t s_rowmask[SDV_MAX_EXPERTS];  // rows choosing each expert (bit r)
  __shared__ int32_t s_cnt[SDV_MAX_EXPERTS];
  __shared__ int32_t s_wave[kRouteThreads / 64];
  __shared__ int32_t s_total;
  __shared__ uint64_t s_cand[SDV_MAX_ROWS][SDV_MAX_TOPK];
  __shared__ int32_t s_nsel[SDV_MAX_ROWS];
  __shared__ float s_mx[SDV_MAX_ROWS], s_part[SDV_MAX_ROWS];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int E = a.E, topk = a.topk;

  for (int t = tid; t < SDV_MAX_EXPERTS; t += kRouteThreads) s_rowmask[t] = 0u;
  for (int t = tid; t < SDV_MAX_EXPERTS; t += kRouteThreads) s_cnt[t] = 0;

  for (int r = wave; r < a.k; r += kRouteThreads / 64) {
    const float* l = a.logits + (size_t)r * E;
    float val[PL];
    uint32_t ord[PL];
#pragma unroll
    for (int j = 0; j < PL; ++j) val[j] = l[min(lane + 64 * j, E - 1)];  // unconditional loads
#pragma unroll
    for (int j = 0; j < PL; ++j) ord[j] = lane + 64 * j < E ? sel_ord(val[j]) : 0u;
    // T = the topk-th largest order value: the largest T with at least topk
    // candidates >= T, found bit by bit from the top (counts by ballots)
    // The search stops early once exactly topk candidates are >= the trial
    // value: T is then a lower bound of the topk-th value that selects the
    // same set (every candidate >= T, no tie to break).
    uint32_t T = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < PL; ++j) cnt += __popcll(__ballot(ord[j] >= cand));
      if (cnt >= topk) T = cand;
      if (cnt == topk) break;
    }
    // selected: every candidate above T, then the lowest indices among those
    // equal to T (T = 0 means fewer than topk candidates: take them all)
    int above = 0;
#pragma unroll
    for (int j = 0; j < PL; ++j) above += __popcll(__ballot(ord[j] > T));
    const int need = T > 0 ? topk - above : 0;
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    int eq_before = 0, sel_before = 0;
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      const bool eq = T > 0 && ord[j] == T;
      const uint64_t eqb = __ballot(eq);
      const bool sel = ord[j] > T || (eq && eq_before + __popcll(eqb & lt_mask) < need);
      const uint64_t selb = __ballot(sel);
      if (sel) s_cand[r][sel_before + __popcll(selb & lt_mask)] = key_of(ord[j], lane + 64 * j);
      eq_before += __popcll(eqb);
      sel_before += __popcll(selb);
    }
    if (lane == 0) s_nsel[r] = sel_before;
    // the row's largest logit (softmax shift) and the softmax denominator
    uint32_t omax = 0;
#pragma unroll
    for (int j = 0; j < PL; ++j) omax = max(omax, ord[j]);
    omax = wave_max_u32(omax);
    if (a.mode == SDV_ROUTE_SOFTMAX) {
      const float mx = ord_value(omax);
      float part = 0.0f;
#pragma unroll
      for (int j = 0; j < PL; ++j)
        if (lane + 64 * j < E) part = part + expf(val[j] - mx);
#pragma unroll
      for (int off = 1; off <= 32; off <<= 1) part = part + __shfl_xor(part, off);
      if (lane == 0) {
        s_mx[r] = mx;
        s_part[r] = part;
      }
    }
  }
  __syncthreads();
  for (int r = wave; r < a.k; r += kRouteThreads / 64) {
    // lane c takes the c-th selected candidate (index order) and places it by
    // its rank among the row's selected keys: slot order is larger logit
    // first, ties to the lower index
    const int nsel = s_nsel[r];
    const bool has = lane < nsel;
    int slot = lane;
    uint64_t key = 0;
    if (has) {
      key = s_cand[r][lane];
      // all the row's candidate reads are issued together (at most
      // SDV_MAX_TOPK, the unused ones predicated off)
      int rank = 0;
#pragma unroll
      for (int c = 0; c < SDV_MAX_TOPK; ++c) rank += (c < nsel && s_cand[r][c] > key) ? 1 : 0;
      slot = rank;
    }
    const float v = key_value(key);
    float p;
    if (a.mode == SDV_ROUTE_SOFTMAX) {
      p = expf(v - s_mx[r]) / s_part[r];
    } else {
      p = 1.0f / (1.0f + expf(-v));
    }
    p = has ? p : 0.0f;
    if (a.renorm) {
      // the row's sum in a fixed order: each 16-lane DPP row, then the four
      // row totals in row order (lanes without a candidate add zeros)
      const float part = row16_sum(p);
      const float den = (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(part), 0)) +
                         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(part), 16))) +
                        (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(part), 32)) +
                         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(part), 48)));
      p = p / den;
    }
    if (lane < topk) {
      const int iv = has ? key_index(key) : -1;
      a.w[r * topk + slot] = has ? p : 0.0f;
      a.idx[r * topk + slot] = iv;
      s_idx[r * topk + slot] = iv;
    }
  }
  __syncthreads();

  // ---- union and pairs
  const int total = a.k * topk;
  if (tid < total) {
    const int e = s_idx[tid];
    if (e >= 0 && e < E) {
      atomicOr(&s_rowmask[e], 1u << (tid / topk));
      atomicAdd(&s_cnt[e], 1);
    }
  }
  __syncthreads();
  // exclusive scan over experts of (present << 16 | count): the high half
  // counts the distinct experts below e, the low half the pairs below e
  int32_t packed = 0;
  if (tid < E) packed = (s_cnt[tid] > 0 ? (1 << 16) : 0) | s_cnt[tid];
  const int32_t incl = wave_incl_scan(packed);
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int32_t base = 0;  // totals of the earlier waves (reads issued together)
#pragma unroll
  for (int w2 = 0; w2 < kRouteThreads / 64; ++w2) base += w2 < wave ? s_wave[w2] : 0;
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
      const uint32_t before = s_rowmask[e] & ((1u << r) - 1u);  // earlier rows with expert e
      const int same_before = __popc(before);
      const bool first = before == 0u;
      const int pos = less + same_before;  // pairs ordered by (expert, row)
      a.pair_row[pos] = r;
      a.pair_slot[pos] = s;
      if (first) {
        a.union_ids[distinct_less] = e;
        a.pair_off[distinct_less] = less;
      }
    }
  }
  {
    const int nu = s_total >> 16, npairs = s_total & 0xFFFF;
    if (tid == 0) *a.n_union = nu;
    // entries past n_union are unused; keep them defined (the last union
    // entry's pair range ends at the number of pairs written)
    for (int u = nu + tid; u <= total; u += kRouteThreads) {
      a.pair_off[u] = npairs;
      if (u < total) a.union_ids[u] = -1;
    }
  }
}

}  // namespace

hipError_t route_launch(const float* logits, int k, int E, int topk, int mode, int renorm,
                        int32_t* idx, float* w, int32_t* union_ids, int32_t* n_union,
                        int32_t* pair_off, int32_t* pair_row, int32_t* pair_slot, hipStream_t st) {
  RouteArgs a{logits, k, E, topk, mode, renorm, idx, w, union_ids, n_union, pair_off, pair_row, pair_slot};
  // candidates per lane: the smallest power of two covering E / 64
  const int per_lane = (E + 63) / 64;
  if (per_lane <= 1)
    hipLaunchKernelGGL(route_kernel<1>, dim3(1), dim3(kRouteThreads), 0, st, a);
  else if (per_lane <= 2)
    hipLaunchKernelGGL(route_kernel<2>, dim3(1), dim3(kRouteThreads), 0, st, a);
  else if (per_lane <= 4)
    hipLaunchKernelGGL(route_kernel<4>, dim3(1), dim3(kRouteThreads), 0, st, a);
  else if (per_lane <= 8)
    hipLaunchKernelGGL(route_kernel<8>, dim3(1), dim3(kRouteThreads), 0, st, a);
  else if (per_lane <= kMaxPerLane)
    hipLaunchKernelGGL(route_kernel<kMaxPerLane>, dim3(1), dim3(kRouteThreads), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sdv
