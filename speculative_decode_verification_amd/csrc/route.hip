// One router dispatch for all k rows: per-row top-k, routing weights, the
// union of the rows' experts and the (expert, row, slot) pair lists
// (Red Lite dev45, "What it is": one router dispatch for both rows and the
// (expert, row) pairs of their union; Flash-Next plan "2.3 MoE").
//
// One workgroup of 16 waves.  Wave r selects row r's top-k by repeated
// argmax over 64-bit (value, index) keys: each lane takes the largest of its
// own candidates, the 16 lanes of a DPP row reduce with DPP moves, and the
// four row winners are compared in scalar registers; the code has no
// data-dependent branches.  Selection compares the raw fp32 logits (higher
// first, ties to the lower index), so it is exact and independent of how the
// scores are rounded.
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

__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t hi = (uint32_t)(key >> 32);
  return __uint_as_float((hi & 0x80000000u) ? (hi & 0x7FFFFFFFu) : ~hi);
}

__device__ __forceinline__ int key_index(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max(uint64_t k) {
  const uint32_t lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)k, CTRL, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(k >> 32), CTRL, 0xF, 0xF, false);
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > k ? o : k;
}

// Largest key of the wave, in every lane (via scalar registers).
__device__ __forceinline__ uint64_t wave_max(uint64_t k) {
  k = dpp_max<0xB1>(k);   // quad_perm [1,0,3,2]
  k = dpp_max<0x4E>(k);   // quad_perm [2,3,0,1]
  k = dpp_max<0x124>(k);  // row_ror:4
  k = dpp_max<0x128>(k);  // row_ror:8   (every lane now holds its row's largest)
  uint64_t best = 0;
#pragma unroll
  for (int row = 0; row < 4; ++row) {
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)k, 16 * row);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(k >> 32), 16 * row);
    const uint64_t rk = ((uint64_t)hi << 32) | lo;
    best = rk > best ? rk : best;
  }
  return best;
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
  __shared__ uint32_t s_rowbits[SDV_MAX_ROWS][kWords];
  __shared__ int32_t s_cnt[SDV_MAX_EXPERTS];
  __shared__ int32_t s_wave[kRouteThreads / 64];
  __shared__ int32_t s_total;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int E = a.E, topk = a.topk;

  for (int t = tid; t < SDV_MAX_ROWS * kWords; t += kRouteThreads) (&s_rowbits[0][0])[t] = 0u;
  for (int t = tid; t < SDV_MAX_EXPERTS; t += kRouteThreads) s_cnt[t] = 0;

  if (wave < a.k) {
    const int r = wave;
    const float* l = a.logits + (size_t)r * E;
    float val[PL];
    uint64_t key[PL];
#pragma unroll
    for (int j = 0; j < PL; ++j) val[j] = l[min(lane + 64 * j, E - 1)];  // unconditional loads
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      const int e = lane + 64 * j;
      key[j] = e < E ? sel_key(val[j], e) : 0ull;
    }
    uint64_t mine = 0;  // lane s keeps slot s's key
    for (int s = 0; s < topk; ++s) {
      // the lane's largest key by a pairwise tree (depth log2 PL)
      uint64_t t[PL];
#pragma unroll
      for (int j = 0; j < PL; ++j) t[j] = key[j];
#pragma unroll
      for (int w = PL / 2; w >= 1; w >>= 1) {
#pragma unroll
        for (int j = 0; j < w; ++j) t[j] = t[j + w] > t[j] ? t[j + w] : t[j];
      }
      const uint64_t win = wave_max(t[0]);
#pragma unroll
      for (int j = 0; j < PL; ++j) key[j] = key[j] == win ? 0ull : key[j];
      mine = lane == s ? win : mine;
    }
    const bool has = lane < topk && mine != 0ull;
    const float v = key_value(mine);
    // score of this lane's slot
    float p;
    if (a.mode == SDV_ROUTE_SOFTMAX) {
      const float mx = __shfl(v, 0);  // slot 0 holds the row's largest logit
      float part = 0.0f;
#pragma unroll
      for (int j = 0; j < PL; ++j)
        if (lane + 64 * j < E) part = part + expf(val[j] - mx);
#pragma unroll
      for (int off = 1; off <= 32; off <<= 1) part = part + __shfl_xor(part, off);
      p = expf(v - mx) / part;
    } else {
      p = 1.0f / (1.0f + expf(-v));
    }
    p = has ? p : 0.0f;
    if (a.renorm) {
      // fixed butterfly over the slots (lanes past topk add exact zeros)
      float den = p;
#pragma unroll
      for (int off = 1; off <= 32; off <<= 1) den = den + __shfl_xor(den, off);
      p = p / den;
    }
    if (lane < topk) {
      const int iv = has ? key_index(mine) : -1;
      a.w[r * topk + lane] = has ? p : 0.0f;
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
  const int32_t incl = wave_incl_scan(packed);
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
