// The router dispatch of one workgroup (the body of sdv_moe_route_k): per-row
// top-k, routing weights, the union of the rows' experts and the (expert,
// row, slot) pair lists (Red Lite dev45, "What it is": one router dispatch
// for both rows and the (expert, row) pairs of their union; Flash-Next plan
// "2.3 MoE").
//
// A workgroup of NT threads (NT / 64 waves).  Wave w selects the top-k of
// rows w, w + NT/64, ... on a key of each fp32 logit: an order word
// (monotone in the value, -0 equal to +0, NaN lowest) above the complement
// of the index, so keys are distinct and a larger key is a larger logit or,
// among equal ones, the lower index.  The topk-th largest of the lanes'
// largest words, L, is found bit by bit from the top with one ballot per
// bit; every word of the top k is at least L.  When at most 64 words reach
// L (the usual case) they are compacted and each is ranked against the
// others; the ranks below k are the selection and its slots.  Otherwise
// (many ties at the top) the topk-th largest word T itself is found the same
// way over all words, the words above T and the lowest-index ones equal to T
// are compacted, and each takes its slot by counting the selected keys that
// beat it.
// Selection compares the raw logits, so it is exact and independent of how
// the scores are rounded.  The union and the pair order come from per-expert
// row masks, per-expert counts and one prefix scan over the experts (E <= NT),
// all integer and independent of thread timing.  The outputs may be global
// or LDS arrays; the scratch is LDS.
#pragma once

#include "common.h"

namespace sdv {

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

// LDS scratch of one dispatch: idx [k][topk], rowmask and cnt [E], wave
// totals [NT / 64], the total, candidate keys [k][SDV_MAX_TOPK], selected
// counts, softmax shifts and sums [k], and 64 keys per wave (pool).
struct RouteSmem {
  int32_t* idx;
  uint32_t* rowmask;
  int32_t* cnt;
  int32_t* wave;
  int32_t* total;
  uint64_t* cand;
  int32_t* nsel;
  float* mx;
  float* part;
  uint64_t* pool;  // [NT / 64][64]
};

namespace route_detail {

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

}  // namespace route_detail

template <int PL, int NT>
__device__ __forceinline__ void route_block(const RouteArgs& a, const RouteSmem& sm) {
  using namespace route_detail;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int E = a.E, topk = a.topk;

  for (int t = tid; t < E; t += NT) sm.rowmask[t] = 0u;
  for (int t = tid; t < E; t += NT) sm.cnt[t] = 0;

  for (int r = wave; r < a.k; r += NT / 64) {
    const float* l = a.logits + (size_t)r * E;
    float val[PL];
    uint32_t ord[PL];
#pragma unroll
    for (int j = 0; j < PL; ++j) val[j] = l[min(lane + 64 * j, E - 1)];  // unconditional loads
#pragma unroll
    for (int j = 0; j < PL; ++j) ord[j] = lane + 64 * j < E ? sel_ord(val[j]) : 0u;
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    // L = the topk-th largest of the lanes' largest words (0 when fewer than
    // topk lanes hold a word above 0): at least topk words reach it, so the
    // topk-th largest word of the row is at least L
    uint32_t lmax = ord[0];
#pragma unroll
    for (int j = 1; j < PL; ++j) lmax = max(lmax, ord[j]);
    uint32_t L = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = L | (1u << bit);
      const int cnt = __popcll(__ballot(lmax >= cand));
      if (cnt >= topk) L = cand;
      if (cnt == topk) break;
    }
    const uint32_t lo = L > 1u ? L : 1u;  // word 0 (NaN, padding) is never selected
    int ncand = 0;
#pragma unroll
    for (int j = 0; j < PL; ++j) ncand += __popcll(__ballot(ord[j] >= lo));
    int nsel;
    if (ncand <= 64) {
      // the candidates (every word >= lo) in the wave's pool; each lane ranks
      // one against all: the top k are the ranks below k, in slot order
      uint64_t* pool = sm.pool + wave * 64;
      int before = 0;
#pragma unroll
      for (int j = 0; j < PL; ++j) {
        const bool c = ord[j] >= lo;
        const uint64_t cb = __ballot(c);
        if (c) pool[before + __popcll(cb & lt_mask)] = key_of(ord[j], lane + 64 * j);
        before += __popcll(cb);
      }
      // the pool is written and read by this wave only: its LDS accesses
      // complete in order, the fence keeps the compiler's order
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const uint64_t key = lane < ncand ? pool[lane] : 0ull;
      int rank = 0;
#pragma unroll 4
      for (int c = 0; c < ncand; ++c) rank += pool[c] > key ? 1 : 0;
      if (lane < ncand && rank < topk) sm.cand[(r) * SDV_MAX_TOPK + rank] = key;
      nsel = min(ncand, topk);
      // the pool is rewritten by the wave's next row
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
      // T = the topk-th largest word: the largest T with at least topk
      // words >= T, found bit by bit from the top.  The search stops early
      // once exactly topk words are >= the trial value: T is then a lower
      // bound of the topk-th word that selects the same set (every word >=
      // T, no tie to break).
      uint32_t T = 0;
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = T | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < PL; ++j) cnt += __popcll(__ballot(ord[j] >= cand));
        if (cnt >= topk) T = cand;
        if (cnt == topk) break;
      }
      // selected: every word above T, then the lowest indices among those
      // equal to T
      int above = 0;
#pragma unroll
      for (int j = 0; j < PL; ++j) above += __popcll(__ballot(ord[j] > T));
      const int need = topk - above;
      int eq_before = 0, sel_before = 0;
#pragma unroll
      for (int j = 0; j < PL; ++j) {
        const bool eq = ord[j] == T;
        const uint64_t eqb = __ballot(eq);
        const bool sel = ord[j] > T || (eq && eq_before + __popcll(eqb & lt_mask) < need);
        const uint64_t selb = __ballot(sel);
        if (sel) sm.cand[(r) * SDV_MAX_TOPK + (sel_before + __popcll(selb & lt_mask))] = key_of(ord[j], lane + 64 * j);
        eq_before += __popcll(eqb);
        sel_before += __popcll(selb);
      }
      nsel = sel_before;
    }
    if (lane == 0) sm.nsel[r] = nsel;
    // the row's largest logit (softmax shift) and the softmax denominator
    const uint32_t omax = wave_max_u32(lmax);
    if (a.mode == SDV_ROUTE_SOFTMAX) {
      const float mx = ord_value(omax);
      float part = 0.0f;
#pragma unroll
      for (int j = 0; j < PL; ++j)
        if (lane + 64 * j < E) part = part + expf(val[j] - mx);
#pragma unroll
      for (int off = 1; off <= 32; off <<= 1) part = part + __shfl_xor(part, off);
      if (lane == 0) {
        sm.mx[r] = mx;
        sm.part[r] = part;
      }
    }
  }
  // the slots of row r read only what wave r wrote while selecting (its
  // candidates, count and softmax terms): a wave-level order suffices
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  for (int r = wave; r < a.k; r += NT / 64) {
    // lane c takes the c-th selected candidate (index order) and places it by
    // its rank among the row's selected keys: slot order is larger logit
    // first, ties to the lower index
    const int nsel = sm.nsel[r];
    const bool has = lane < nsel;
    // all SDV_MAX_TOPK entries of the row are read unconditionally, so the
    // reads issue back to back; entries at or past nsel are masked out
    uint64_t ck[SDV_MAX_TOPK];
#pragma unroll
    for (int c = 0; c < SDV_MAX_TOPK; ++c) ck[c] = sm.cand[(r) * SDV_MAX_TOPK + c];
    const uint64_t key = has ? sm.cand[(r) * SDV_MAX_TOPK + min(lane, SDV_MAX_TOPK - 1)] : 0ull;
    int rank = 0;
#pragma unroll
    for (int c = 0; c < SDV_MAX_TOPK; ++c) rank += (c < nsel && ck[c] > key) ? 1 : 0;
    const int slot = has ? rank : lane;
    const float v = key_value(key);
    float p;
    if (a.mode == SDV_ROUTE_SOFTMAX) {
      p = expf(v - sm.mx[r]) / sm.part[r];
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
      sm.idx[r * topk + slot] = iv;
    }
  }
  __syncthreads();

  // ---- union and pairs
  const int total = a.k * topk;
  if (tid < total) {
    const int e = sm.idx[tid];
    if (e >= 0 && e < E) {
      atomicOr(&sm.rowmask[e], 1u << (tid / topk));
      atomicAdd(&sm.cnt[e], 1);
    }
  }
  __syncthreads();
  // exclusive scan over experts of (present << 16 | count): the high half
  // counts the distinct experts below e, the low half the pairs below e
  int32_t packed = 0;
  if (tid < E) packed = (sm.cnt[tid] > 0 ? (1 << 16) : 0) | sm.cnt[tid];
  const int32_t incl = wave_incl_scan(packed);
  if (lane == 63) sm.wave[wave] = incl;
  __syncthreads();
  int32_t base = 0;  // totals of the earlier waves (reads issued together)
#pragma unroll
  for (int w2 = 0; w2 < NT / 64; ++w2) base += w2 < wave ? sm.wave[w2] : 0;
  if (tid == NT - 1) *sm.total = base + incl;
  // thread tid alone read cnt[tid] (its scan input), so it may overwrite it
  if (tid < E) sm.cnt[tid] = base + incl - packed;  // exclusive prefix of expert tid
  __syncthreads();
  if (tid < total) {
    const int r = tid / topk, s = tid - r * topk;
    const int e = sm.idx[tid];
    if (e >= 0 && e < E) {
      const int32_t pre = sm.cnt[e];
      const int less = pre & 0xFFFF, distinct_less = pre >> 16;
      const uint32_t before = sm.rowmask[e] & ((1u << r) - 1u);  // earlier rows with expert e
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
    const int nu = *sm.total >> 16, npairs = *sm.total & 0xFFFF;
    if (tid == 0) *a.n_union = nu;
    // entries past n_union are unused; keep them defined (the last union
    // entry's pair range ends at the number of pairs written)
    for (int u = nu + tid; u <= total; u += NT) {
      a.pair_off[u] = npairs;
      if (u < total) a.union_ids[u] = -1;
    }
  }
}

}  // namespace sdv
