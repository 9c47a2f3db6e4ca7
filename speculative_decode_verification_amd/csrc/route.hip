// One router dispatch for all k rows in one workgroup of 16 waves: the
// body is route_block (route_core.h).

#include "route_core.h"

namespace sdv {

namespace {

constexpr int kRouteThreads = 1024;
constexpr int kMaxPerLane = SDV_MAX_EXPERTS / 64;

template <int PL>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteArgs a) {
  __shared__ int32_t s_idx[SDV_MAX_ROWS * SDV_MAX_TOPK];
  __shared__ uint32_t s_rowmask[SDV_MAX_EXPERTS];  // rows choosing each expert (bit r)
  __shared__ int32_t s_cnt[SDV_MAX_EXPERTS];
  __shared__ int32_t s_wave[kRouteThreads / 64];
  __shared__ int32_t s_total;
  __shared__ uint64_t s_cand[SDV_MAX_ROWS * SDV_MAX_TOPK];
  __shared__ int32_t s_nsel[SDV_MAX_ROWS];
  __shared__ float s_mx[SDV_MAX_ROWS], s_part[SDV_MAX_ROWS];
  __shared__ uint64_t s_pool[kRouteThreads];  // 64 keys per wave
  const RouteSmem s{s_idx, s_rowmask, s_cnt, s_wave, &s_total, s_cand, s_nsel, s_mx, s_part, s_pool};
  route_block<PL, kRouteThreads>(a, s);
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
