// One MoE tail for all k rows: the weighted sum of the rows' expert outputs in
// slot order, plus the sigmoid-gated shared expert (Red Lite dev45, "What it
// is": one tail for both rows; Flash-Next plan "5.3 MoE deltas": fixed-width
// weighted expert sums).  Each output is summed by one thread in slot order,
// so a row's result is independent of k.  The sliced form reads the fused
// expert kernel's per-slice partial outputs and adds a slot's slices in slice
// order before weighting it.

#include "common.h"

namespace sdv {

namespace {

struct CombineArgs {
  const float* partial;
  const float* w;
  const float* shared_out;
  const float* shared_logit;
  int k, topk, H;
  float* y;
};

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int r = blockIdx.y;
  const int n4 = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (n4 >= a.H) return;
  const float* pr = a.partial + (size_t)r * a.topk * a.H;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int s = 0; s < a.topk; ++s) {
    const float ws = a.w[r * a.topk + s];
    const float4 p = *reinterpret_cast<const float4*>(pr + (size_t)s * a.H + n4);
    acc.x = fmaf(ws, p.x, acc.x);
    acc.y = fmaf(ws, p.y, acc.y);
    acc.z = fmaf(ws, p.z, acc.z);
    acc.w = fmaf(ws, p.w, acc.w);
  }
  if (a.shared_out) {
    const float gate = a.shared_logit ? sigmoidf_(a.shared_logit[r]) : 1.0f;
    const float4 sh = *reinterpret_cast<const float4*>(a.shared_out + (size_t)r * a.H + n4);
    acc.x = fmaf(gate, sh.x, acc.x);
    acc.y = fmaf(gate, sh.y, acc.y);
    acc.z = fmaf(gate, sh.z, acc.z);
    acc.w = fmaf(gate, sh.w, acc.w);
  }
  *reinterpret_cast<float4*>(a.y + (size_t)r * a.H + n4) = acc;
}

struct SlicedArgs {
  const float* partial;  // [S][k][topk + 1][H]
  const int32_t* idx;    // [k][topk]
  const float* w;        // [k][topk]
  const float* shared_logit;
  int S, k, topk, H, has_shared;
  float* y;
};

// Slot (r, s) contributes w[r][s] * sum_j partial[j][r][s] (slices in order);
// slots without an expert (idx < 0) contribute nothing.  A workgroup takes 64
// output columns of one row in two stages: its four waves first add the
// slices of every slot (wave q takes slots q, q + 4, ...; all of a thread's
// loads are issued before any is added) into LDS, then one wave runs the
// slot-ordered fused multiply-add chain for each column.  The chain is the
// same for every row count, so a row's result does not depend on k.
constexpr int kSlotsMax = SDV_MAX_TOPK + 1;
constexpr int kSlotGroups = 4;
constexpr int kSlotsPerThread = (kSlotsMax + kSlotGroups - 1) / kSlotGroups;

template <int S>
__global__ __launch_bounds__(256) void combine_sliced_kernel(SlicedArgs a) {
  __shared__ float s_p[kSlotsMax][64];
  const int r = blockIdx.y;
  const int col = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int n = min((int)blockIdx.x * 64 + col, a.H - 1);  // columns past H re-read the last one
  const size_t slice_stride = (size_t)a.k * (a.topk + 1) * a.H;
  const float* pr = a.partial + (size_t)r * (a.topk + 1) * a.H + n;
  const int nslots = a.topk + (a.has_shared ? 1 : 0);
  // the row's expert indices and weights (lane c of wave 0 holds slot c),
  // loaded before the partial outputs so that the slot chain below waits on
  // no load of its own
  int slot_idx = -1;
  float slot_w = 0.0f;
  if (q == 0) {
    const int c = min(col, a.topk - 1);
    slot_idx = a.idx[r * a.topk + c];
    slot_w = a.w[r * a.topk + c];
  }
  float v[kSlotsPerThread][S];
#pragma unroll
  for (int c = 0; c < kSlotsPerThread; ++c) {
    const int s = min(q + kSlotGroups * c, nslots - 1);  // past the last slot: a harmless re-read
#pragma unroll
    for (int j = 0; j < S; ++j) v[c][j] = pr[j * slice_stride + (size_t)s * a.H];
  }
  const float zl = a.shared_logit ? a.shared_logit[r] : 0.0f;  // issued after the partial loads
#pragma unroll
  for (int c = 0; c < kSlotsPerThread; ++c) {
    const int s = q + kSlotGroups * c;
    if (s < nslots) {
      float p = v[c][0];
#pragma unroll
      for (int j = 1; j < S; ++j) p = p + v[c][j];
      s_p[s][col] = p;
    }
  }
  __syncthreads();
  if (q != 0) return;
  const float gate = a.shared_logit ? sigmoidf_(zl) : 1.0f;
  float acc = 0.0f;
#pragma unroll
  for (int s = 0; s < kSlotsMax; ++s) {
    if (s < nslots) {
      if (s < a.topk) {
        const int e = __builtin_amdgcn_readlane(slot_idx, s);
        const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(slot_w), s));
        if (e >= 0) acc = fmaf(ws, s_p[s][col], acc);
      } else {
        acc = fmaf(gate, s_p[s][col], acc);
      }
    }
  }
  if ((int)blockIdx.x * 64 + col < a.H) a.y[(size_t)r * a.H + n] = acc;
}

}  // namespace

hipError_t combine_sliced_launch(const float* partial, const int32_t* idx, const float* w,
                                 const float* shared_logit, int S, int k, int topk, int H, int has_shared,
                                 float* y, hipStream_t st) {
  SlicedArgs a{partial, idx, w, shared_logit, S, k, topk, H, has_shared, y};
  const int threads = 256;
  const dim3 grid((H + 63) / 64, k);
  switch (S) {
    case 1: hipLaunchKernelGGL(combine_sliced_kernel<1>, grid, dim3(threads), 0, st, a); break;
    case 2: hipLaunchKernelGGL(combine_sliced_kernel<2>, grid, dim3(threads), 0, st, a); break;
    case 3: hipLaunchKernelGGL(combine_sliced_kernel<3>, grid, dim3(threads), 0, st, a); break;
    case 4: hipLaunchKernelGGL(combine_sliced_kernel<4>, grid, dim3(threads), 0, st, a); break;
    case 5: hipLaunchKernelGGL(combine_sliced_kernel<5>, grid, dim3(threads), 0, st, a); break;
    case 6: hipLaunchKernelGGL(combine_sliced_kernel<6>, grid, dim3(threads), 0, st, a); break;
    case 7: hipLaunchKernelGGL(combine_sliced_kernel<7>, grid, dim3(threads), 0, st, a); break;
    case 8: hipLaunchKernelGGL(combine_sliced_kernel<8>, grid, dim3(threads), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t combine_launch(const float* partial, const float* w, const float* shared_out,
                          const float* shared_logit, int k, int topk, int H, float* y,
                          hipStream_t st) {
  CombineArgs a{partial, w, shared_out, shared_logit, k, topk, H, y};
  const int threads = 256;
  const int blocks = (H / 4 + threads - 1) / threads;
  hipLaunchKernelGGL(combine_kernel, dim3(blocks, k), dim3(threads), 0, st, a);
  return hipGetLastError();
}

}  // namespace sdv
