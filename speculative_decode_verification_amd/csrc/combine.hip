// One MoE tail for all k rows: the weighted sum of the rows' expert outputs in
// slot order, plus the sigmoid-gated shared expert (Red Lite dev45, "What it
// is": one tail for both rows; Flash-Next plan "5.3 MoE deltas": fixed-width
// weighted expert sums).  Each output is summed by one thread in slot order,
// so a row's result is independent of k.

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

}  // namespace

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
