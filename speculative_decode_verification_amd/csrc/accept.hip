// Acceptance of a verified block on the device: the token sampled from each
// row and the number of leading drafts accepted (Red Lite dev45,
// "Acceptance": draft t stands when it equals the token sampled from row
// t-1's logits, so the output distribution stays that of plain decoding for
// any sampler; dev45b: a draft that matches the end-of-answer token is refused,
// so that token is kept out of the state).
//
// A row's sample is its largest score, ties to the lower index.  Greedy
// scores are the logits; with Gumbel noise g (passed in) a score is
// fp32(fp32(l * inv_temp) + g), each operation rounded.  A score becomes a
// 64-bit key whose high word maps fp32 onto an unsigned order (-0 taken as
// +0; NaN gets key 0 and never wins) and whose low word is the complemented
// index, so the largest key is the sample.
//
// Stage 1, grid (chunks, rows) of 256 threads: each workgroup takes the
// largest key of a 4096-element chunk of one row (16 coalesced loads per
// thread, all issued before any is used) and writes it to the workspace.
// Stage 2, one workgroup of up to 16 waves: wave w reduces the chunk keys of
// rows w, w + 16 to their tokens, then one thread counts the accepted
// drafts.  Integer keys make the result independent of the reduction order.

#include <mutex>

#include "common.h"

namespace sdv {

namespace {

constexpr int kAcceptThreads = 256;
constexpr int kAcceptPerThread = 16;
constexpr int kAcceptChunk = kAcceptThreads * kAcceptPerThread;

struct AcceptArgs {
  const float* logits;  // [k][V]
  const float* noise;   // [k][V] or null
  float inv_temp;
  const int32_t* drafts;  // [k - 1]
  int k, V, eos, chunks;
  int32_t* tokens;    // [k]
  int32_t* accepted;  // [1]
  uint64_t* keys;     // workspace [k][chunks]
};

__device__ __forceinline__ uint64_t score_key(float z, int i) {
  const float c = z + 0.0f;  // -0 + +0 = +0 under round-to-nearest
  const uint32_t b = __float_as_uint(c);
  const uint32_t hi = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (c != c) ? 0ull : (((uint64_t)hi << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)i));
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = __shfl_xor(x, off);
    x = o > x ? o : x;
  }
  return x;
}

__global__ __launch_bounds__(kAcceptThreads) void accept_partial_kernel(AcceptArgs a) {
  __shared__ uint64_t s_best[kAcceptThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.y, c = blockIdx.x;
  const int V = a.V;
  const float* lrow = a.logits + (size_t)r * V;
  const int base = c * kAcceptChunk + tid;
  float z[kAcceptPerThread];
#pragma unroll
  for (int j = 0; j < kAcceptPerThread; ++j) z[j] = lrow[min(base + kAcceptThreads * j, V - 1)];
  if (a.noise) {
    const float* nrow = a.noise + (size_t)r * V;
    float g[kAcceptPerThread];
#pragma unroll
    for (int j = 0; j < kAcceptPerThread; ++j) g[j] = nrow[min(base + kAcceptThreads * j, V - 1)];
#pragma unroll
    for (int j = 0; j < kAcceptPerThread; ++j) z[j] = __fadd_rn(__fmul_rn(z[j], a.inv_temp), g[j]);
  }
  uint64_t best = 0;
#pragma unroll
  for (int j = 0; j < kAcceptPerThread; ++j) {
    const int i = base + kAcceptThreads * j;
    const uint64_t key = i < V ? score_key(z[j], i) : 0ull;
    best = key > best ? key : best;
  }
  best = wave_max_u64(best);
  if (lane == 0) s_best[wave] = best;
  __syncthreads();
  if (tid == 0) {
    uint64_t m = s_best[0];
#pragma unroll
    for (int w = 1; w < kAcceptThreads / 64; ++w) m = s_best[w] > m ? s_best[w] : m;
    a.keys[(size_t)r * a.chunks + c] = m;
  }
}

constexpr int kFinalWaves = 16;

__global__ __launch_bounds__(64 * kFinalWaves) void accept_final_kernel(AcceptArgs a) {
  __shared__ int32_t s_tok[SDV_MAX_ROWS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = blockDim.x >> 6;
  for (int r = wave; r < a.k; r += nw) {
    uint64_t best = 0;
    for (int c = lane; c < a.chunks; c += 64) {
      const uint64_t key = a.keys[(size_t)r * a.chunks + c];
      best = key > best ? key : best;
    }
    best = wave_max_u64(best);
    const int tok = best ? (int)(0xFFFFFFFFu - (uint32_t)best) : -1;
    if (lane == 0) {
      a.tokens[r] = tok;
      s_tok[r] = tok;
    }
  }
  __syncthreads();
  if (tid == 0) {
    int n = 0;
    for (int t = 0; t + 1 < a.k; ++t) {
      const int d = a.drafts[t];
      if (d == s_tok[t] && (a.eos < 0 || d != a.eos)) {
        ++n;
      } else {
        break;
      }
    }
    *a.accepted = n;
  }
}

}  // namespace

// The allocation-free form's workspace: file-scope device memory, one copy
// per GPU the library runs on, held until the process ends.  Host code uses
// only the address hipGetSymbolAddress returns for the device (kept per
// device below), never the array's name.
constexpr size_t kAcceptScratchBytes = size_t(1) << 20;
static __device__ __align__(256) uint64_t scratch[kAcceptScratchBytes / 8];

int accept_chunks(int V) { return (V + kAcceptChunk - 1) / kAcceptChunk; }

size_t accept_workspace_bytes(int k, int V) { return (size_t)k * accept_chunks(V) * 8; }

hipError_t accept_launch(const float* logits, const float* noise, float inv_temp, const int32_t* drafts, int k,
                         int V, int eos, int32_t* tokens, int32_t* accepted, void* workspace, hipStream_t st) {
  AcceptArgs a;
  a.logits = logits;
  a.noise = noise;
  a.inv_temp = inv_temp;
  a.drafts = drafts;
  a.k = k;
  a.V = V;
  a.eos = eos;
  a.chunks = accept_chunks(V);
  a.tokens = tokens;
  a.accepted = accepted;
  a.keys = static_cast<uint64_t*>(workspace);
  hipLaunchKernelGGL(accept_partial_kernel, dim3(a.chunks, k), dim3(kAcceptThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(accept_final_kernel, dim3(1), dim3(64 * (k < kFinalWaves ? k : kFinalWaves)), 0, st, a);
  return hipGetLastError();
}

size_t accept_scratch_bytes() { return kAcceptScratchBytes; }

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The device address of `scratch` on the device that runs `st` (the current
// device for the null stream), looked up once per device with that device
// current.
hipError_t scratch_for(hipStream_t st, void** out) {
  int dev = 0;
  hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

// accept_launch with the per-device scratch array as its workspace: no
// allocation.  The caller has checked accept_workspace_bytes(k, V) against
// accept_scratch_bytes().  Every (row, chunk) key is written by the first
// launch before the second reads it, so nothing needs clearing.
hipError_t accept_noalloc_launch(const float* logits, const float* noise, float inv_temp, const int32_t* drafts,
                                 int k, int V, int eos, int32_t* tokens, int32_t* accepted, hipStream_t st) {
  void* ws = nullptr;
  const hipError_t e = scratch_for(st, &ws);
  if (e != hipSuccess) return e;
  return accept_launch(logits, noise, inv_temp, drafts, k, V, eos, tokens, accepted, ws, st);
}

}  // namespace sdv
