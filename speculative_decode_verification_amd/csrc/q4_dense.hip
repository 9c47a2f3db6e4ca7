// Dense multi-row affine-Q4 (group 64) product for gfx950: one workgroup per
// 32-column weight tile, the tile's K range split over up to 16 waves.
//
// Each packed weight is read from HBM once and decoded once for all k rows
// (mere.run transfer report, "Exact verification kernels and benchmark
// admission": the few-row Q4 projection checked bit for bit against one-row
// products at widths 4, 8 and 9; Red Lite dev45, "What it is": one decode of
// the weights serves every row, and each row keeps the summation order of
// the one-row kernel).
//
// A dense projection has few tiles (160 for 5120 outputs) and a long K, so
// the time of one launch is a latency chain: load, stage, the tile's group
// steps, the cross-wave sum, the store.  The chain is kept short:
//   * wave w owns groups [G w / nw, G (w + 1) / nw) of the tile and stages
//     only that slice of the activation rows, in its own LDS region, so the
//     staging needs no workgroup barrier;
//   * the slice's loads go out first, then the wave's weight blocks (up to 8
//     in flight); loads complete in issue order, so staging never waits for
//     the weights, and each group step waits only for its own block;
//   * with 16 waves a wave takes 5 groups at K = 5120.
// The waves' partial sums meet in LDS and are added in wave order.  nw
// depends on K only, so every row is computed in the same order at every
// width: a width-k row equals the width-1 row bit for bit.
//
// A launch over several weights that share the rows (sdv_qmv_k_multi) has
// T x nmulti (tile, weight) items; when they outnumber the compute units, one
// workgroup per compute unit takes an equal share of them: the rows are
// staged once per workgroup, each wave streams its K range of every item in
// turn through the same ring, and each item's sums are taken in a table
// beside the staging as its last group completes.
//
// The arithmetic of a group step is the one of the other Q4 kernels: codes
// decode exactly to bf16 128 + q, the matrix core returns P = sum (128 + q) x
// and the group adds s P + (b - 128 s) X, X being the group sum of the
// activation row (fp32 activations as three exact bf16 parts).

#include <atomic>

#include "q4_core.h"

namespace sdv {

// Compute units of the current device (cached per device).
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

namespace {

using namespace q4;

constexpr int kDenseMaxWaves = 16;
constexpr size_t kDenseMaxLds = 160 * 1024;  // LDS of one gfx950 workgroup
constexpr int kDenseMulti = 16;  // weights of one multi-weight launch

struct DenseArgs {
  // weight blockIdx.y of the launch (one for sdv_qmv_k)
  const uint4* codes[kDenseMulti];  // tiled: [T][G][64] uint4
  const uint32_t* sb[kDenseMulti];  // tiled: [T][G][32]
  float* out[kDenseMulti];          // [k][n_out]
  const void* act;       // [k][K] bf16 bits or fp32, shared by the weights
  int N, K, T, G, k, n_out, nw;
  int nmulti, mw;        // weights of the launch; items per workgroup (at most; > 1: the several-item form)
  int items;             // T * nmulti: item i is tile i % T of weight i / T
  int gwmax;             // groups of the widest wave range
  int cap;               // staged rows per wave (k or 3k); row cap is all zero
  int region;            // bytes of one wave's LDS region
};

__host__ __device__ inline int dense_row_stride(int gwmax) { return gwmax * 64 + 8; }

// One wave's region: (cap + 1) staged rows of the wave's K slice, then the
// rows' activation sums [kPassRows + 1][gwmax][spg] (row k all zero; spg = 1
// sum per group for Q4, 2 per group (one per 32-element block) for Q8_0).
__host__ __device__ inline size_t dense_region_bytes(int cap, int gwmax, int spg) {
  return ((size_t)(cap + 1) * dense_row_stride(gwmax) * 2 + (size_t)(kPassRows + 1) * gwmax * spg * 4 + 15) &
         ~(size_t)15;
}

// The cross-wave sums [nw][kPassRows][33] reuse the regions when a workgroup
// takes one weight, and follow them when it takes several (the staged rows
// serve every weight).
__host__ __device__ inline size_t dense_red_bytes(int nw) { return (size_t)nw * kPassRows * 33 * 4; }

// Sum of 8 consecutive bf16 values (natural order), and their NU packing.
__device__ __forceinline__ float block8(const uint4 v, uint4& packed) {
  const uint32_t e8[8] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16,
                          v.z & 0xFFFFu, v.z >> 16, v.w & 0xFFFFu, v.w >> 16};
  float acc = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c) acc = acc + bf16_bits_to_f32(e8[c]);
  packed = nu_pack(e8);
  return acc;
}

// Pairwise totals of a group's 8 block sums: the first four (elements
// 0-31), the last four, and the whole group.
__device__ __forceinline__ float half_total(const float (&b)[8], int h) {
  return (b[4 * h] + b[4 * h + 1]) + (b[4 * h + 2] + b[4 * h + 3]);
}
__device__ __forceinline__ float group_total(const float (&b)[8]) { return half_total(b, 0) + half_total(b, 1); }

// FMT = SDV_FMT_Q8_0: two 1 KB code chunks per group step, activation sums
// per 32-element block, and the Q8_0 group step.
template <int FMT, int MODE, int ACT, int PF, bool MW>
__global__ __launch_bounds__(1024, 1) void q4_dense_k_kernel(DenseArgs a) {
  constexpr bool Q8 = FMT == SDV_FMT_Q8_0;
  constexpr int SPG = Q8 ? 2 : 1;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int t = blockIdx.x;
  const int G = a.G, K = a.K, k = a.k, nw = a.nw;
  const int gb = __builtin_amdgcn_readfirstlane((G * wave) / nw);
  const int gw = __builtin_amdgcn_readfirstlane((G * (wave + 1)) / nw - gb);  // >= 1: nw <= G
  const int rs = dense_row_stride(a.gwmax);
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem + (size_t)wave * a.region);
  float* xsum = reinterpret_cast<float*>(smem + (size_t)wave * a.region + (size_t)(a.cap + 1) * rs * 2);

  // ---- activation slice: lane task = (row i, group g of the wave's range);
  // the first task's loads go out before anything else
  const int ntask = k * gw;
  uint4 xv[8];  // a bf16 task, or the first half of an fp32 task
  auto task_src = [&](int task) {
    const int i = task / gw, g = task - i * gw;
    const size_t e0 = (size_t)i * K + (size_t)(gb + g) * 64;  // first element
    return e0;
  };
  {
    const size_t e0 = task_src(min(lane, ntask - 1));
#pragma unroll
    for (int q = 0; q < 8; ++q)
      xv[q] = ACT == SDV_ACT_BF16 ? reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.act) + e0)[q]
                                  : reinterpret_cast<const uint4*>(static_cast<const float*>(a.act) + e0)[q];
  }

  // ---- the wave's weight blocks.  One item: tile t (blockIdx.x) of weight
  // blockIdx.y.  MW: the workgroup's items it0 .. it0 + nm - 1 of the (tile,
  // weight) space, an equal share for every workgroup, one after the other;
  // step s reads block gb + s % gw of item it0 + s / gw (steps past the end
  // re-read the last block)
  const int it0 = MW ? (int)(((long)blockIdx.x * a.items) / gridDim.x) : 0;
  const int nm = MW ? (int)(((long)(blockIdx.x + 1) * a.items) / gridDim.x) - it0 : 1;
  const int ns = nm * gw;
  // the tile and weight of item mi of the workgroup
  auto item_tile = [&](int mi) { return MW ? __builtin_amdgcn_readfirstlane((it0 + mi) % a.T) : t; };
  auto item_weight = [&](int mi) { return MW ? __builtin_amdgcn_readfirstlane((it0 + mi) / a.T) : (int)blockIdx.y; };
  uint4 cbuf[PF], cbuf2[Q8 ? PF : 1];
  uint32_t sbuf[PF];
  // MW: the loads walk the steps in order, so a cursor (step, group in the
  // item, the item's tile and weight) advances by one step per load, by
  // selects, and stops at the last step: no step divides.
  int ls = 0, lg = 0, lt = item_tile(0), lw = item_weight(0);
  auto issue = [&](int slot, int s) {
    const uint4* codes;
    const uint32_t* sbp;
    size_t blk;
    if constexpr (MW) {
      codes = a.codes[lw];
      sbp = a.sb[lw];
      blk = (size_t)lt * G + gb + lg;
      const bool adv = ls + 1 < ns, wg = adv && lg + 1 == gw, wt = wg && lt + 1 == a.T;
      ls += adv;
      lg = wg ? 0 : lg + adv;
      lt = wt ? 0 : lt + wg;
      lw += wt;
    } else {
      codes = a.codes[blockIdx.y];
      sbp = a.sb[blockIdx.y];
      blk = (size_t)t * G + gb + min(s, ns - 1);
    }
    if constexpr (Q8) {
      cbuf[slot] = load_nt(codes + blk * 128 + lane);  // weights: read once per call
      cbuf2[slot] = load_nt(codes + blk * 128 + 64 + lane);
    } else if constexpr (FMT == SDV_FMT_AFFINE_Q3) {
      const uint32_t* w = reinterpret_cast<const uint32_t*>(codes) + blk * 192 + lane;
      cbuf[slot] = make_uint4(load_nt(w), load_nt(w + 64), load_nt(w + 128), 0u);
    } else {
      cbuf[slot] = load_nt(codes + blk * 64 + lane);
    }
    sbuf[slot] = load_nt(sbp + blk * 32 + col);
  };
#pragma unroll
  for (int i = 0; i < PF; ++i) issue(i, i);

  // ---- staging into the wave's own region (no workgroup barrier)
  for (int tq = lane; tq < rs / 2; tq += 64) reinterpret_cast<uint32_t*>(xs + (size_t)a.cap * rs)[tq] = 0u;
  for (int tq = lane; tq < gw * SPG; tq += 64) xsum[k * gw * SPG + tq] = 0.0f;
  auto put_bf16 = [&](int task, const uint4 (&v)[8]) {
    const int i = task / gw, g = task - i * gw;
    float bsum[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      uint4 pk;
      bsum[q] = block8(v[q], pk);
      *reinterpret_cast<uint4*>(xs + (size_t)i * rs + g * 64 + q * 8) = pk;
    }
    if constexpr (Q8) {
      xsum[(i * gw + g) * 2] = half_total(bsum, 0);
      xsum[(i * gw + g) * 2 + 1] = half_total(bsum, 1);
    } else {
      xsum[i * gw + g] = group_total(bsum);
    }
  };
  // fp32 task: 64 values in two halves of 8 loads; each 8-value block is split
  // into three bf16 parts (hi, mid, lo), each part row summed as bf16 rows are,
  // and the row's group sum is the parts' sums added in part order
  auto put_f32 = [&](int task, const uint4 (&v0)[8], const float* src) {
    const int i = task / gw, g = task - i * gw;
    float bs[3][8];
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      // blocks 0-3 come from the first half already loaded, 4-7 one at a time
      uint4 u0, u1;
      if (blk < 4) {
        u0 = v0[2 * blk];
        u1 = v0[2 * blk + 1];
      } else {
        u0 = reinterpret_cast<const uint4*>(src)[2 * blk];
        u1 = reinterpret_cast<const uint4*>(src)[2 * blk + 1];
      }
      const float f[8] = {__uint_as_float(u0.x), __uint_as_float(u0.y), __uint_as_float(u0.z), __uint_as_float(u0.w),
                          __uint_as_float(u1.x), __uint_as_float(u1.y), __uint_as_float(u1.z), __uint_as_float(u1.w)};
      uint32_t hi[8], mi[8], lo[8];
      float acc[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        hi[c] = f32_to_bf16_rne(f[c]);
        const float r1 = f[c] - bf16_bits_to_f32(hi[c]);
        mi[c] = f32_to_bf16_rne(r1);
        const float r2 = r1 - bf16_bits_to_f32(mi[c]);
        lo[c] = f32_to_bf16_rne(r2);
        acc[0] = acc[0] + bf16_bits_to_f32(hi[c]);
        acc[1] = acc[1] + bf16_bits_to_f32(mi[c]);
        acc[2] = acc[2] + bf16_bits_to_f32(lo[c]);
      }
      *reinterpret_cast<uint4*>(xs + (size_t)(3 * i + 0) * rs + g * 64 + blk * 8) = nu_pack(hi);
      *reinterpret_cast<uint4*>(xs + (size_t)(3 * i + 1) * rs + g * 64 + blk * 8) = nu_pack(mi);
      *reinterpret_cast<uint4*>(xs + (size_t)(3 * i + 2) * rs + g * 64 + blk * 8) = nu_pack(lo);
#pragma unroll
      for (int p = 0; p < 3; ++p) bs[p][blk] = acc[p];
    }
    if constexpr (Q8) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        xsum[(i * gw + g) * 2 + h] = (half_total(bs[0], h) + half_total(bs[1], h)) + half_total(bs[2], h);
    } else {
      xsum[i * gw + g] = (group_total(bs[0]) + group_total(bs[1])) + group_total(bs[2]);
    }
  };
  for (int task = lane; task < ntask; task += 64) {
    if (task != lane) {
      const size_t e0 = task_src(task);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        xv[q] = ACT == SDV_ACT_BF16 ? reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.act) + e0)[q]
                                    : reinterpret_cast<const uint4*>(static_cast<const float*>(a.act) + e0)[q];
    }
    if (ACT == SDV_ACT_BF16) {
      put_bf16(task, xv);
    } else {
      put_f32(task, xv, static_cast<const float*>(a.act) + task_src(task));
    }
  }
  // the wave reads what its own lanes wrote: LDS operations of a wave complete
  // in order, so a compiler barrier suffices
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // ---- the wave's group steps: five accumulators per lane, y[i] for row
  // 4 half + i (i < 4) and y[4] for row 8 (in half 0)
  const int slot = slot_of_arow<ACT>(col, k);
  // a lane half reads elements 32 h .. of a Q4 group, 8 h .. (every 16) of a Q8_0 group
  const uint16_t* ap = xs + (size_t)(slot >= 0 ? slot : a.cap) * rs + half * (Q8 ? 8 : 32);
  const float* xr[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int r = i < 4 ? 4 * half + i : 8;
    xr[i] = xsum + (r < k ? r : k) * gw * SPG;
  }
  const DecodeK dk = decode_k();
  float y[5] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  // ---- cross-wave sum of item mi in wave order, then its epilogue
  float* red = reinterpret_cast<float*>(smem + (MW ? (size_t)nw * a.region : 0));
  const int cols_out = (MODE == SDV_MODE_PLAIN) ? 32 : 16;
  auto finish = [&](int tt, int wt) {
    __syncthreads();  // every wave is done with its region (one weight), or with the last weight's sums
    float* myred = red + (size_t)wave * kPassRows * 33;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int r = i < 4 ? 4 * half + i : 8;
      if (r < k && (i < 4 || half == 0)) myred[r * 33 + col] = y[i];
      y[i] = 0.0f;
    }
    __syncthreads();
    float* const out = a.out[wt];
    for (int q = tid; q < k * cols_out; q += blockDim.x) {
      const int i = q / cols_out, cc = q - i * cols_out;
      float val[2];
      const int ncol = (MODE == SDV_MODE_PLAIN) ? 1 : 2;
      for (int h2 = 0; h2 < ncol; ++h2) {
        const int cidx = cc + 16 * h2;
        float sum = 0.0f;
        for (int w = 0; w < nw; ++w) sum = sum + red[((size_t)w * kPassRows + i) * 33 + cidx];
        val[h2] = sum;
      }
      if (MODE == SDV_MODE_PLAIN) {
        const int on = tt * 32 + cc;
        if (on < a.N) out[(size_t)i * a.n_out + on] = val[0];
      } else {
        const int on = tt * 16 + cc;
        if (on < a.n_out) out[(size_t)i * a.n_out + on] = siluf_(val[0]) * val[1];
      }
    }
  };
  // step s: group cg of the item with tile ct and weight cw (MW: a cursor
  // that advances by one step per call; an item's sums are taken after its
  // last group).  Rounds before the last refill their slot after the step,
  // the last does not.
  int cg = 0, ct = item_tile(0), cw = item_weight(0);
  auto gstep = [&](int i, int s) {
    const int g = MW ? cg : s;
    if constexpr (Q8) {
      group_mac_rows_q8<ACT>(cbuf[i], cbuf2[i], sbuf[i], ap + g * 64, xr, g, y);
    } else {
      group_mac_rows<ACT, FMT>(cbuf[i], sbuf[i], ap + g * 64, xr, g, y, dk);
    }
    if constexpr (MW) {
      if (cg + 1 == gw) {
        finish(ct, cw);
        cg = 0;
        const bool wt = ct + 1 == a.T;
        ct = wt ? 0 : ct + 1;
        cw += wt;
      } else {
        ++cg;
      }
    }
  };
  const int nround = (ns + PF - 1) / PF;
  for (int r = 0; r + 1 < nround; ++r) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int s = r * PF + i;
      gstep(i, s);
      issue(i, s + PF);
    }
  }
  {
    const int s0 = (nround - 1) * PF;
#pragma unroll
    for (int i = 0; i < PF; ++i)
      if (s0 + i < ns) gstep(i, s0 + i);
  }
  if (!MW) finish(t, (int)blockIdx.y);
}

// Wide form: bf16 activations, more rows than one narrow pass (up to 32),
// affine Q4 or Q3.  The 32 rows of a tile's activation slices do not fit the
// LDS (32 rows of K = 5120 are 328 KB), so each wave reads the activation
// rows of one group at a time (an L2 hit after the first tile) in its load
// ring: lane l loads 8-element block l % 8 of rows l / 8 + 8 j (four loads,
// 8 cache lines each), NU-packs and sums it, and passes it through a small
// per-wave LDS tile to the lane that feeds it to the MFMA (lane (row r, half
// h) takes blocks 4 h .. 4 h + 3 of row r).  The group sum of a row adds its
// 8 block sums across the 8 lanes that hold them; the sums meet in a per-wave
// table, read back in the accumulator layout (lane half h holds rows
// 8 q + 4 h + 0..3).  A wave takes RPW consecutive K ranges of the narrow
// kernel, one after the other, and keeps their results apart.  The K
// ranges, the group step (the same MFMA chain and epilogue),
// the order of every sum and the cross-range sum are the narrow kernel's, so
// each row equals its narrow (and width-1) result bit for bit.
constexpr int kWideTileRow = 9;  // 16-byte blocks per tile row: 8 and one of padding
// Ring depth and K ranges per wave: one range per wave (16 waves at K >=
// 1024) with two groups in flight fits 128 VGPRs, so four waves share a SIMD;
// two ranges per wave with five in flight (2 waves per SIMD) measured 15.4
// against 12.8 us at 32 rows of 5120 x 5120.
constexpr int kWidePF = 2, kWideRPW = 1;

// sum8 by DPP moves within each 8-lane half row (pairs, then quads, then the
// two quads by the half-row mirror): ((b0 + b1) + (b2 + b3)) + ((b4 + b5) +
// (b6 + b7)) in every lane, the same value as sum8.
__device__ __forceinline__ float sum8_dpp(float x) {
  auto dpp = [](float v, int ctrl) -> float {
    switch (ctrl) {
      case 0xB1: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
      case 0x4E: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
      default: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
    }
  };
  x = x + dpp(x, 0xB1);   // quad_perm [1, 0, 3, 2]: lane ^ 1
  x = x + dpp(x, 0x4E);   // quad_perm [2, 3, 0, 1]: lane ^ 2
  return x + dpp(x, 0x141);  // row_half_mirror: lane 7 - lane within 8
}

template <int FMT, int MODE, int PF, int RPW>
__global__ __launch_bounds__(1024 / RPW, 1) void q4_dense_wide_kernel(DenseArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int t = blockIdx.x;
  const int G = a.G, K = a.K, k = a.k, nw = a.nw;  // nw: the narrow kernel's K ranges
  // ranges r0 = RPW wave and (RPW = 2) r0 + 1 if any: groups [gb, gm) and [gm, ge)
  const int r0 = RPW * wave, nr = min(RPW, nw - r0);
  const int gb = __builtin_amdgcn_readfirstlane((G * r0) / nw);
  const int gm = __builtin_amdgcn_readfirstlane((G * (r0 + 1)) / nw);
  const int ge = __builtin_amdgcn_readfirstlane((G * (r0 + nr)) / nw);
  const int ga = gm - gb, gn = ge - gb;  // steps of the first range, of both
  float* red = reinterpret_cast<float*>(smem);                          // [nw][32][33]
  float* xtab = red + (size_t)nw * 32 * 33 + wave * 32;                 // the current group's row sums
  uint4* xt = reinterpret_cast<uint4*>(red + (size_t)nw * 32 * 33 + (size_t)((nw + RPW - 1) / RPW) * 32) +
              (size_t)wave * 32 * kWideTileRow;                         // the group's rows, NU-packed blocks

  const uint4* const codes = a.codes[blockIdx.y];
  const uint32_t* const sbp = a.sb[blockIdx.y];
  float* const out = a.out[blockIdx.y];
  const size_t blk0 = (size_t)t * G + gb;
  // load j of a group: block lane % 8 of row lane / 8 + 8 j (rows past k: zeros)
  const int xr0 = lane >> 3, xq = lane & 7;
  const uint4* const xp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.act) + (size_t)gb * 64 + xq * 8);
  uint4 cbuf[PF], xbuf[PF][4];
  uint32_t sbuf[PF];
  auto issue = [&](int slot, int s) {
    const int g = min(s, gn - 1);
    const size_t blk = blk0 + g;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = xr0 + 8 * j;
      xbuf[slot][j] = row < k ? xp[(size_t)row * (K / 8) + g * 8] : make_uint4(0u, 0u, 0u, 0u);
    }
    if constexpr (FMT == SDV_FMT_AFFINE_Q3) {
      const uint32_t* w = reinterpret_cast<const uint32_t*>(codes) + blk * 192 + lane;
      cbuf[slot] = make_uint4(load_nt(w), load_nt(w + 64), load_nt(w + 128), 0u);
    } else {
      cbuf[slot] = load_nt(codes + blk * 64 + lane);  // weights: read once per call
    }
    sbuf[slot] = load_nt(sbp + blk * 32 + col);
  };
#pragma unroll
  for (int i = 0; i < PF; ++i) issue(i, i);

  const DecodeK dk = decode_k();
  float y[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) y[v] = 0.0f;
  // a range's results go to its row of the cross-range table
  auto put = [&](int r) {
    float* myred = red + (size_t)r * 32 * 33;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = 8 * (v >> 2) + 4 * half + (v & 3);
      if (row < k) myred[row * 33 + col] = y[v];
      y[v] = 0.0f;
    }
  };
  // One group step: the row's operands NU-packed and summed as the narrow
  // staging sums them (each 8-element block in order from zero, the half's
  // four blocks pairwise, then half 0 + half 1), the MFMA chain, and the
  // epilogue y += s P + (b - 128 s) X for each of the lane's 16 rows.
  auto step = [&](int i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4 pk;
      const float bs = block8(xbuf[i][j], pk);
      const int row = xr0 + 8 * j;
      xt[row * kWideTileRow + xq] = pk;
      const float X = sum8_dpp(bs);  // ((b0 + b1) + (b2 + b3)) + ((b4 + b5) + (b6 + b7)) of the row
      if (xq == 0) xtab[row] = X;
    }
    // The tile and the table are read back by the same wave: LDS operations
    // of a wave take effect in program order, and the compiler keeps these
    // accesses (all through smem) in that order.
    uint4 av[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) av[j] = xt[col * kWideTileRow + 4 * half + j];
    const float s = __uint_as_float(sbuf[i] << 16);
    const float b = __uint_as_float(sbuf[i] & 0xFFFF0000u);
    const float c = fmaf(-128.0f, s, b);
    f32x16 acc = {};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[j]), decode_step<FMT>(cbuf[i], j, dk),
                                                    acc, 0, 0, 0);
    float xg[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 x4 = *reinterpret_cast<const float4*>(xtab + 8 * q + 4 * half);
      xg[4 * q + 0] = x4.x;
      xg[4 * q + 1] = x4.y;
      xg[4 * q + 2] = x4.z;
      xg[4 * q + 3] = x4.w;
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      y[v] = fmaf(s, acc[v], y[v]);
      y[v] = fmaf(c, xg[v], y[v]);
    }
  };
  const int nround = (gn + PF - 1) / PF;
  for (int r = 0; r < nround; ++r) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int st = r * PF + i;
      if (st < gn) {
        if (st == ga) put(r0);  // the first range is complete
        step(i);
      }
      if (r + 1 < nround) issue(i, st + PF);
    }
  }
  put(nr == 2 ? r0 + 1 : r0);

  // ---- cross-range sum in range order, then the epilogue (as the narrow kernel)
  __syncthreads();
  const int cols_out = (MODE == SDV_MODE_PLAIN) ? 32 : 16;
  for (int q = tid; q < k * cols_out; q += blockDim.x) {
    const int i = q / cols_out, cc = q - i * cols_out;
    float val[2];
    const int ncol = (MODE == SDV_MODE_PLAIN) ? 1 : 2;
    for (int h2 = 0; h2 < ncol; ++h2) {
      const int cidx = cc + 16 * h2;
      float sum = 0.0f;
      for (int w = 0; w < nw; ++w) sum = sum + red[((size_t)w * 32 + i) * 33 + cidx];
      val[h2] = sum;
    }
    if (MODE == SDV_MODE_PLAIN) {
      const int on = t * 32 + cc;
      if (on < a.N) out[(size_t)i * a.n_out + on] = val[0];
    } else {
      const int on = t * 16 + cc;
      if (on < a.n_out) out[(size_t)i * a.n_out + on] = siluf_(val[0]) * val[1];
    }
  }
}

// the cross-range table [nw][32][33], then per wave a 32-float table and a
// tile of 32 rows x kWideTileRow blocks of 16 bytes
__host__ __device__ inline size_t dense_wide_lds_bytes(int nw, int rpw) {
  const size_t waves = (size_t)(nw + rpw - 1) / rpw;
  return (size_t)nw * 32 * 33 * 4 + waves * 32 * 4 + waves * 32 * kWideTileRow * 16;
}

template <int FMT, int MODE>
hipError_t dense_wide_launch_one(const DenseArgs& a, int nmulti, hipStream_t st) {
  constexpr int PF = kWidePF, RPW = kWideRPW;
  void (*kern)(DenseArgs) = q4_dense_wide_kernel<FMT, MODE, PF, RPW>;
  const size_t lds = dense_wide_lds_bytes(a.nw, RPW);
  static std::atomic<size_t> lds_limit{65536};
  size_t cur = lds_limit.load(std::memory_order_relaxed);
  if (lds > cur) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    while (cur < lds && !lds_limit.compare_exchange_weak(cur, lds)) {
    }
  }
  hipLaunchKernelGGL(kern, dim3(a.T, nmulti), dim3(64 * ((a.nw + RPW - 1) / RPW)), lds, st, a);
  return hipGetLastError();
}

// Raise a kernel's dynamic LDS limit once per process (the largest size
// asked for so far; the attribute is per function).
template <void (*KERN)(DenseArgs)>
hipError_t raise_dense_lds(size_t lds) {
  static std::atomic<size_t> lds_limit{65536};
  size_t cur = lds_limit.load(std::memory_order_relaxed);
  if (lds > cur) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(KERN),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    while (cur < lds && !lds_limit.compare_exchange_weak(cur, lds)) {
    }
  }
  return hipSuccess;
}

template <int FMT, int MODE, int ACT, int PF>
hipError_t dense_launch_one(const DenseArgs& a, int nmulti, size_t lds, hipStream_t st) {
  (void)nmulti;
  // (rings of 6 or 8 for the several-item stream measured no faster than the
  // range's own depth)
  constexpr auto one = q4_dense_k_kernel<FMT, MODE, ACT, PF, false>;
  constexpr auto several = q4_dense_k_kernel<FMT, MODE, ACT, PF, true>;
  const hipError_t err = a.mw > 1 ? raise_dense_lds<several>(lds) : raise_dense_lds<one>(lds);
  if (err != hipSuccess) return err;
  // several: one workgroup per compute unit, sharing the items evenly
  const dim3 grid = a.mw > 1 ? dim3((unsigned)min(a.items, device_cus())) : dim3(a.T, a.nmulti);
  hipLaunchKernelGGL(a.mw > 1 ? several : one, grid, dim3(64 * a.nw), lds, st, a);
  return hipGetLastError();
}

template <int FMT, int MODE, int ACT>
hipError_t dense_launch_pf(const DenseArgs& a, int nmulti, size_t lds, hipStream_t st) {
  // ring depth: the wave's whole range when it is short, else 8 with refills
  // (fp32 rows: 2, since staging the parts takes the registers; Q8_0 blocks
  // take two chunks, so at most 4; a Q3 ring of 5 spills, so 4)
  if constexpr (ACT == SDV_ACT_F32) {
    return dense_launch_one<FMT, MODE, ACT, 2>(a, nmulti, lds, st);
  } else if constexpr (FMT == SDV_FMT_AFFINE_Q3) {
    if (a.gwmax <= 2) return dense_launch_one<FMT, MODE, ACT, 2>(a, nmulti, lds, st);
    if (a.gwmax <= 5) return dense_launch_one<FMT, MODE, ACT, 4>(a, nmulti, lds, st);
    return dense_launch_one<FMT, MODE, ACT, 8>(a, nmulti, lds, st);
  } else if constexpr (FMT == SDV_FMT_Q8_0) {
    if (a.gwmax <= 2) return dense_launch_one<FMT, MODE, ACT, 2>(a, nmulti, lds, st);
    return dense_launch_one<FMT, MODE, ACT, 4>(a, nmulti, lds, st);
  } else {
    if (a.gwmax <= 2) return dense_launch_one<FMT, MODE, ACT, 2>(a, nmulti, lds, st);
    if (a.gwmax <= 4) return dense_launch_one<FMT, MODE, ACT, 4>(a, nmulti, lds, st);
    if (a.gwmax <= 5) return dense_launch_one<FMT, MODE, ACT, 5>(a, nmulti, lds, st);
    return dense_launch_one<FMT, MODE, ACT, 8>(a, nmulti, lds, st);
  }
}

}  // namespace

// Waves per tile: a function of K only, so the summation order is the same at
// every width.
int dense_waves_for(int K) {
  const int G = K / 64;
  return G < kDenseMaxWaves ? (G > 0 ? G : 1) : kDenseMaxWaves;
}

size_t dense_lds_bytes(int K, int act_dtype, int k, int fmt, int mw) {
  if (act_dtype == SDV_ACT_BF16 && k > kPassRows && fmt != SDV_FMT_Q8_0)
    return dense_wide_lds_bytes(dense_waves_for(K), kWideRPW);  // the wide form
  if (k > kPassRows) k = kPassRows;  // one launch per pass
  const int G = K / 64, nw = dense_waves_for(K);
  const int gwmax = (G + nw - 1) / nw;
  const int cap = act_dtype == SDV_ACT_F32 ? 3 * k : k;
  const size_t regions = (size_t)nw * dense_region_bytes(cap, gwmax, fmt == SDV_FMT_Q8_0 ? 2 : 1);
  const size_t red = dense_red_bytes(nw);
  if (mw > 1) return regions + red;  // the staged rows serve every item of the workgroup
  return regions > red ? regions : red;
}

// Items (tile, weight) per narrow workgroup in a launch over nmulti weights
// of T tiles: one per workgroup while they fit one workgroup per compute
// unit; beyond that one workgroup per compute unit, each taking an equal
// share of the items, so the rows are staged once per compute unit and no
// second round of workgroups leaves CUs idle at the end.
int dense_items_per_wg(int T, int nmulti) {
  const int items = T * nmulti, cus = device_cus();
  return items > cus ? (items + cus - 1) / cus : 1;
}

namespace {

// One launch over nmulti weights of W's shape and format (Ws[i], outputs
// outs[i]) that share the activation rows.
DenseArgs dense_args(const sdv_q4t* Ws, int nmulti, int mode, const void* act, int act_dtype, int k,
                     float* const* outs) {
  const sdv_q4t& W = Ws[0];
  DenseArgs a{};
  for (int m = 0; m < nmulti; ++m) {
    a.codes[m] = static_cast<const uint4*>(Ws[m].codes);
    a.sb[m] = Ws[m].sb;
    a.out[m] = outs[m];
  }
  a.act = act;
  a.N = W.N;
  a.K = W.K;
  a.T = (W.N + 31) / 32;
  a.G = W.K / 64;
  a.k = k;
  a.n_out = (mode == SDV_MODE_PLAIN) ? W.N : W.N / 2;
  a.nw = dense_waves_for(W.K);
  a.gwmax = (a.G + a.nw - 1) / a.nw;
  a.cap = act_dtype == SDV_ACT_F32 ? 3 * k : k;
  a.region = (int)dense_region_bytes(a.cap, a.gwmax, W.format == SDV_FMT_Q8_0 ? 2 : 1);
  a.nmulti = nmulti;
  a.items = a.T * nmulti;
  a.mw = 1;  // the wide form takes one item per workgroup; the narrow pass sets its own
  return a;
}

// Whether k rows take the wide form (one pass) instead of narrow passes.
bool dense_wide(int act_dtype, int k, int fmt) {
  return act_dtype == SDV_ACT_BF16 && k > kPassRows && fmt != SDV_FMT_Q8_0;
}

hipError_t dense_launch_wide(const sdv_q4t* Ws, int nmulti, int mode, const void* act, int k, float* const* outs,
                             hipStream_t st) {
  const DenseArgs a = dense_args(Ws, nmulti, mode, act, SDV_ACT_BF16, k, outs);
  const int fmt = Ws[0].format;
  if (fmt == SDV_FMT_AFFINE_Q4 && mode == SDV_MODE_PLAIN)
    return dense_wide_launch_one<SDV_FMT_AFFINE_Q4, SDV_MODE_PLAIN>(a, nmulti, st);
  if (fmt == SDV_FMT_AFFINE_Q4 && mode == SDV_MODE_GATEUP_SWIGLU)
    return dense_wide_launch_one<SDV_FMT_AFFINE_Q4, SDV_MODE_GATEUP_SWIGLU>(a, nmulti, st);
  if (fmt == SDV_FMT_AFFINE_Q3 && mode == SDV_MODE_PLAIN)
    return dense_wide_launch_one<SDV_FMT_AFFINE_Q3, SDV_MODE_PLAIN>(a, nmulti, st);
  if (fmt == SDV_FMT_AFFINE_Q3 && mode == SDV_MODE_GATEUP_SWIGLU)
    return dense_wide_launch_one<SDV_FMT_AFFINE_Q3, SDV_MODE_GATEUP_SWIGLU>(a, nmulti, st);
  return hipErrorInvalidValue;
}

hipError_t dense_launch_pass(const sdv_q4t* Ws, int nmulti, int mode, const void* act, int act_dtype, int k,
                             float* const* outs, hipStream_t st) {
  const sdv_q4t& W = Ws[0];
  DenseArgs a = dense_args(Ws, nmulti, mode, act, act_dtype, k, outs);
  a.mw = dense_items_per_wg(a.T, nmulti);
  // several items per workgroup keep the staged rows and add the sums'
  // table; past the LDS a workgroup takes one item (the size checked on the
  // host before the launch)
  if (a.mw > 1 && dense_lds_bytes(W.K, act_dtype, k, W.format, a.mw) > kDenseMaxLds) a.mw = 1;
  const size_t lds = dense_lds_bytes(W.K, act_dtype, k, W.format, a.mw);
#define SDV_DENSE(F, M, A) \
  if (W.format == F && mode == M && act_dtype == A) return dense_launch_pf<F, M, A>(a, nmulti, lds, st);
  SDV_DENSE(SDV_FMT_AFFINE_Q4, SDV_MODE_PLAIN, SDV_ACT_BF16)
  SDV_DENSE(SDV_FMT_AFFINE_Q4, SDV_MODE_PLAIN, SDV_ACT_F32)
  SDV_DENSE(SDV_FMT_AFFINE_Q4, SDV_MODE_GATEUP_SWIGLU, SDV_ACT_BF16)
  SDV_DENSE(SDV_FMT_AFFINE_Q4, SDV_MODE_GATEUP_SWIGLU, SDV_ACT_F32)
  SDV_DENSE(SDV_FMT_Q8_0, SDV_MODE_PLAIN, SDV_ACT_BF16)
  SDV_DENSE(SDV_FMT_Q8_0, SDV_MODE_PLAIN, SDV_ACT_F32)
  SDV_DENSE(SDV_FMT_Q8_0, SDV_MODE_GATEUP_SWIGLU, SDV_ACT_BF16)
  SDV_DENSE(SDV_FMT_Q8_0, SDV_MODE_GATEUP_SWIGLU, SDV_ACT_F32)
  SDV_DENSE(SDV_FMT_AFFINE_Q3, SDV_MODE_PLAIN, SDV_ACT_BF16)
  SDV_DENSE(SDV_FMT_AFFINE_Q3, SDV_MODE_PLAIN, SDV_ACT_F32)
  SDV_DENSE(SDV_FMT_AFFINE_Q3, SDV_MODE_GATEUP_SWIGLU, SDV_ACT_BF16)
  SDV_DENSE(SDV_FMT_AFFINE_Q3, SDV_MODE_GATEUP_SWIGLU, SDV_ACT_F32)
#undef SDV_DENSE
  return hipErrorInvalidValue;
}

}  // namespace

// Widths above one pass take the wide form (bf16 rows, affine Q4 or Q3: one
// launch for all rows); otherwise one launch per pass of at most kPassRows
// rows (rows 9c .. 9c + 8 of the activations and outputs), each reading the
// weights again.
hipError_t dense_multi_launch(const sdv_q4t* Ws, int nmulti, int mode, const void* act, int act_dtype, int k,
                              float* const* outs, hipStream_t st) {
  const sdv_q4t& W = Ws[0];
  if (nmulti < 1 || nmulti > kDenseMulti) return hipErrorInvalidValue;
  if (dense_wide(act_dtype, k, W.format)) return dense_launch_wide(Ws, nmulti, mode, act, k, outs, st);
  const size_t act_row = (size_t)W.K * (act_dtype == SDV_ACT_F32 ? 4 : 2);
  const int n_out = (mode == SDV_MODE_PLAIN) ? W.N : W.N / 2;
  for (int r0 = 0; r0 < k; r0 += kPassRows) {
    const int kc = k - r0 < kPassRows ? k - r0 : kPassRows;
    float* o[kDenseMulti];
    for (int m = 0; m < nmulti; ++m) o[m] = outs[m] + (size_t)r0 * n_out;
    const hipError_t e = dense_launch_pass(Ws, nmulti, mode, static_cast<const unsigned char*>(act) + r0 * act_row,
                                           act_dtype, kc, o, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t dense_launch(const sdv_q4t& W, int mode, const void* act, int act_dtype, int k, float* out,
                        hipStream_t st) {
  return dense_multi_launch(&W, 1, mode, act, act_dtype, k, &out, st);
}

int dense_multi_max() { return kDenseMulti; }

}  // namespace sdv
