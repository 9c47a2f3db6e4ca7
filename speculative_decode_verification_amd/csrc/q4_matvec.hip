// Multi-row affine-Q4 (group 64) products for gfx950: dense and gathered
// experts, plain or fused gate/up with SwiGLU, bf16 or fp32 activations.
//
// Each packed weight is read from HBM once and decoded once for all rows
// routed to it (mere.run transfer report, "Exact verification kernels and
// benchmark admission"; Red Lite dev45, "What it is").  On MI355X the product
// of up to 32 activation rows with a 32-column weight tile runs on the
// matrix cores (v_mfma_f32_32x32x16_bf16):
//
//   * A operand: activation rows staged once per workgroup in LDS as bf16.
//     fp32 activations are split exactly into three bf16 parts (hi, mid, lo),
//     each its own virtual row; the part results are added after the K loop.
//   * B operand: each code q becomes the bf16 value 128 + q with a single
//     and-or per two codes (0x4300 | q), which is exact.  Per 64-element group
//     the matrix core returns P = sum (128 + q) x, and the group contributes
//     s * P + (b - 128 s) * X to the output, X being the group sum of the
//     activation row (computed once, in a fixed order, while staging).
//   * Every output row's arithmetic depends only on its own activation row
//     and the weights: the K partition (fixed by K), the per-group epilogue
//     order and the cross-wave sum order do not depend on k or on which other
//     rows share the expert, so a width-k row is bit-identical to the width-1
//     row.
//
// Weight layout.  The kernels read the tiled layout written by
// sdv_q4_repack: for expert e, tile t (32 weight rows) and group g, a 1 KB
// block of codes in lane order (lane l = 32*half + col holds words
// 4*half .. 4*half+3 of the group in row col) and a 128-byte block of 32
// packed (scale | bias << 16) words.  A wave-step therefore reads 1 KB of
// contiguous codes and one 128-byte line of scales and biases, instead of 32
// scattered rows.  With fused gate/up weights, tile t holds gate rows
// 16t .. 16t+15 in columns 0-15 and the matching up rows in columns 16-31.
//
// Work decomposition.  Gathered units (union experts) run one wave per weight
// tile over the whole K: a workgroup of 8 waves takes 8 tiles of one expert,
// stages that expert's activation rows once, and each wave streams its tile
// through a ring of prefetched loads (8 groups deep).  The first loads are
// issued before staging, and finished tiles go through LDS so no global store
// sits among the stream's loads (on gfx9 loads and stores share one counter,
// and a pending store forces full waits).  Dense matrices (few tiles, long K)
// split K over the waves of a workgroup instead and add the partial results
// in wave order through LDS.
//
// Lane layout of v_mfma_f32_32x32x16_bf16 (64 lanes, l = lane):
//   A: lane l holds row l%32, K slots 8*(l/32) .. +7 (8 bf16)
//   B: lane l holds col l%32, the same K slots
//   D: lane l, register v holds row 8*(v/4) + 4*(l/32) + v%4, col l%32
// MFMA step j of a group consumes word j of the lane's 16 bytes.  Decoding a
// word gives bf16 pairs (n0,n4) (n1,n5) (n2,n6) (n3,n7), i.e. K slot i <->
// nibble NU[i] with NU = {0,4,1,5,2,6,3,7}; activations are stored in LDS in
// that order within each 8-element block so the A slots match.
//
// Virtual rows (MFMA rows).  bf16 activations: row i is MFMA row i.  fp32
// activations: part p of row i is MFMA row i + 8p for i < 8 and 24 + p for
// i = 8, so the three parts of a row land in one lane's registers.

#include <atomic>

#include "q4_core.h"

namespace sdv {

namespace {

using namespace q4;

constexpr int kTileCols = 32;
constexpr int kGatherWaves = 8;
constexpr int kGatherTilesPerWave = 1;  // tiles one wave streams back to back
constexpr int kPF = 8;        // groups in flight per lane (gathered units)

struct Q4Args {
  const uint4* codes;    // tiled: [E][T][G][64] uint4
  const uint32_t* sb;    // tiled: [E][T][G][32] (scale | bias << 16)
  int E, N, K, T;
  const void* act;
  // gathered
  const int32_t* union_ids;
  const int32_t* n_union;
  const int32_t* pair_off;
  const int32_t* pair_row;
  const int32_t* pair_slot;
  int k, topk;
  float* out;
  // optional extra unit (the shared expert): a dense weight with the same
  // geometry, applied to all k rows of xact ([k][K]), written to xout [k][n_out]
  const uint4* xcodes;
  const uint32_t* xsb;
  const void* xact;
  float* xout;
  int n_out;       // outputs per row: N (plain) or N/2 (gate/up)
  int slot_cap;    // activation rows staged in LDS (k or 3k)
  int tiles_per_block;
};

// FMT: SDV_FMT_AFFINE_Q4 or SDV_FMT_Q8_0 (two 1 KB code halves per group
// step, activation sums per 32-element block).
template <int FMT, int MODE, int ACT, int PF>
__device__ __forceinline__ void q4_matvec_body(const Q4Args& a, unsigned char* smem, int* s_src, int* s_dst) {
  constexpr bool Q8 = FMT == SDV_FMT_Q8_0;
  constexpr int SPG = Q8 ? 2 : 1;  // activation sums per group
  const int K = a.K;
  const int G = K >> 6;
  const int rs = K + 8;  // LDS row stride in bf16 (16-byte pad against bank conflicts)
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* xsum = reinterpret_cast<float*>(smem + (size_t)(a.slot_cap + 1) * rs * 2);  // [32][G * SPG]
  float* red = xsum + 32 * G * SPG;  // per-wave tile outputs

  const int tid = threadIdx.x;
  const int nw = blockDim.x >> 6;
  // wave-uniform values live in scalar registers, so the stream loop below
  // branches on scalars and keeps its loads in flight
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;

  // ---- the unit (union expert, the shared expert, or the dense matrix) and its rows
  // A unit's rows are taken kPassRows at a time: pass c = blockIdx.z takes
  // its rows 9c .. 9c + 8 (one pass unless k > kPassRows).
  int e = 0, p0 = 0, nrows = a.k, r0 = 0;
  const uint4* codes = a.codes;
  const uint32_t* sbp = a.sb;
  const void* act = a.act;
  float* out = a.out;
  bool pairs = true;  // rows come from the pair lists
  {
    const int u = blockIdx.y, pass0 = blockIdx.z * kPassRows;
    if (u == a.k * a.topk) {
      // the shared expert: all k rows, its own weight, input and output
      codes = a.xcodes;
      sbp = a.xsb;
      act = a.xact;
      out = a.xout;
      pairs = false;
      r0 = pass0;
      nrows = min(a.k - pass0, kPassRows);
      if (nrows <= 0) return;
    } else {
      const int nu = *a.n_union;
      if (u >= nu) return;
      e = a.union_ids[u];
      if (e < 0 || e >= a.E) return;
      p0 = a.pair_off[u];
      const int p1 = a.pair_off[u + 1];
      if (p0 < 0 || p1 <= p0 || p1 > a.k * a.topk) return;
      p0 += pass0;
      nrows = min(p1 - p0, kPassRows);
      if (nrows <= 0) return;
      e = __builtin_amdgcn_readfirstlane(e);
      p0 = __builtin_amdgcn_readfirstlane(p0);
      nrows = __builtin_amdgcn_readfirstlane(nrows);
    }
  }

  // ---- this wave's tiles (all groups of each), and its load stream
  const int tb0 = blockIdx.x * a.tiles_per_block;
  const int tb1 = min(tb0 + a.tiles_per_block, a.T);
  const int t_first = tb0 + wave, t_step = nw;
  const int t_count = t_first < tb1 ? (tb1 - t_first + nw - 1) / nw : 0;
  const int gb = 0, ge = G;
  const int gn = ge - gb;
  const int total = __builtin_amdgcn_readfirstlane(t_count * gn);

  // (tile, group) steps in order; block (t, g) of expert e starts at
  // ((e * T + t) * G + g) in units of 64 uint4 (Q4 codes), 128 uint4 (Q8_0
  // codes) or 32 words (sb)
  size_t ld_blk = ((size_t)e * a.T + t_first) * G + gb;
  int ld_g = gb;
  const size_t tile_jump = (size_t)t_step * G - gn;  // from the end of one tile's range to the next
  uint4 cbuf[PF], cbuf2[Q8 ? PF : 1];
  uint32_t sbuf[PF];
  auto issue = [&](int slot) {
    if constexpr (Q8) {
      cbuf[slot] = load_nt(codes + ld_blk * 128 + lane);  // weights: read once per call
      cbuf2[slot] = load_nt(codes + ld_blk * 128 + 64 + lane);
    } else if constexpr (FMT == SDV_FMT_AFFINE_Q3) {
      const uint32_t* w = reinterpret_cast<const uint32_t*>(codes) + ld_blk * 192 + lane;
      cbuf[slot] = make_uint4(load_nt(w), load_nt(w + 64), load_nt(w + 128), 0u);
    } else {
      cbuf[slot] = load_nt(codes + ld_blk * 64 + lane);
    }
    sbuf[slot] = load_nt(sbp + ld_blk * 32 + col);
    ++ld_blk;
    if (++ld_g == ge) {
      ld_g = gb;
      ld_blk += tile_jump;
    }
  };
#pragma unroll
  for (int i = 0; i < PF; ++i)
    if (i < total) issue(i);

  // ---- rows, then staging (the loads above are already in flight)
  if (tid < kPassRows) {
    int src = -1, dst = -1;
    if (tid < nrows) {
      if (pairs) {
        const int r = a.pair_row[p0 + tid], s = a.pair_slot[p0 + tid];
        if (r >= 0 && r < a.k && s >= 0 && s < a.topk) {
          src = (ACT == SDV_ACT_F32) ? r * a.topk + s : r;
          dst = r * a.topk + s;
        }
      } else {
        src = dst = r0 + tid;
      }
    }
    s_src[tid] = src;
    s_dst[tid] = dst;
  }
  __syncthreads();
  stage_rows<ACT, FMT>(act, a.K, a.slot_cap, nrows, xs, xsum, rs, s_src);
  __syncthreads();
  // The first ring loads were issued before staging and have had the staging
  // time to land; wait for them here so the stream loop is entered with no
  // load outstanding and its waits only count the loop's own refills.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0) (gfx9 encoding: expcnt 7, lgkmcnt 15)

  const int max_vrow = (ACT == SDV_ACT_F32) ? (nrows == 9 ? 27 : 16 + nrows) : nrows;
  const int nquads = (max_vrow + 7) >> 3;
  const int slot = slot_of_arow<ACT>(col, nrows);
  // rows without data read the zero row (LDS row slot_cap); a lane half
  // reads elements 32 h .. of a Q4 group, 8 h .. (every 16) of a Q8_0 group
  const uint16_t* arow_ptr = xs + (size_t)(slot >= 0 ? slot : a.slot_cap) * rs + half * (Q8 ? 8 : 32);

  float yacc[16];
  const DecodeK dk = decode_k();
  int cur_g = gb, cur_tl = 0;
  const int tiles_per_wave = (a.tiles_per_block + nw - 1) / nw;
  // One (tile, group) step: consume ring slot i, refill it (if asked) after
  // the slot's data has been decoded, and finish the tile after its last group.
  auto step = [&](int i, bool refill) {
    if (cur_g == gb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) yacc[v] = 0.0f;
    }
    if constexpr (Q8) {
      group_mac_q8(cbuf[i], cbuf2[i], sbuf[i], arow_ptr + cur_g * 64, xsum + 2 * cur_g, 2 * G, half, nquads, yacc);
    } else {
      group_mac<FMT>(cbuf[i], sbuf[i], arow_ptr + cur_g * 64, xsum + cur_g, G, half, nquads, yacc, dk);
    }
    if (refill) issue(i);
    if (++cur_g == ge) {
      {
        // finished tile values go to this wave's LDS area; the global stores
        // happen after the stream loop
        float* o = red + ((size_t)wave * tiles_per_wave + cur_tl) * kPassRows * 32;
#pragma unroll
        for (int r = 0; r < kPassRows; ++r) {
          if (r < nrows) {
            const float val = row_value<ACT>(yacc, r);
            const bool mine = half == half_of_row<ACT>(r);
            if (MODE == SDV_MODE_PLAIN) {
              if (mine) o[r * 32 + col] = val;
            } else {
              const float up = __shfl_xor(val, 16);
              if (mine && col < 16) o[r * 32 + col] = siluf_(val) * up;
            }
          }
        }
      }
      cur_g = gb;
      ++cur_tl;
    }
  };
  int st0 = 0;
  // steady state: every slot is refilled right after it is consumed
  for (; st0 + 2 * PF <= total; st0 += PF) {
#pragma unroll
    for (int i = 0; i < PF; ++i) step(i, true);
  }
  // drain: the last (< 2 PF) steps
  for (; st0 < total; st0 += PF) {
#pragma unroll
    for (int i = 0; i < PF; ++i)
      if (st0 + i < total) step(i, st0 + i + PF < total);
  }

  {
    __syncthreads();
    const int cols_out = (MODE == SDV_MODE_PLAIN) ? 32 : 16;
    const float* o = red + (size_t)wave * tiles_per_wave * kPassRows * 32;
    for (int tl = 0; tl < t_count; ++tl) {
      const int t = t_first + tl * t_step;
      const int on = t * cols_out + col;
      if (col < cols_out && on < a.n_out) {
        for (int r = 0; r < nrows; ++r) {
          const int orow = s_dst[r];
          if (orow >= 0) out[(size_t)orow * a.n_out + on] = o[(tl * kPassRows + r) * 32 + col];
        }
      }
    }
  }
}

// Gathered units: 8 waves per workgroup (one weight tile each), at most 128
// VGPRs so 4 waves fit per SIMD.
// (Q8_0: a ring of 4 two-chunk blocks keeps the same register budget.)
template <int FMT, int MODE, int ACT>
__global__ __launch_bounds__(512, 4) void q4_gather_kernel(Q4Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_src[kPassRows], s_dst[kPassRows];
  q4_matvec_body<FMT, MODE, ACT, FMT == SDV_FMT_Q8_0 ? kPF / 2 : kPF>(a, smem, s_src, s_dst);
}

template <int FMT, int MODE, int ACT>
hipError_t launch_one(const Q4Args& a, int blocks_x, int units, int nw, size_t lds, hipStream_t st) {
  void (*kern)(Q4Args) = q4_gather_kernel<FMT, MODE, ACT>;
  // raise the kernel's dynamic LDS limit once per process (the largest size
  // asked for so far; the attribute is per function, not per device)
  static std::atomic<size_t> lds_limit{65536};
  size_t cur = lds_limit.load(std::memory_order_relaxed);
  if (lds > cur) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    while (cur < lds && !lds_limit.compare_exchange_weak(cur, lds)) {
    }
  }
  const int passes = (a.k + kPassRows - 1) / kPassRows;
  hipLaunchKernelGGL(kern, dim3(blocks_x, units, passes), dim3(64 * nw), lds, st, a);
  return hipGetLastError();
}

// ---- repack: row-major affine Q4 -> tiled layout ---------------------------

struct RepackArgs {
  const uint32_t* codes;   // [E][N][K/8]
  const uint16_t* scales;  // [E][N][K/64]
  const uint16_t* biases;
  int E, N, K, T, fused;
  uint4* tcodes;           // [E][T][G][64]
  uint32_t* tsb;           // [E][T][G][32]
};

// Source row of column c of tile t (or -1 for a padding column).
__device__ __forceinline__ int repack_row(const RepackArgs& r, int t, int c) {
  if (!r.fused) {
    const int n = t * kTileCols + c;
    return n < r.N ? n : -1;
  }
  const int ihalf = r.N >> 1;
  const int i = t * 16 + (c & 15);
  if (i >= ihalf) return -1;
  return c < 16 ? i : ihalf + i;
}

__global__ __launch_bounds__(256) void q4_repack_kernel(RepackArgs r) {
  const int G = r.K >> 6;
  const size_t nblk = (size_t)r.E * r.T * G;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  // codes: one thread per 16-byte lane chunk
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < nblk * 64; idx += stride) {
    const int lane = (int)(idx & 63);
    const size_t blk = idx >> 6;
    const int g = (int)(blk % G);
    const size_t et = blk / G;
    const int t = (int)(et % r.T);
    const int e = (int)(et / r.T);
    const int n = repack_row(r, t, lane & 31);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (n >= 0) {
      const uint4* src = reinterpret_cast<const uint4*>(r.codes + ((size_t)e * r.N + n) * (r.K >> 3));
      v = src[2 * g + (lane >> 5)];
    }
    r.tcodes[idx] = v;
  }
  // scales and biases: one thread per (block, column)
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < nblk * 32; idx += stride) {
    const int c = (int)(idx & 31);
    const size_t blk = idx >> 5;
    const int g = (int)(blk % G);
    const size_t et = blk / G;
    const int t = (int)(et % r.T);
    const int e = (int)(et / r.T);
    const int n = repack_row(r, t, c);
    uint32_t w = 0;
    if (n >= 0) {
      const size_t o = ((size_t)e * r.N + n) * G + g;
      w = (uint32_t)r.scales[o] | ((uint32_t)r.biases[o] << 16);
    }
    r.tsb[idx] = w;
  }
}

// ---- repack: row-major Q8_0 -> tiled layout --------------------------------

struct Q8RepackArgs {
  const int8_t* qs;   // [E][N][K]
  const uint16_t* d;  // [E][N][K/32]
  int E, N, K, T, fused;
  uint4* tcodes;      // [E][T][G][2][64]
  uint32_t* tsb;      // [E][T][G][32]
};

__global__ __launch_bounds__(256) void q8_0_repack_kernel(Q8RepackArgs r) {
  const int G = r.K >> 6;
  const size_t nblk = (size_t)r.E * r.T * G;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const RepackArgs rows{nullptr, nullptr, nullptr, r.E, r.N, r.K, r.T, r.fused, nullptr, nullptr};
  // codes: one thread per 16-byte chunk (half p, lane l = 32 h + c): the
  // bytes of elements 32p + 8h + 0..7 and 32p + 16 + 8h + 0..7, as u = q + 128
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < nblk * 128; idx += stride) {
    const int lane = (int)(idx & 63), p = (int)((idx >> 6) & 1);
    const size_t blk = idx >> 7;
    const int g = (int)(blk % G);
    const size_t et = blk / G;
    const int t = (int)(et % r.T);
    const int e = (int)(et / r.T);
    const int n = repack_row(rows, t, lane & 31);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (n >= 0) {
      const int8_t* src = r.qs + ((size_t)e * r.N + n) * r.K + (size_t)g * 64 + 32 * p + 8 * (lane >> 5);
      const uint2 a = *reinterpret_cast<const uint2*>(src);
      const uint2 b = *reinterpret_cast<const uint2*>(src + 16);
      v = make_uint4(a.x ^ 0x80808080u, a.y ^ 0x80808080u, b.x ^ 0x80808080u, b.y ^ 0x80808080u);
    }
    r.tcodes[idx] = v;
  }
  // the two blocks' half scales: one thread per (block, column)
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < nblk * 32; idx += stride) {
    const int c = (int)(idx & 31);
    const size_t blk = idx >> 5;
    const int g = (int)(blk % G);
    const size_t et = blk / G;
    const int t = (int)(et % r.T);
    const int e = (int)(et / r.T);
    const int n = repack_row(rows, t, c);
    uint32_t w = 0;
    if (n >= 0) {
      const size_t o = ((size_t)e * r.N + n) * (2 * G) + 2 * g;
      w = (uint32_t)r.d[o] | ((uint32_t)r.d[o + 1] << 16);
    }
    r.tsb[idx] = w;
  }
}

// ---- repack: row-major affine Q3 -> tiled layout ----------------------------

struct Q3RepackArgs {
  const uint8_t* codes;  // [E][N][3K/8]
  const uint16_t* scales;
  const uint16_t* biases;
  int E, N, K, T, fused;
  uint32_t* tcodes;  // [E][T][G][3][64]
  uint32_t* tsb;     // [E][T][G][32]
};

__global__ __launch_bounds__(256) void q3_repack_kernel(Q3RepackArgs r) {
  const int G = r.K >> 6;
  const size_t nblk = (size_t)r.E * r.T * G;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const RepackArgs rows{nullptr, nullptr, nullptr, r.E, r.N, r.K, r.T, r.fused, nullptr, nullptr};
  // codes: one thread per (block, lane): the lane's 32 codes (12 bytes of the
  // row's stream, 4-byte aligned) into the three plane words
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < nblk * 64; idx += stride) {
    const int lane = (int)(idx & 63);
    const size_t blk = idx >> 6;
    const int g = (int)(blk % G);
    const size_t et = blk / G;
    const int t = (int)(et % r.T);
    const int e = (int)(et / r.T);
    const int n = repack_row(rows, t, lane & 31);
    uint32_t w[3] = {0u, 0u, 0u};
    if (n >= 0) {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(r.codes + ((size_t)e * r.N + n) * (3 * (size_t)r.K / 8) +
                                                              24 * (size_t)g + 12 * (lane >> 5));
      const uint64_t lo = (uint64_t)src[0] | ((uint64_t)src[1] << 32);
      const uint32_t hi = src[2];
      for (int el = 0; el < 32; ++el) {
        const int b = 3 * el;  // bits b .. b + 2 of the 96-bit value hi:lo
        uint32_t q;
        if (b + 3 <= 64)
          q = (uint32_t)(lo >> b) & 7u;
        else if (b < 64)
          q = (uint32_t)((lo >> b) | ((uint64_t)hi << (64 - b))) & 7u;
        else
          q = (hi >> (b - 64)) & 7u;
        // pair P = 4 j + i of MFMA step j holds elements i (low half) and
        // i + 4 (high half): bits 3 (P % 5) .. +2 of word P / 5, or, for P =
        // 15, bit b of the code in bit 15 of word b
        const int j = el >> 3, i8 = el & 7, i = i8 & 3, up = (i8 >> 2) * 16;
        const int P = 4 * j + i;
        if (P < 15) {
          const uint32_t v = q << (up + 3 * (P % 5));
          if (P < 5)
            w[0] |= v;
          else if (P < 10)
            w[1] |= v;
          else
            w[2] |= v;
        } else {
          w[0] |= (q & 1u) << (up + 15);
          w[1] |= ((q >> 1) & 1u) << (up + 15);
          w[2] |= ((q >> 2) & 1u) << (up + 15);
        }
      }
    }
#pragma unroll
    for (int p = 0; p < 3; ++p) r.tcodes[(blk * 3 + p) * 64 + lane] = w[p];
  }
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < nblk * 32; idx += stride) {
    const int c = (int)(idx & 31);
    const size_t blk = idx >> 5;
    const int g = (int)(blk % G);
    const size_t et = blk / G;
    const int t = (int)(et % r.T);
    const int e = (int)(et / r.T);
    const int n = repack_row(rows, t, c);
    uint32_t w = 0;
    if (n >= 0) {
      const size_t o = ((size_t)e * r.N + n) * G + g;
      w = (uint32_t)r.scales[o] | ((uint32_t)r.biases[o] << 16);
    }
    r.tsb[idx] = w;
  }
}

}  // namespace

int q4_tiles(int N, int fused);

size_t q3t_codes_bytes(int E, int N, int K, int fused) {
  return (size_t)E * q4_tiles(N, fused) * (K / 64) * 768;
}

hipError_t q3_repack_launch(const sdv_q3& src, int fused, void* tcodes, uint32_t* tsb, hipStream_t st) {
  Q3RepackArgs r{src.codes, src.scales, src.biases, src.E, src.N, src.K, q4_tiles(src.N, fused), fused,
                 static_cast<uint32_t*>(tcodes), tsb};
  const size_t n = (size_t)src.E * r.T * (src.K / 64) * 64;
  size_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(q3_repack_kernel, dim3((unsigned)blocks), dim3(256), 0, st, r);
  return hipGetLastError();
}

size_t q8_0t_codes_bytes(int E, int N, int K, int fused) {
  return (size_t)E * q4_tiles(N, fused) * (K / 64) * 2048;
}

hipError_t q8_0_repack_launch(const sdv_q8_0& src, int fused, void* tcodes, uint32_t* tsb, hipStream_t st) {
  Q8RepackArgs r{src.qs, src.d, src.E, src.N, src.K, q4_tiles(src.N, fused), fused, static_cast<uint4*>(tcodes), tsb};
  const size_t n = (size_t)src.E * r.T * (src.K / 64) * 128;
  size_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(q8_0_repack_kernel, dim3((unsigned)blocks), dim3(256), 0, st, r);
  return hipGetLastError();
}

// Tiles of a weight: 32 rows each, or 16 gate + 16 up rows when fused.
int q4_tiles(int N, int fused) { return fused ? (N / 2 + 15) / 16 : (N + kTileCols - 1) / kTileCols; }

size_t q4t_codes_bytes(int E, int N, int K, int fused) {
  return (size_t)E * q4_tiles(N, fused) * (K / 64) * 1024;
}

size_t q4t_sb_bytes(int E, int N, int K, int fused) { return (size_t)E * q4_tiles(N, fused) * (K / 64) * 128; }

hipError_t q4_repack_launch(const sdv_q4& src, int fused, void* tcodes, uint32_t* tsb, hipStream_t st) {
  RepackArgs r{src.codes, src.scales, src.biases, src.E, src.N, src.K, q4_tiles(src.N, fused), fused,
               static_cast<uint4*>(tcodes), tsb};
  const size_t n = (size_t)src.E * r.T * (src.K / 64) * 64;
  size_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(q4_repack_kernel, dim3((unsigned)blocks), dim3(256), 0, st, r);
  return hipGetLastError();
}

size_t dense_lds_bytes(int K, int act_dtype, int k, int fmt, int mw);
hipError_t dense_launch(const sdv_q4t& W, int mode, const void* act, int act_dtype, int k, float* out,
                        hipStream_t st);

size_t q4_lds_bytes_for(int K, int act_dtype, int k, bool gather, int fmt) {
  if (k > kPassRows) k = kPassRows;  // rows are staged one pass at a time
  const int cap = act_dtype == SDV_ACT_F32 ? 3 * k : k;
  const int spg = fmt == SDV_FMT_Q8_0 ? 2 : 1;  // activation sums per group
  // gathered: per-wave output staging for one tile of up to 9 rows x 32 columns
  return gather ? (size_t)(cap + 1) * (K + 8) * 2 + (size_t)32 * (K / 64) * spg * 4 +
                      (size_t)kGatherWaves * kGatherTilesPerWave * kPassRows * 32 * 4
                : dense_lds_bytes(K, act_dtype, k, fmt, 1);
}

hipError_t q4_launch(const sdv_q4t& W, int mode, const void* act, int act_dtype, bool gather,
                     const int32_t* union_ids, const int32_t* n_union, const int32_t* pair_off,
                     const int32_t* pair_row, const int32_t* pair_slot, int k, int topk, float* out,
                     const sdv_q4t* shared, const void* shared_act, float* shared_out, hipStream_t st) {
  Q4Args a;
  a.codes = static_cast<const uint4*>(W.codes);
  a.sb = W.sb;
  a.E = W.E;
  a.N = W.N;
  a.K = W.K;
  a.T = q4_tiles(W.N, W.fused_gateup);
  a.act = act;
  a.union_ids = union_ids;
  a.n_union = n_union;
  a.pair_off = pair_off;
  a.pair_row = pair_row;
  a.pair_slot = pair_slot;
  a.k = k;
  a.topk = topk;
  a.out = out;
  a.xcodes = shared ? static_cast<const uint4*>(shared->codes) : nullptr;
  a.xsb = shared ? shared->sb : nullptr;
  a.xact = shared_act;
  a.xout = shared_out;
  a.n_out = (mode == SDV_MODE_PLAIN) ? W.N : W.N / 2;
  const int kp = k < kPassRows ? k : kPassRows;  // rows staged per pass
  a.slot_cap = (act_dtype == SDV_ACT_F32) ? 3 * kp : kp;
  if (gather) {
    const int nw = kGatherWaves;
    a.tiles_per_block = nw * kGatherTilesPerWave;
    const int bx = (a.T + a.tiles_per_block - 1) / a.tiles_per_block;
    const int units = k * topk + (shared ? 1 : 0);
    const size_t lds = q4_lds_bytes_for(W.K, act_dtype, k, true, W.format);
#define SDV_Q4_G(F, M, A) \
  if (W.format == F && mode == M && act_dtype == A) return launch_one<F, M, A>(a, bx, units, nw, lds, st);
    SDV_Q4_G(SDV_FMT_AFFINE_Q4, SDV_MODE_PLAIN, SDV_ACT_BF16)
    SDV_Q4_G(SDV_FMT_AFFINE_Q4, SDV_MODE_PLAIN, SDV_ACT_F32)
    SDV_Q4_G(SDV_FMT_AFFINE_Q4, SDV_MODE_GATEUP_SWIGLU, SDV_ACT_BF16)
    SDV_Q4_G(SDV_FMT_AFFINE_Q4, SDV_MODE_GATEUP_SWIGLU, SDV_ACT_F32)
    SDV_Q4_G(SDV_FMT_Q8_0, SDV_MODE_PLAIN, SDV_ACT_BF16)
    SDV_Q4_G(SDV_FMT_Q8_0, SDV_MODE_PLAIN, SDV_ACT_F32)
    SDV_Q4_G(SDV_FMT_Q8_0, SDV_MODE_GATEUP_SWIGLU, SDV_ACT_BF16)
    SDV_Q4_G(SDV_FMT_Q8_0, SDV_MODE_GATEUP_SWIGLU, SDV_ACT_F32)
    SDV_Q4_G(SDV_FMT_AFFINE_Q3, SDV_MODE_PLAIN, SDV_ACT_BF16)
    SDV_Q4_G(SDV_FMT_AFFINE_Q3, SDV_MODE_PLAIN, SDV_ACT_F32)
    SDV_Q4_G(SDV_FMT_AFFINE_Q3, SDV_MODE_GATEUP_SWIGLU, SDV_ACT_BF16)
    SDV_Q4_G(SDV_FMT_AFFINE_Q3, SDV_MODE_GATEUP_SWIGLU, SDV_ACT_F32)
#undef SDV_Q4_G
  } else {
    return dense_launch(W, mode, act, act_dtype, k, out, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace sdv
