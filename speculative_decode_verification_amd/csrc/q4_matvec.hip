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
//     and the weights: the K partition (contiguous group ranges per wave,
//     fixed by K), the per-group epilogue order and the cross-wave sum order
//     do not depend on k or on which other rows share the expert, so a
//     width-k row is bit-identical to the width-1 row.
//
// Lane layout of v_mfma_f32_32x32x16_bf16 (64 lanes, l = lane):
//   A: lane l holds row l%32, K slots 8*(l/32) .. +7 (8 bf16)
//   B: lane l holds col l%32, the same K slots
//   D: lane l, register v holds row 8*(v/4) + 4*(l/32) + v%4, col l%32
// A lane (col, half) loads 16 bytes of codes = words 4*half .. 4*half+3 of its
// group; MFMA step j consumes word j.  Decoding word j gives bf16 pairs
// (n0,n4) (n1,n5) (n2,n6) (n3,n7), i.e. K slot i <-> nibble NU[i] with
// NU = {0,4,1,5,2,6,3,7}; activations are stored in LDS in that order within
// each 8-element block so the A slots match.

#include "common.h"

namespace sdv {

namespace {

constexpr int kTileCols = 32;
constexpr int kMaxVRows = 32;
constexpr int kMaxWaves = 8;
constexpr int kPF = 4;  // groups of codes in flight per lane

struct Q4Args {
  const uint32_t* codes;
  const uint16_t* scales;
  const uint16_t* biases;
  int E, N, K;
  const void* act;
  // gathered
  const int32_t* union_ids;
  const int32_t* n_union;
  const int32_t* pair_off;
  const int32_t* pair_row;
  const int32_t* pair_slot;
  int k, topk;
  float* out;
  int n_out;      // outputs per row: N (plain) or N/2 (gate/up)
  int vrow_cap;   // LDS rows reserved (k or 3k)
};

__device__ __forceinline__ uint32_t dec_pair(uint32_t w, int sh) {
  return ((w >> sh) & 0x000F000Fu) | 0x43004300u;
}

__device__ __forceinline__ bf16x8 decode_word(uint32_t w) {
  uint32_t p[4] = {dec_pair(w, 0), dec_pair(w, 4), dec_pair(w, 8), dec_pair(w, 12)};
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<uint4*>(p));
}

// Permute 8 bf16 values (natural K order in e[0..7]) into slot order NU.
__device__ __forceinline__ uint4 nu_pack(const uint32_t e[8]) {
  uint4 r;
  r.x = e[0] | (e[4] << 16);
  r.y = e[1] | (e[5] << 16);
  r.z = e[2] | (e[6] << 16);
  r.w = e[3] | (e[7] << 16);
  return r;
}

template <int MODE, int ACT, bool GATHER>
__global__ __launch_bounds__(512) void q4_matvec_kernel(Q4Args a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int K = a.K;
  const int G = K >> 6;
  const int rs = K + 8;  // LDS row stride in bf16 (16-byte pad against bank conflicts)
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  float* xsum = reinterpret_cast<float*>(smem + (size_t)a.vrow_cap * rs * 2);
  float* red = xsum + (size_t)a.vrow_cap * G;  // [nw][vrow_cap][33]

  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int nw = nthreads >> 6;
  const int wave = tid >> 6;
  const int lane = tid & 63;

  // ---- resolve the unit (union expert or the dense matrix) and its rows
  int e = 0, p0 = 0, nrows = a.k;
  if (GATHER) {
    const int u = blockIdx.y;
    int nu = *a.n_union;
    if (u >= nu) return;
    e = a.union_ids[u];
    if (e < 0 || e >= a.E) return;
    p0 = a.pair_off[u];
    const int p1 = a.pair_off[u + 1];
    nrows = p1 - p0;
    if (p0 < 0 || nrows <= 0 || p1 > a.k * a.topk) return;
    if (nrows > a.k) nrows = a.k;
  }
  const int nparts = (ACT == SDV_ACT_F32) ? 3 : 1;
  const int vrows = nrows * nparts;

  // ---- stage activation rows (bf16, NU order) and per-group sums into LDS.
  // One task = (real row, group): 64 consecutive inputs summed in order.
  for (int task = tid; task < nrows * G; task += nthreads) {
    const int i = task / G, g = task - i * G;
    bool ok = true;
    size_t src_row = (size_t)i;
    if (GATHER) {
      const int r = a.pair_row[p0 + i], s = a.pair_slot[p0 + i];
      ok = (r >= 0 && r < a.k && s >= 0 && s < a.topk);
      src_row = (ACT == SDV_ACT_F32) ? (size_t)(ok ? r : 0) * a.topk + (ok ? s : 0)
                                     : (size_t)(ok ? r : 0);
    }
    if (ACT == SDV_ACT_BF16) {
      const uint4* src = reinterpret_cast<const uint4*>(
          static_cast<const uint16_t*>(a.act) + src_row * K + (size_t)g * 64);
      float acc = 0.0f;
      uint16_t* dst = xs + (size_t)i * rs + g * 64;
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        uint4 v = ok ? src[b] : make_uint4(0, 0, 0, 0);
        uint32_t e8[8] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16,
                          v.z & 0xFFFFu, v.z >> 16, v.w & 0xFFFFu, v.w >> 16};
#pragma unroll
        for (int c = 0; c < 8; ++c) acc = acc + bf16_bits_to_f32(e8[c]);
        *reinterpret_cast<uint4*>(dst + b * 8) = nu_pack(e8);
      }
      xsum[(size_t)i * G + g] = acc;
    } else {
      const float4* src = reinterpret_cast<const float4*>(
          static_cast<const float*>(a.act) + src_row * K + (size_t)g * 64);
      float acc[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        float4 v0 = ok ? src[2 * b] : make_float4(0, 0, 0, 0);
        float4 v1 = ok ? src[2 * b + 1] : make_float4(0, 0, 0, 0);
        float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        uint32_t hi[8], mi[8], lo[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          hi[c] = f32_to_bf16_rne(f[c]);
          float r1 = f[c] - bf16_bits_to_f32(hi[c]);
          mi[c] = f32_to_bf16_rne(r1);
          float r2 = r1 - bf16_bits_to_f32(mi[c]);
          lo[c] = f32_to_bf16_rne(r2);
          acc[0] = acc[0] + bf16_bits_to_f32(hi[c]);
          acc[1] = acc[1] + bf16_bits_to_f32(mi[c]);
          acc[2] = acc[2] + bf16_bits_to_f32(lo[c]);
        }
        *reinterpret_cast<uint4*>(xs + (size_t)(3 * i + 0) * rs + g * 64 + b * 8) = nu_pack(hi);
        *reinterpret_cast<uint4*>(xs + (size_t)(3 * i + 1) * rs + g * 64 + b * 8) = nu_pack(mi);
        *reinterpret_cast<uint4*>(xs + (size_t)(3 * i + 2) * rs + g * 64 + b * 8) = nu_pack(lo);
      }
#pragma unroll
      for (int p = 0; p < 3; ++p) xsum[(size_t)(3 * i + p) * G + g] = acc[p];
    }
  }
  __syncthreads();

  // ---- this lane's weight column
  const int col = lane & 31, half = lane >> 5;
  int n;
  bool col_ok;
  if (MODE == SDV_MODE_PLAIN) {
    n = blockIdx.x * kTileCols + col;
    col_ok = n < a.N;
  } else {
    const int ihalf = a.N >> 1;
    const int i = blockIdx.x * 16 + (col & 15);
    col_ok = i < ihalf;
    n = (col < 16) ? i : ihalf + i;
  }
  if (!col_ok) n = 0;  // in-bounds dummy column; its results are never stored
  const size_t wrow = (size_t)e * a.N + n;
  const uint4* crow = reinterpret_cast<const uint4*>(a.codes + wrow * (size_t)(K >> 3)) + half;
  const uint16_t* srow = a.scales + wrow * (size_t)G;
  const uint16_t* brow = a.biases + wrow * (size_t)G;

  // contiguous group range of this wave (depends on K and the wave count only)
  const int gb = (G * wave) / nw;
  const int ge = (G * (wave + 1)) / nw;

  const int nquads = (vrows + 7) >> 3;
  const int arow = col;  // A operand row of this lane
  const bool a_ok = arow < vrows;
  const uint16_t* arow_ptr = xs + (size_t)(a_ok ? arow : 0) * rs + half * 32;

  float yacc[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) yacc[v] = 0.0f;

  uint4 cbuf[kPF];
  uint32_t sbuf[kPF], bbuf[kPF];
#pragma unroll
  for (int i = 0; i < kPF; ++i) {
    if (gb + i < ge) {
      cbuf[i] = crow[(size_t)(gb + i) * 2];
      sbuf[i] = srow[gb + i];
      bbuf[i] = brow[gb + i];
    }
  }

  for (int g0 = gb; g0 < ge; g0 += kPF) {
#pragma unroll
    for (int i = 0; i < kPF; ++i) {
      const int g = g0 + i;
      if (g < ge) {
        const uint4 cw = cbuf[i];
        const float s = bf16_bits_to_f32(sbuf[i]);
        const float b = bf16_bits_to_f32(bbuf[i]);
        if (g + kPF < ge) {
          cbuf[i] = crow[(size_t)(g + kPF) * 2];
          sbuf[i] = srow[g + kPF];
          bbuf[i] = brow[g + kPF];
        }
        const float c = fmaf(-128.0f, s, b);
        const uint16_t* ap = arow_ptr + g * 64;
        f32x16 acc = {};
        const uint32_t cws[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint4 av = a_ok ? *reinterpret_cast<const uint4*>(ap + j * 8) : make_uint4(0, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                        decode_word(cws[j]), acc, 0, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (q < nquads) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int v = 4 * q + r;
              const int vr = 8 * q + 4 * half + r;
              const float xg = (vr < vrows) ? xsum[(size_t)vr * G + g] : 0.0f;
              yacc[v] = fmaf(s, acc[v], yacc[v]);
              yacc[v] = fmaf(c, xg, yacc[v]);
            }
          }
        }
      }
    }
  }

  // ---- cross-wave reduction in wave order, then the epilogue
  float* myred = red + (size_t)wave * a.vrow_cap * 33;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (q < nquads) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int vr = 8 * q + 4 * half + r;
        if (vr < vrows) myred[(size_t)vr * 33 + col] = yacc[4 * q + r];
      }
    }
  }
  __syncthreads();

  const int cols_out = (MODE == SDV_MODE_PLAIN) ? 32 : 16;
  for (int t = tid; t < nrows * cols_out; t += nthreads) {
    const int i = t / cols_out, cc = t - i * cols_out;
    size_t orow = (size_t)i;
    if (GATHER) {
      const int r = a.pair_row[p0 + i], s = a.pair_slot[p0 + i];
      if (r < 0 || r >= a.k || s < 0 || s >= a.topk) continue;
      orow = (size_t)r * a.topk + s;
    }
    float val[2];
    const int ncol = (MODE == SDV_MODE_PLAIN) ? 1 : 2;
    for (int h2 = 0; h2 < ncol; ++h2) {
      const int cidx = cc + 16 * h2;
      float part[3];
      for (int p = 0; p < nparts; ++p) {
        const int vr = nparts * i + p;
        float sum = 0.0f;
        for (int w = 0; w < nw; ++w) sum = sum + red[((size_t)w * a.vrow_cap + vr) * 33 + cidx];
        part[p] = sum;
      }
      val[h2] = (nparts == 3) ? (part[0] + part[1]) + part[2] : part[0];
    }
    if (MODE == SDV_MODE_PLAIN) {
      const int on = blockIdx.x * kTileCols + cc;
      if (on < a.N) a.out[orow * a.n_out + on] = val[0];
    } else {
      const int on = blockIdx.x * 16 + cc;
      if (on < a.n_out) a.out[orow * a.n_out + on] = siluf_(val[0]) * val[1];
    }
  }
}

template <int MODE, int ACT, bool GATHER>
hipError_t launch_one(const Q4Args& a, int tiles, int units, int nw, size_t lds, hipStream_t st) {
  auto kern = q4_matvec_kernel<MODE, ACT, GATHER>;
  if (lds > 65536) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(kern, dim3(tiles, units), dim3(64 * nw), lds, st, a);
  return hipGetLastError();
}

}  // namespace

// Waves per workgroup (split of the K groups): a function of K only, so the
// summation order never depends on the row count.
int q4_waves_for(int K) {
  const int G = K / 64;
  int nw = G / 5;
  if (nw < 1) nw = 1;
  if (nw > kMaxWaves) nw = kMaxWaves;
  return nw;
}

size_t q4_lds_bytes(int K, int vrow_cap, int nw) {
  const int G = K / 64;
  return (size_t)vrow_cap * (K + 8) * 2 + (size_t)vrow_cap * G * 4 + (size_t)nw * vrow_cap * 33 * 4;
}

hipError_t q4_launch(const sdv_q4& W, int mode, const void* act, int act_dtype, bool gather,
                     const int32_t* union_ids, const int32_t* n_union, const int32_t* pair_off,
                     const int32_t* pair_row, const int32_t* pair_slot, int k, int topk, float* out,
                     hipStream_t st) {
  Q4Args a;
  a.codes = W.codes;
  a.scales = W.scales;
  a.biases = W.biases;
  a.E = W.E;
  a.N = W.N;
  a.K = W.K;
  a.act = act;
  a.union_ids = union_ids;
  a.n_union = n_union;
  a.pair_off = pair_off;
  a.pair_row = pair_row;
  a.pair_slot = pair_slot;
  a.k = k;
  a.topk = topk;
  a.out = out;
  a.n_out = (mode == SDV_MODE_PLAIN) ? W.N : W.N / 2;
  a.vrow_cap = (act_dtype == SDV_ACT_F32) ? 3 * k : k;
  const int nw = q4_waves_for(W.K);
  const size_t lds = q4_lds_bytes(W.K, a.vrow_cap, nw);
  const int tiles = (mode == SDV_MODE_PLAIN) ? (W.N + kTileCols - 1) / kTileCols : (W.N / 2 + 15) / 16;
  const int units = gather ? k * topk : 1;
#define SDV_Q4_CASE(M, A, GA)                                                  \
  if (mode == M && act_dtype == A && gather == GA)                             \
    return launch_one<M, A, GA>(a, tiles, units, nw, lds, st);
  SDV_Q4_CASE(SDV_MODE_PLAIN, SDV_ACT_BF16, false)
  SDV_Q4_CASE(SDV_MODE_PLAIN, SDV_ACT_F32, false)
  SDV_Q4_CASE(SDV_MODE_GATEUP_SWIGLU, SDV_ACT_BF16, false)
  SDV_Q4_CASE(SDV_MODE_GATEUP_SWIGLU, SDV_ACT_F32, false)
  SDV_Q4_CASE(SDV_MODE_PLAIN, SDV_ACT_BF16, true)
  SDV_Q4_CASE(SDV_MODE_PLAIN, SDV_ACT_F32, true)
  SDV_Q4_CASE(SDV_MODE_GATEUP_SWIGLU, SDV_ACT_BF16, true)
  SDV_Q4_CASE(SDV_MODE_GATEUP_SWIGLU, SDV_ACT_F32, true)
#undef SDV_Q4_CASE
  return hipErrorInvalidValue;
}

}  // namespace sdv
