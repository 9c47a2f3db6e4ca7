// Device helpers of the affine-Q4 products (gfx950): code decode, the
// activation staging in MFMA slot order and the per-group MFMA step with its
// scale/bias epilogue.  Layout conventions of v_mfma_f32_32x32x16_bf16:
//   A: lane l holds row l%32, K slots 8*(l/32) .. +7 (8 bf16)
//   B: lane l holds col l%32, the same K slots
//   D: lane l, register v holds row 8*(v/4) + 4*(l/32) + v%4, col l%32
// A code q decodes to the bf16 value 128 + q; decoding a 32-bit word gives the
// bf16 pairs (n0,n4) (n1,n5) (n2,n6) (n3,n7), so K slot i holds nibble NU[i]
// with NU = {0,4,1,5,2,6,3,7}, and activations are staged in that order.
// fp32 activations are split into three bf16 parts; part p of row i is MFMA
// row i + 8p for i < 8 and 24 + p for i = 8.
#pragma once

#include "common.h"

namespace sdv {
namespace q4 {

// The decode's mask and bf16 bias pattern, held in registers.  A gfx9 VOP3
// instruction takes at most one literal, so with both constants as literals
// the and-or of a pair becomes two instructions; from registers it is one
// v_and_or_b32.  The empty asm makes the values opaque so they stay in VGPRs.
struct DecodeK {
  uint32_t mask, bias;
};

__device__ __forceinline__ DecodeK decode_k() {
  DecodeK d{0x000F000Fu, 0x43004300u};
  asm volatile("" : "+v"(d.mask), "+v"(d.bias));
  return d;
}

__device__ __forceinline__ uint32_t dec_pair(uint32_t w, int sh, DecodeK d) { return ((w >> sh) & d.mask) | d.bias; }

__device__ __forceinline__ bf16x8 decode_word(uint32_t w, DecodeK d) {
  uint32_t p[4] = {dec_pair(w, 0, d), dec_pair(w, 4, d), dec_pair(w, 8, d), dec_pair(w, 12, d)};
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<uint4*>(p));
}

// Affine Q3: a lane's 32 codes of a group in three words (the tiled layout
// of SDV_FMT_AFFINE_Q3).  Code pair P = 4 j + i (MFMA step j, elements i and
// i + 4, i < 4) holds element i's three bits at bit 3 (P % 5) of word P / 5
// and element i + 4's sixteen bits higher, for P < 15, so the pair decodes
// like a Q4 nibble pair: one shift and one and-or give the bf16 values
// 128 + q of elements (i, i + 4).  Pair 15 keeps bit b of its two codes in
// bits 15 and 31 of word b (the bits the five 3-bit fields of each half
// leave over).
__device__ __forceinline__ uint32_t q3_pair(uint32_t w, int s, DecodeK d) { return ((w >> s) & 0x00070007u) | d.bias; }

__device__ __forceinline__ bf16x8 decode_q3(const uint4 cw, int j, DecodeK d) {
  uint32_t p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int P = 4 * j + i;
    if (P < 15) {
      const uint32_t w = P < 5 ? cw.x : (P < 10 ? cw.y : cw.z);
      p[i] = q3_pair(w, 3 * (P % 5), d);
    } else {
      p[i] = ((cw.x >> 15) & 0x00010001u) | ((cw.y >> 14) & 0x00020002u) | ((cw.z >> 13) & 0x00040004u) | d.bias;
    }
  }
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<uint4*>(p));
}

// The codes of MFMA step j of a Q4 or Q3 block.
template <int FMT>
__device__ __forceinline__ bf16x8 decode_step(const uint4 cw, int j, DecodeK d) {
  if constexpr (FMT == SDV_FMT_AFFINE_Q3) {
    return decode_q3(cw, j, d);
  } else {
    const uint32_t cws[4] = {cw.x, cw.y, cw.z, cw.w};
    return decode_word(cws[j], d);
  }
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

// MFMA row of part p of activation row i.
template <int ACT>
__device__ __forceinline__ int vrow_of(int i, int p) {
  if (ACT == SDV_ACT_BF16) return i;
  return i < 8 ? i + 8 * p : 24 + p;
}

// Register of the D layout holding MFMA row vr (for the lane half (vr/4)%2).
__device__ __forceinline__ int reg_of(int vr) { return 4 * (vr >> 3) + (vr & 3); }

// Sum over the 8 lanes l .. l+7 (l a multiple of 8); every lane of the group
// ends with the same total (xor pairing adds the same two operands in both
// lanes of a pair).
__device__ __forceinline__ float sum8(float x) {
  x = x + __shfl_xor(x, 1);
  x = x + __shfl_xor(x, 2);
  x = x + __shfl_xor(x, 4);
  return x;
}

// The same over the 4 lanes l .. l+3 (l a multiple of 4).
__device__ __forceinline__ float sum4(float x) {
  x = x + __shfl_xor(x, 1);
  x = x + __shfl_xor(x, 2);
  return x;
}

// Stage the unit's activation rows into LDS (NU order, bf16 parts) and their
// per-group sums (indexed by MFMA row).  One task = (row, 8-element block):
// the block's elements are summed in order, then the 8 blocks of a group are
// summed by the fixed 8-lane pairing above.
//   act       rows of K elements (bf16 bits or fp32), row s_src[i] feeds row i
//   slot_cap  LDS row of the all-zero row (rows past the data read it)
//   FMT       SDV_FMT_AFFINE_Q4: one sum per 64-element group (xsum [32][G]);
//             SDV_FMT_Q8_0: one per 32-element block (xsum [32][2G]), the
//             first four 8-blocks then the last four, each added pairwise
template <int ACT, int FMT = SDV_FMT_AFFINE_Q4>
__device__ __forceinline__ void stage_rows(const void* act, int K, int slot_cap, int nrows, uint16_t* xs,
                                           float* xsum, int rs, const int* s_src) {
  const int G = K >> 6, nb = K >> 3;
  constexpr int SPG = FMT == SDV_FMT_Q8_0 ? 2 : 1;  // sums per group
  const int tid = threadIdx.x, nthreads = blockDim.x;
  for (int t = tid; t < 32 * G * SPG; t += nthreads) xsum[t] = 0.0f;
  uint32_t* zrow = reinterpret_cast<uint32_t*>(xs + (size_t)slot_cap * rs);
  for (int t = tid; t < rs / 2; t += nthreads) zrow[t] = 0u;
  __syncthreads();
  // nthreads is a multiple of 64 and the task count a multiple of 8, so the 8
  // tasks of a group share one 8-lane set and are all valid or all not.  A
  // thread loads a batch of its tasks before processing any of them, so it
  // waits for memory once per batch instead of once per task.
  constexpr int B = ACT == SDV_ACT_BF16 ? 4 : 2;
  const int ntask = nrows * nb;
  for (int base = tid; base < ntask; base += B * nthreads) {
    if (ACT == SDV_ACT_BF16) {
      uint4 v[B];
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const int task = base + u * nthreads;
        const int i = task / nb, b8 = task - i * nb;
        const int src = task < ntask ? s_src[i] : -1;
        v[u] = src >= 0 ? reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(act) + (size_t)src * K)[b8]
                        : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const int task = base + u * nthreads;
        if (task >= ntask) break;
        const int i = task / nb, b8 = task - i * nb;
        const uint32_t e8[8] = {v[u].x & 0xFFFFu, v[u].x >> 16, v[u].y & 0xFFFFu, v[u].y >> 16,
                                v[u].z & 0xFFFFu, v[u].z >> 16, v[u].w & 0xFFFFu, v[u].w >> 16};
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) acc = acc + bf16_bits_to_f32(e8[c]);
        *reinterpret_cast<uint4*>(xs + (size_t)i * rs + b8 * 8) = nu_pack(e8);
        if constexpr (FMT == SDV_FMT_Q8_0) {
          acc = sum4(acc);
          if ((b8 & 3) == 0) xsum[vrow_of<ACT>(i, 0) * 2 * G + (b8 >> 2)] = acc;
        } else {
          acc = sum8(acc);
          if ((b8 & 7) == 0) xsum[vrow_of<ACT>(i, 0) * G + (b8 >> 3)] = acc;
        }
      }
    } else {
      float4 v0[B], v1[B];
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const int task = base + u * nthreads;
        const int i = task / nb, b8 = task - i * nb;
        const int src = task < ntask ? s_src[i] : -1;
        const float4* sp = reinterpret_cast<const float4*>(static_cast<const float*>(act) + (size_t)(src >= 0 ? src : 0) * K) + 2 * b8;
        v0[u] = src >= 0 ? sp[0] : make_float4(0, 0, 0, 0);
        v1[u] = src >= 0 ? sp[1] : make_float4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const int task = base + u * nthreads;
        if (task >= ntask) break;
        const int i = task / nb, b8 = task - i * nb;
        const float f[8] = {v0[u].x, v0[u].y, v0[u].z, v0[u].w, v1[u].x, v1[u].y, v1[u].z, v1[u].w};
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
        *reinterpret_cast<uint4*>(xs + (size_t)(3 * i + 0) * rs + b8 * 8) = nu_pack(hi);
        *reinterpret_cast<uint4*>(xs + (size_t)(3 * i + 1) * rs + b8 * 8) = nu_pack(mi);
        *reinterpret_cast<uint4*>(xs + (size_t)(3 * i + 2) * rs + b8 * 8) = nu_pack(lo);
#pragma unroll
        for (int p = 0; p < 3; ++p) {
          if constexpr (FMT == SDV_FMT_Q8_0) {
            const float t = sum4(acc[p]);
            if ((b8 & 3) == 0) xsum[vrow_of<ACT>(i, p) * 2 * G + (b8 >> 2)] = t;
          } else {
            const float t = sum8(acc[p]);
            if ((b8 & 7) == 0) xsum[vrow_of<ACT>(i, p) * G + (b8 >> 3)] = t;
          }
        }
      }
    }
  }
}

// LDS slot of the activation data for MFMA row `arow` (or -1 if unused).
template <int ACT>
__device__ __forceinline__ int slot_of_arow(int arow, int nrows) {
  if (ACT == SDV_ACT_BF16) return arow < nrows ? arow : -1;
  if (arow < 24) {
    const int i = arow & 7, p = arow >> 3;
    return i < nrows ? 3 * i + p : -1;
  }
  const int p = arow - 24;
  return (nrows == 9 && p < 3) ? 24 + p : -1;
}

// One 64-element group: 4 MFMA steps, then the group's scale/bias epilogue
// into yacc for the first `nquads` register quads.  `ap` points at this
// lane's activation row (or at an all-zero LDS row), so the four A reads are
// issued together, unconditionally, before the decode.
template <int FMT = SDV_FMT_AFFINE_Q4>
__device__ __forceinline__ void group_mac(const uint4 cw, uint32_t sbw, const uint16_t* ap, const float* xs_g,
                                          int G, int half, int nquads, float yacc[16], DecodeK dk) {
  uint4 av[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) av[j] = *reinterpret_cast<const uint4*>(ap + j * 8);
  const float s = __uint_as_float(sbw << 16);
  const float b = __uint_as_float(sbw & 0xFFFF0000u);
  const float c = fmaf(-128.0f, s, b);
  f32x16 acc = {};
#pragma unroll
  for (int j = 0; j < 4; ++j)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[j]), decode_step<FMT>(cw, j, dk), acc,
                                                  0, 0, 0);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (q < nquads) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = 4 * q + r;
        const float xg = xs_g[(8 * q + 4 * half + r) * G];
        yacc[v] = fmaf(s, acc[v], yacc[v]);
        yacc[v] = fmaf(c, xg, yacc[v]);
      }
    }
  }
}

// The same group step with the parts of each activation row summed right after
// the matrix product, so a lane keeps five accumulators: y[i] for row
// 4*half + i (i < 4) and y[4] for row 8 (meaningful in half 0).  xr[i] points
// at the group sums of the row behind y[i] (for fp32 rows, of all three parts)
// and s_idx is the group.  Per group,
//   y += s * P + (b - 128 s) * X,   P = the row's parts' products summed in part order.
template <int ACT, int FMT = SDV_FMT_AFFINE_Q4>
__device__ __forceinline__ void group_mac_rows(const uint4 cw, uint32_t sbw, const uint16_t* ap,
                                               const float* const (&xr)[5], int s_idx, float y[5], DecodeK dk) {
  uint4 av[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) av[j] = *reinterpret_cast<const uint4*>(ap + j * 8);
  const float s = __uint_as_float(sbw << 16);
  const float b = __uint_as_float(sbw & 0xFFFF0000u);
  const float c = fmaf(-128.0f, s, b);
  f32x16 acc = {};
#pragma unroll
  for (int j = 0; j < 4; ++j)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[j]), decode_step<FMT>(cw, j, dk), acc,
                                                  0, 0, 0);
  float t[5];
  if (ACT == SDV_ACT_BF16) {
#pragma unroll
    for (int i = 0; i < 5; ++i) t[i] = acc[i];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = (acc[i] + acc[4 + i]) + acc[8 + i];
    t[4] = (acc[12] + acc[13]) + acc[14];
  }
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    y[i] = fmaf(s, t[i], y[i]);
    y[i] = fmaf(c, xr[i][s_idx], y[i]);
  }
}

// ---- Q8_0 ---------------------------------------------------------------
// The tiled code byte is u = q + 128 (0..255): it converts exactly to fp32,
// and with at most 8 significant bits its bf16 is the fp32's high half.  The
// matrix core returns P = sum u x = sum q x + 128 X per 32-element block, so
// a block adds d P - 128 d X.  MFMA step j of lane half h takes elements
// 16 j + 8 h .. + 7 of the group (steps 0-1: block 0, steps 2-3: block 1);
// its two code words hold elements 0-3 and 4-7, and the pairs (byte i of
// word 0, byte i of word 1) give K slots in the Q4 decode's NU order.
__device__ __forceinline__ uint32_t q8_pair(uint32_t w0, uint32_t w1, int i) {
  const float lo = (float)((w0 >> (8 * i)) & 0xFFu);
  const float hi = (float)((w1 >> (8 * i)) & 0xFFu);
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);  // hi.h16 : lo.h16
}

__device__ __forceinline__ bf16x8 decode_q8(uint32_t w0, uint32_t w1) {
  uint32_t p[4] = {q8_pair(w0, w1, 0), q8_pair(w0, w1, 1), q8_pair(w0, w1, 2), q8_pair(w0, w1, 3)};
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<uint4*>(p));
}

__device__ __forceinline__ float half_bits_to_f32(uint32_t h16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);
}

// The two blocks' matrix products of one Q8_0 group: acc[0] over block 0,
// acc[1] over block 1.  `ap` points at the lane's row at element 8 h of the
// group (steps at + 16 j); c0 holds code words 0-3 (steps 0, 1), c1 words
// 4-7 (steps 2, 3).
__device__ __forceinline__ void q8_products(const uint4 c0, const uint4 c1, const uint16_t* ap, f32x16 (&acc)[2]) {
  uint4 av[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) av[j] = *reinterpret_cast<const uint4*>(ap + j * 16);
  acc[0] = f32x16{};
  acc[1] = f32x16{};
  acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[0]), decode_q8(c0.x, c0.y), acc[0],
                                                   0, 0, 0);
  acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[1]), decode_q8(c0.z, c0.w), acc[0],
                                                   0, 0, 0);
  acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[2]), decode_q8(c1.x, c1.y), acc[1],
                                                   0, 0, 0);
  acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[3]), decode_q8(c1.z, c1.w), acc[1],
                                                   0, 0, 0);
}

// group_mac for a Q8_0 group: xs_g points at the group's two block sums of
// MFMA row 0 (row vr at xs_g[vr * G2], G2 = 2 G); sbw holds the blocks' half
// scales (block 0 low, block 1 high).  Per block b: yacc += d_b P_b - 128 d_b X_b.
__device__ __forceinline__ void group_mac_q8(const uint4 c0, const uint4 c1, uint32_t sbw, const uint16_t* ap,
                                             const float* xs_g, int G2, int half, int nquads, float yacc[16]) {
  f32x16 acc[2];
  q8_products(c0, c1, ap, acc);
  const float d[2] = {half_bits_to_f32(sbw & 0xFFFFu), half_bits_to_f32(sbw >> 16)};
  const float c[2] = {-128.0f * d[0], -128.0f * d[1]};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (q < nquads) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = 4 * q + r;
        const float* xg = xs_g + (8 * q + 4 * half + r) * G2;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          yacc[v] = fmaf(d[b], acc[b][v], yacc[v]);
          yacc[v] = fmaf(c[b], xg[b], yacc[v]);
        }
      }
    }
  }
}

// group_mac_rows for a Q8_0 group: xr[i] points at the block sums of the row
// behind y[i] (two per group: xr[i][2 s_idx + b]).
template <int ACT>
__device__ __forceinline__ void group_mac_rows_q8(const uint4 c0, const uint4 c1, uint32_t sbw, const uint16_t* ap,
                                                  const float* const (&xr)[5], int s_idx, float y[5]) {
  f32x16 acc[2];
  q8_products(c0, c1, ap, acc);
  const float d[2] = {half_bits_to_f32(sbw & 0xFFFFu), half_bits_to_f32(sbw >> 16)};
  const float c[2] = {-128.0f * d[0], -128.0f * d[1]};
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    float t[5];
    if (ACT == SDV_ACT_BF16) {
#pragma unroll
      for (int i = 0; i < 5; ++i) t[i] = acc[b][i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) t[i] = (acc[b][i] + acc[b][4 + i]) + acc[b][8 + i];
      t[4] = (acc[b][12] + acc[b][13]) + acc[b][14];
    }
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      y[i] = fmaf(d[b], t[i], y[i]);
      y[i] = fmaf(c[b], xr[i][2 * s_idx + b], y[i]);
    }
  }
}

// Row r's value from group_mac_rows accumulators (valid in half (r / 4) % 2
// for r < 8, in half 0 for r = 8).
__device__ __forceinline__ float rows_value(const float y[5], int r) { return r < 8 ? y[r & 3] : y[4]; }

__device__ __forceinline__ int rows_half(int r) { return r < 8 ? (r >> 2) & 1 : 0; }

// Final value of activation row i from the wave's accumulators (valid in the
// lanes of half (vrow/4)%2).
template <int ACT>
__device__ __forceinline__ float row_value(const float yacc[16], int i) {
  if (ACT == SDV_ACT_BF16) {
    const int v = reg_of(i);
    float r = 0.0f;
#pragma unroll
    for (int t = 0; t < 16; ++t)
      if (t == v) r = yacc[t];
    return r;
  }
  float p[3];
#pragma unroll
  for (int pp = 0; pp < 3; ++pp) {
    const int v = reg_of(vrow_of<ACT>(i, pp));
    float r = 0.0f;
#pragma unroll
    for (int t = 0; t < 16; ++t)
      if (t == v) r = yacc[t];
    p[pp] = r;
  }
  return (p[0] + p[1]) + p[2];
}

template <int ACT>
__device__ __forceinline__ int half_of_row(int i) {
  return (vrow_of<ACT>(i, 0) >> 2) & 1;
}

}  // namespace q4
}  // namespace sdv
