/*
 * sdv.h -- C ABI of libsdv: exact k-row speculative-verification kernels for
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes one verification step of a Gated-DeltaNet / MoE
 * hybrid layer for k = 1..SDV_MAX_ROWS (32) draft rows at once:
 *
 *   - affine-Q4 (group 64, bf16 scale and bias) multi-row matvec that decodes
 *     each packed weight once for all k rows, dense and gathered-expert
 *     (top-k of E experts, fused gate/up with SwiGLU) -- the exact multi-row
 *     projection and gathered-expert kernels of the mere.run transfer report
 *     ("Flash-Next optimization transfer to Ornith and Qwen 27B", sections
 *     "Shared architecture and implemented paths" and "Exact verification
 *     kernels and benchmark admission") and Red Lite dev45's two-vector
 *     kernels, router dispatch and merged experts ("What it is");
 *   - the multi-row Gated DeltaNet delta-rule recurrence on an fp32
 *     [Hv, Dv, Dk] state with a snapshot after every row, and rollback to the
 *     accepted prefix by selecting a snapshot (Flash-Next plan QWEN38FLASH.md,
 *     "2.1 Gated DeltaNet"; Red Lite dev45, "What it is": in-kernel snapshots
 *     and rejection by choosing which state buffer is live, with no copy).
 *
 * Conventions for every entry point
 *   - Return value: SDV_OK (0) or a negative SDV_E* status.  Arguments are
 *     validated on the host before any launch; on error nothing is launched
 *     and no device memory is written.  sdv_last_error() gives a message for
 *     the calling thread's most recent failure.
 *   - Pointers named "device" are device memory owned by the caller; the
 *     library never allocates or frees device memory and keeps no pointer
 *     after a call returns.  Device pointers must be 16-byte aligned.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *     the default stream).  Results are visible after the stream reaches the
 *     call.  Calls are reentrant; two calls whose outputs overlap race.
 *   - Row width k must be 1..SDV_MAX_ROWS (32): the widths 1-9 of the dense and
 *     MoE checkpoints and the widths 1, 4, 8, 16, 32 of the Flash-Next verifier.
 *   - Every row of a width-k call is bit-identical to the same row computed
 *     by a width-1 call (fixed per-output reduction order, independent of k
 *     and of which other rows share an expert).
 *   - bf16 values are passed as their uint16_t bit patterns.
 *   - Weights: the products (sdv_qmv_k, sdv_gather_qmv_k, sdv_moe_experts_k and
 *     the calls built on them) read only the tiled sdv_q4t layout, written once
 *     per weight by sdv_q4_repack (sdv_q8_0_repack, sdv_q3_repack for the other
 *     formats).  The row-major sdv_q4 is the interchange form those repacks
 *     read.  In the tiled layout one matrix-core step of a wave reads one
 *     contiguous 1 KB block of codes plus one 128-byte line holding the 32
 *     rows' scales and biases; the row-major form would need 32 scattered rows
 *     and 64 scattered 2-byte loads per step, which measured 2.4-3.8x slower.
 */
#ifndef SDV_H
#define SDV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef SDV_API
#define SDV_API __attribute__((visibility("default")))
#endif

typedef void *sdv_stream_t; /* hipStream_t */

/* status codes */
#define SDV_OK 0
#define SDV_EINVAL (-1)  /* null pointer, bad shape or count, misaligned pointer */
#define SDV_EWIDTH (-2)  /* k outside 1..SDV_MAX_ROWS */
#define SDV_ELAYOUT (-3) /* group != 64, K % 64 != 0, unsupported head dim or fused layout */
#define SDV_ERANGE (-4)  /* accepted prefix outside 0..k, topk outside 1..min(E,16), E > 1024 */
#define SDV_EALIAS (-5)  /* an output overlaps an input or another output */
#define SDV_EHIP (-6)    /* the HIP runtime reported an error at launch */

#define SDV_MAX_ROWS 32
#define SDV_GROUP 64
#define SDV_MAX_EXPERTS 1024
#define SDV_MAX_TOPK 16

/* product modes */
#define SDV_MODE_PLAIN 0         /* y[r, n] = W[n, :] . a[r, :] */
#define SDV_MODE_GATEUP_SWIGLU 1 /* W rows [0, N/2) gate, [N/2, N) up: y[r, i] = silu(gate_i) * up_i */

/* activation types */
#define SDV_ACT_BF16 0 /* bf16 bits */
#define SDV_ACT_F32 1  /* fp32 */

/* router score functions */
#define SDV_ROUTE_SOFTMAX 0 /* softmax over all E logits */
#define SDV_ROUTE_SIGMOID 1 /* independent sigmoid per logit */

/* Activation after the GDN input conv (sdv_gdn_prepare_k). */
#define SDV_CONV_NONE 0
#define SDV_CONV_SILU 1

/* Gate activation of the GDN output norm (sdv_gdn_gated_norm_k). */
#define SDV_GATE_SIGMOID 0
#define SDV_GATE_SILU 1

/*
 * An affine-Q4, group-64 weight in row-major interchange layout: E matrices of
 * N rows by K inputs.
 *   codes  [E][N][K/8] uint32: element 8w+i of a row in bits [4i, 4i+4) of word w,
 *          an unsigned code q in 0..15
 *   scales [E][N][K/64] bf16, biases [E][N][K/64] bf16
 *   value  W[e][n][c] = scales[e][n][c/64] * q + biases[e][n][c/64]
 * E = 1 is a dense matrix.  group must be 64 and K a positive multiple of 64.
 * (mere.run transfer report, "Shared architecture and implemented paths":
 * affine Q4, group size 64, compatible bf16 tensors; the nibble order is this
 * library's definition.)  The products read the tiled layout below, written
 * once per weight by sdv_q4_repack.
 */
typedef struct sdv_q4 {
  const uint32_t *codes;
  const uint16_t *scales;
  const uint16_t *biases;
  int32_t E, N, K, group;
} sdv_q4;

/*
 * The same weight in the tiled layout the kernels stream (written by
 * sdv_q4_repack).  Columns are grouped into T tiles of 32 weight rows:
 *   fused_gateup = 0: tile t holds rows 32t .. 32t+31 (T = ceil(N/32));
 *   fused_gateup = 1: the rows are [gate; up] halves of N/2 each, and tile t
 *     holds gate rows 16t .. 16t+15 then up rows N/2+16t .. (T = ceil(N/32)).
 *   codes  [E][T][K/64][64][16 bytes]: for tile t and group g, 16-byte chunk
 *          l = 32h + c holds words 4h .. 4h+3 of group g of the tile's row c;
 *   sb     [E][T][K/64][32] uint32: scale bits | bias bits << 16 of row c.
 * Padding rows (past N) are zero.  Sizes: sdv_q4t_codes_bytes / sdv_q4t_sb_bytes.
 */
typedef struct sdv_q4t {
  const void *codes;
  const uint32_t *sb;
  int32_t E, N, K, group;
  int32_t fused_gateup;
  int32_t format; /* SDV_FMT_AFFINE_Q4 (0, the layout above), SDV_FMT_Q8_0 or SDV_FMT_AFFINE_Q3 (below) */
} sdv_q4t;

/* Formats of a tiled weight (sdv_q4t.format). */
#define SDV_FMT_AFFINE_Q4 0
#define SDV_FMT_Q8_0 1
#define SDV_FMT_AFFINE_Q3 2

/*
 * An affine-Q3, group-64 weight in row-major interchange layout (mere.run
 * transfer report, "Shared architecture and implemented paths": the gathered
 * expert kernel's Q3 specialization beside affine Q4/g64; the bit packing is
 * this library's definition):
 *   codes  [E][N][3K/8] bytes: element c of a row is bits [3c, 3c+3) of the
 *          row's little-endian bit stream, an unsigned code q in 0..7
 *   scales, biases  [E][N][K/64] bf16;  value = scales * q + biases per group
 * The tiled form (sdv_q3_repack; format = SDV_FMT_AFFINE_Q3) keeps the Q4
 * tiles and sb words; codes [E][T][K/64][3][64] uint32: for tile t and group
 * g, the three words w of chunk l = 32h + c hold the tile's row c, elements
 * 32h + 8j + i (step j, i < 8), as code pairs P = 4j + i (i < 4): element i
 * at bits 3 (P % 5) .. +2 of word P / 5 and element i + 4 sixteen bits
 * higher for P < 15; for P = 15, bit b of element i in bit 15 of word b and
 * of element i + 4 in bit 31.  Sizes: sdv_q3t_codes_bytes; sdv_q4t_sb_bytes.
 */
typedef struct sdv_q3 {
  const uint8_t *codes;
  const uint16_t *scales;
  const uint16_t *biases;
  int32_t E, N, K;
} sdv_q3;

SDV_API size_t sdv_q3t_codes_bytes(int E, int N, int K, int fused_gateup);

/* sdv_q3_repack -- as sdv_q4_repack for an affine-Q3 weight.  Errors: EINVAL, ELAYOUT, EALIAS, EHIP. */
SDV_API int sdv_q3_repack(const sdv_q3 *src, int fused_gateup, void *codes_out, uint32_t *sb_out,
                          sdv_stream_t stream);

/*
 * A Q8_0 weight in row-major interchange layout (the GGUF Q8_0 block: 32
 * signed 8-bit codes sharing one IEEE half scale; Red Lite dev45, "What it
 * is": the MTP block's Q8_0 experts; mere.run transfer report, "Shared
 * architecture and implemented paths": Q8 router and shared-gate weights).
 *   qs  [E][N][K] int8 codes q;  d  [E][N][K/32] binary16 scale bits
 *   value  W[e][n][c] = d[e][n][c/32] * q[e][n][c]
 * K must be a positive multiple of 64 (the tiled group).
 */
typedef struct sdv_q8_0 {
  const int8_t *qs;
  const uint16_t *d;
  int32_t E, N, K;
} sdv_q8_0;

/*
 * The tiled Q8_0 layout (format = SDV_FMT_Q8_0, written by sdv_q8_0_repack),
 * tiles as above:
 *   codes  [E][T][K/64][2][64][16 bytes]: for tile t, group g and half p,
 *          chunk l = 32h + c holds the bytes u = q + 128 of elements
 *          32p + 8h + i (words 0, 1: i = 0..3, 4..7) and 32p + 16 + 8h + i
 *          (words 2, 3) of the group, of the tile's row c;
 *   sb     [E][T][K/64][32] uint32: half scale bits of block 2g | block 2g + 1 << 16.
 * Sizes: sdv_q8_0t_codes_bytes; sdv_q4t_sb_bytes.
 */
SDV_API size_t sdv_q8_0t_codes_bytes(int E, int N, int K, int fused_gateup);

/*
 * sdv_q8_0_repack -- rewrite a row-major Q8_0 weight into the tiled layout
 * (device to device, on `stream`); fused_gateup as for sdv_q4_repack.
 *   codes_out  device, sdv_q8_0t_codes_bytes(...) bytes; sb_out device, sdv_q4t_sb_bytes(...)
 * Errors: EINVAL, ELAYOUT, EALIAS, EHIP.
 */
SDV_API int sdv_q8_0_repack(const sdv_q8_0 *src, int fused_gateup, void *codes_out, uint32_t *sb_out,
                            sdv_stream_t stream);

/* Bytes of the tiled codes / scale-bias arrays of an E x N x K weight. */
SDV_API size_t sdv_q4t_codes_bytes(int E, int N, int K, int fused_gateup);
SDV_API size_t sdv_q4t_sb_bytes(int E, int N, int K, int fused_gateup);

/*
 * sdv_q4_repack -- rewrite a row-major weight into the tiled layout (device to
 * device, on `stream`).  fused_gateup = 1 pairs row i of the first half with
 * row N/2 + i in one tile (N must be even) for SDV_MODE_GATEUP_SWIGLU.
 *   src        row-major descriptor (device arrays)
 *   codes_out  device, sdv_q4t_codes_bytes(...) bytes; sb_out device, sdv_q4t_sb_bytes(...)
 * Errors: EINVAL, ELAYOUT, EALIAS, EHIP.
 */
SDV_API int sdv_q4_repack(const sdv_q4 *src, int fused_gateup, void *codes_out, uint32_t *sb_out,
                          sdv_stream_t stream);

/*
 * sdv_qmv_k -- dense multi-row affine-Q4 matvec (E must be 1).
 * The width-k product decodes each weight once for all k rows; each row
 * equals the width-1 result bit for bit (mere.run report, "Exact verification
 * kernels and benchmark admission": the few-row Q4 product agrees bit for bit
 * with one-row products at widths 4, 8 and 9; Red Lite dev45 "What it is": one
 * decode of the weights serves every row, each row summed in the one-row
 * kernel's order).
 *   W         tiled weight descriptor (host struct, device arrays)
 *   act       device, [k][K]: bf16 bits (act_dtype SDV_ACT_BF16) or fp32 (SDV_ACT_F32)
 *   k         rows, 1..SDV_MAX_ROWS
 *   mode      SDV_MODE_PLAIN: y [k][N], needs fused_gateup = 0;
 *             SDV_MODE_GATEUP_SWIGLU: y [k][N/2], needs fused_gateup = 1
 *   y         device fp32 output
 * Errors: EINVAL, EWIDTH, ELAYOUT (also a mode that does not match the layout), EALIAS, EHIP.
 */
SDV_API int sdv_qmv_k(const sdv_q4t *W, const void *act, int act_dtype, int k, int mode, float *y,
                      sdv_stream_t stream);

/*
 * sdv_qmv_k_multi -- sdv_qmv_k for nw weights (1..16) of one shape, format
 * and layout that read the same activation rows, in one launch: for example
 * the projections of a layer that share their input.  W is a host array of
 * nw tiled descriptors (E = 1), y a host array of nw device outputs (each
 * as sdv_qmv_k's y).  Each output equals the separate sdv_qmv_k call's bit
 * for bit: the launch only places the weights' tiles side by side in one
 * grid (more workgroups to fill the chip, one launch ramp for all).
 * Errors: those of sdv_qmv_k; ERANGE for nw outside 1..16; ELAYOUT when a
 * weight differs from W[0] in shape, format or layout.
 */
SDV_API int sdv_qmv_k_multi(const sdv_q4t *W, int nw, const void *act, int act_dtype, int k, int mode,
                            float *const *y, sdv_stream_t stream);

/*
 * sdv_moe_route_k -- one router dispatch for all k rows: per-row top-k, the
 * routing weights, the union of the rows' experts and the (expert, row, slot)
 * pairs, all on the device with no host synchronisation (Red Lite dev45,
 * "What it is": one router dispatch for both rows; "Scope boundary": the
 * union of the rows' experts; Flash-Next plan "2.3 MoE": top-10 of 512).
 *   logits     device fp32 [k][E]
 *   score_mode SDV_ROUTE_SOFTMAX (over all E) or SDV_ROUTE_SIGMOID
 *   renorm     nonzero: weights divided by their sum over the row's top-k
 *   idx        device int32 [k][topk]: experts by logit descending, ties to the lower index
 *   w          device fp32 [k][topk]: weight of each slot
 *   union_ids  device int32 [k*topk]: distinct experts ascending (first n_union valid)
 *   n_union    device int32 [1]
 *   pair_off   device int32 [k*topk + 1]: pairs of union entry u are [pair_off[u], pair_off[u+1])
 *   pair_row, pair_slot  device int32 [k*topk]: ordered by (expert, row) ascending
 * E in topk..1024, topk in 1..16.  NaN logits are never preferred to a number;
 * a slot left with no candidate (all remaining logits NaN) gets idx -1 and no
 * pair, so every written index and pair stays in range.
 * Errors: EINVAL, EWIDTH, ERANGE, EALIAS, EHIP.
 */
SDV_API int sdv_moe_route_k(const float *logits, int k, int E, int topk, int score_mode, int renorm,
                    int32_t *idx, float *w, int32_t *union_ids, int32_t *n_union,
                    int32_t *pair_off, int32_t *pair_row, int32_t *pair_slot,
                    sdv_stream_t stream);

/*
 * sdv_gather_qmv_k -- multi-row affine-Q4 product over the union of the rows'
 * experts: each union expert's weights are decoded once for all rows routed
 * to it (mere.run report, "Exact verification kernels and benchmark
 * admission": gathered expert kernel, affine Q4/group 64, widths 2..9, fused
 * gate/up weights, unsupported layouts rejected; Red Lite dev45, "What it is":
 * all (expert, row) pairs of the union go out in one dispatch, gate and up
 * read together).
 *   bank       tiled weight descriptor, E experts of [N][K]
 *   mode       SDV_MODE_GATEUP_SWIGLU (fused [gate; up] rows, output N/2; needs
 *              fused_gateup = 1) or SDV_MODE_PLAIN (needs fused_gateup = 0)
 *   act        device: SDV_ACT_BF16 shared rows [k][K] (row r's input for every slot),
 *              or SDV_ACT_F32 per pair [k][topk][K] (e.g. the SwiGLU output)
 *   union_ids, n_union, pair_off, pair_row, pair_slot  device, as written by sdv_moe_route_k
 *   out        device fp32 [k][topk][N or N/2]; entry (r, s) holds expert idx[r][s]'s output
 *   shared     optional always-on expert (Flash-Next plan "2.3 MoE": one shared
 *              expert beside the routed ones): a tiled descriptor with E = 1 and
 *              the bank's N, K and fused_gateup, applied to all k rows in the same
 *              launch; NULL for none (then shared_act and shared_out must be NULL)
 *   shared_act device, the shared expert's rows [k][K] in act_dtype
 *   shared_out device fp32 [k][N or N/2]
 * The grid covers k*topk union entries (plus one for the shared expert) and
 * entries past n_union exit; expert ids, rows and slots outside their ranges
 * are skipped on the device.
 * Errors: EINVAL, EWIDTH, ELAYOUT, ERANGE, EALIAS, EHIP.
 */
SDV_API int sdv_gather_qmv_k(const sdv_q4t *bank, int mode, const void *act, int act_dtype,
                     const int32_t *union_ids, const int32_t *n_union, const int32_t *pair_off,
                     const int32_t *pair_row, const int32_t *pair_slot, int k, int topk,
                     float *out, const sdv_q4t *shared, const void *shared_act,
                     float *shared_out, sdv_stream_t stream);

/*
 * sdv_moe_experts_k -- the union experts' whole MLP in one launch: fused
 * gate/up with SwiGLU, then the down projection, each union expert's packed
 * weights read once for all rows routed to it (mere.run report, "Exact
 * verification kernels and benchmark admission": gathered expert kernel with
 * fused gate/up weights; Red Lite dev45, "What it is": one dispatch for all
 * of the union's (expert, row) pairs, gate and up read together; Flash-Next
 * plan "2.3 MoE": top-10 of 512 plus one shared expert).  The intermediate
 * dimension is cut into S = ceil(I / 128) slices; workgroup (expert, slice)
 * computes h = silu(gate) * up for its slice and multiplies it by the matching
 * K slice of the down weight, so for slot (r, s) of row r
 *   sum_{j = 0..S-1, ascending} partial[j][r][s] = down_e(silu(gate_e x_r) * up_e x_r)
 * with e = idx[r][s]; sdv_moe_combine_sliced_k adds the slices in that order.
 *   gate_up    tiled bank with fused_gateup = 1: E experts of [2I][H] (gate rows, then up rows)
 *   down       tiled bank with fused_gateup = 0: E experts of [H][I]
 *   x          device bf16 bits [k][H], row r's input for all of its slots
 *   union_ids, n_union, pair_off, pair_row, pair_slot  device, as written by sdv_moe_route_k
 *   shared_gate_up, shared_down  optional always-on expert (E = 1, same geometry), applied to
 *              all k rows and written to slot topk; both NULL for none
 *   partial    device fp32 [S][k][topk + 1][H] (sdv_moe_experts_partial_bytes); entries of
 *              slots without an expert, and slot topk without a shared expert, are not written
 * H and I must be multiples of 64, I at most 1024; LDS limits H (about 7000 at k = 9).
 * The four weights share one format: affine Q4, Q8_0 or affine Q3 (the
 * descriptors' format field; mixed formats are ELAYOUT).
 * Errors: EINVAL, EWIDTH, ELAYOUT, ERANGE, EALIAS, EHIP.
 */
SDV_API int sdv_moe_experts_k(const sdv_q4t *gate_up, const sdv_q4t *down, const void *x,
                              const int32_t *union_ids, const int32_t *n_union, const int32_t *pair_off,
                              const int32_t *pair_row, const int32_t *pair_slot, int k, int topk,
                              const sdv_q4t *shared_gate_up, const sdv_q4t *shared_down, float *partial,
                              sdv_stream_t stream);

/*
 * sdv_moe_route_experts_k -- sdv_moe_route_k and sdv_moe_experts_k as one
 * call (Red Lite dev45, "What it is": one router dispatch, then the union's
 * (expert, row) pairs in one dispatch).  For k <= 9 and E <= 512 it is one
 * launch: every expert workgroup runs the router dispatch itself on the
 * logits (identical results everywhere; workgroup (0, 0) writes them), so the
 * routing needs no launch of its own.  Otherwise it runs the two launches.
 * The outputs equal those of the two calls bit for bit.  Every expert
 * workgroup then waits for the whole dispatch before its first weight load:
 * at 512 experts and nine rows the two separate launches are faster.  The
 * weights must be affine Q4 (ELAYOUT otherwise: route Q8_0 and Q3 layers
 * with sdv_moe_route_k, then call sdv_moe_experts_k).
 *   logits, score_mode, renorm  as sdv_moe_route_k (E = gate_up->E)
 *   idx, w, union_ids, n_union, pair_off, pair_row, pair_slot  outputs, as sdv_moe_route_k
 *   gate_up, down, x, shared_gate_up, shared_down, partial  as sdv_moe_experts_k
 * Errors: EINVAL, EWIDTH, ELAYOUT, ERANGE, EALIAS, EHIP.
 */
SDV_API int sdv_moe_route_experts_k(const float *logits, int score_mode, int renorm, const sdv_q4t *gate_up,
                                    const sdv_q4t *down, const void *x, int k, int topk,
                                    const sdv_q4t *shared_gate_up, const sdv_q4t *shared_down, int32_t *idx,
                                    float *w, int32_t *union_ids, int32_t *n_union, int32_t *pair_off,
                                    int32_t *pair_row, int32_t *pair_slot, float *partial, sdv_stream_t stream);

/* Bytes of sdv_moe_experts_k's partial output, or 0 for invalid sizes. */
SDV_API size_t sdv_moe_experts_partial_bytes(int k, int topk, int H, int I);

/*
 * sdv_moe_combine_sliced_k -- the MoE tail over sdv_moe_experts_k's output
 * (Red Lite dev45, "What it is": one tail for all rows; Flash-Next plan "5.3
 * MoE deltas": fixed-width weighted expert sums):
 *   P[r][s][n] = sum_{j = 0..S-1, ascending} partial[j][r][s][n]
 *   y[r][n]    = sum_{s = 0..topk-1, ascending, idx[r][s] >= 0} w[r][s] * P[r][s][n]
 *                + sigmoid(shared_logit[r]) * P[r][topk][n]     (if has_shared)
 *   partial device fp32 [S][k][topk + 1][H] with S = ceil(I / 128); idx device int32 [k][topk];
 *   w device fp32 [k][topk]; shared_logit device fp32 [k] or NULL (gate 1); y device fp32 [k][H].
 * I at most 1024.  Errors: EINVAL, EWIDTH, ERANGE, EALIAS, EHIP.
 */
SDV_API int sdv_moe_combine_sliced_k(const float *partial, const int32_t *idx, const float *w,
                                     const float *shared_logit, int k, int topk, int H, int I, int has_shared,
                                     float *y, sdv_stream_t stream);

/*
 * sdv_moe_combine_k -- one MoE tail for all rows (Red Lite dev45, "What it
 * is": one tail for both rows; Flash-Next plan "5.3 MoE deltas": fixed-width
 * weighted expert sum):
 *   y[r][n] = sum_{s = 0..topk-1, ascending} w[r][s] * partial[r][s][n]
 *             + sigmoid(shared_logit[r]) * shared_out[r][n]
 * shared_out may be NULL (no shared expert); shared_logit may be NULL (gate 1).
 *   partial device fp32 [k][topk][H], w device fp32 [k][topk],
 *   shared_out device fp32 [k][H] or NULL, shared_logit device fp32 [k] or NULL,
 *   y device fp32 [k][H].
 * Errors: EINVAL, EWIDTH, ERANGE, EALIAS, EHIP.
 */
SDV_API int sdv_moe_combine_k(const float *partial, const float *w, const float *shared_out,
                      const float *shared_logit, int k, int topk, int H, float *y,
                      sdv_stream_t stream);

/*
 * sdv_gdn_verify_k -- k-row Gated DeltaNet recurrence with a state snapshot
 * after every row (Flash-Next plan, "2.1 Gated DeltaNet": decay, kv_mem,
 * delta, rank-1 update, readout on an fp32 [Hv, Dv, Dk] state; "3.1": per-head
 * scalar decay and beta, each qk head shared by Hv/Hk v heads; Red Lite
 * dev45 "What it is": row t runs from row t-1's state and the state after
 * each row is written from inside the kernel).  For t = 0..k-1, v head h,
 * qk head c = h / (Hv/Hk), value row i:
 *   S_h <- g[t][h] * S_h;  m_i = sum_j S_h[i][j] k[t][c][j];
 *   d_i = beta[t][h] * (v[t][h][i] - m_i);  S_h[i][j] += d_i * k[t][c][j];
 *   y[t][h][i] = sum_j S_h[i][j] q[t][c][j];  snaps[t] = S.
 *   S_in   device fp32 [Hv][Dv][Dk], read only (never written)
 *   q, kk  device fp32 [k][Hk][Dk];  v device fp32 [k][Hv][Dv];  g, beta device fp32 [k][Hv]
 *   y      device fp32 [k][Hv][Dv]
 *   snaps  host array of k device pointers, each an fp32 [Hv][Dv][Dk] state;
 *          they must not overlap S_in, the inputs, y or each other
 * Dk must be 64 or 128; Hv a multiple of Hk.
 * Errors: EINVAL, EWIDTH, ELAYOUT, EALIAS, EHIP.
 */
SDV_API int sdv_gdn_verify_k(const float *S_in, const float *q, const float *kk, const float *v,
                     const float *g, const float *beta, int k, int Hv, int Hk, int Dk, int Dv,
                     float *y, float *const *snaps, sdv_stream_t stream);

/*
 * sdv_gdn_rollback -- select the state for an accepted prefix of length j
 * (mere.run report: accepted-prefix rollback, every prefix at widths 4, 8, 9;
 * Red Lite dev45 "What it is": rejection picks which state buffer is live,
 * nothing is copied).  Host only, no device work:
 *   *selected_slot = 0 (the verify call's S_in) for j = 0, else j (snaps[j-1]).
 * Errors: EINVAL (null), EWIDTH, ERANGE (j outside 0..k).
 */
SDV_API int sdv_gdn_rollback(int k, int j, int *selected_slot);

/*
 * sdv_gdn_rollback_copy -- the same selection, copied into a caller-owned
 * state at a fixed address: dst <- (j == 0 ? S_in : snaps[j-1]), state_elems
 * floats, enqueued on `stream` (device-to-device).  dst may equal the selected
 * source (then nothing is copied) but may not partially overlap it.
 * Errors: EINVAL, EWIDTH, ERANGE, EALIAS, EHIP.
 */
SDV_API int sdv_gdn_rollback_copy(float *dst, const float *S_in, float *const *snaps, int k, int j,
                          size_t state_elems, sdv_stream_t stream);

/*
 * sdv_gdn_prepare_k -- the inputs of the k-row recurrence from their
 * projections (Flash-Next plan, "2.1 Gated DeltaNet": every q, k and v
 * channel is filtered along time by its own short filter that sees only the
 * current and earlier inputs, the last three inputs carried from call to
 * call; q and k are scaled to unit L2 norm per head; g comes from A_log and
 * dt_bias through softplus and exp, and beta = sigmoid(b);
 * "5.1 Gated DeltaNet": 4 taps; Red Lite dev45, "What it is": the per-row
 * conv shift, q/k norm and beta/decay kernels).
 *   qkv      device fp32 [k][C], C = 2 Hk Dk + Hv Dv, channels [q heads | k heads | v heads]
 *   hist     device fp32 [3][C]: the three inputs before row 0, oldest first
 *   conv_w   device fp32 [C][4]: tap i multiplies the input 3 - i steps before the current one
 *   a, b     device fp32 [k][Hv];  A_log, dt_bias  device fp32 [Hv]
 *   conv_act SDV_CONV_NONE or SDV_CONV_SILU (applied to the conv output)
 *   eps      >= 0: q and k are multiplied per (row, head) by rsqrt(sum of squares + eps)
 *            (the device reciprocal square root, within 2 ulp of 1 / sqrt)
 *   q, kk    device fp32 [k][Hk][Dk] out;  v  device fp32 [k][Hv][Dv] out
 *   g, beta  device fp32 [k][Hv] out: g = exp(-exp(A_log) softplus(a + dt_bias)), beta = sigmoid(b)
 *   window   device fp32 [k + 3][C] out: [hist; qkv].  The conv history after an
 *            accepted prefix of j rows (0..k) is window + j C (rollback by
 *            selection); the next call takes it as `hist` and writes another window.
 * Dk = Dv in {64, 128}; Hv a multiple of Hk.  Each row is computed in the same order
 * at every width.  Errors: EINVAL, EWIDTH, ELAYOUT, ERANGE (eps), EALIAS, EHIP.
 */
SDV_API int sdv_gdn_prepare_k(const float *qkv, const float *hist, const float *conv_w, const float *a,
                              const float *b, const float *A_log, const float *dt_bias, int k, int Hv, int Hk,
                              int Dk, int Dv, int conv_act, float eps, float *q, float *kk, float *v, float *g,
                              float *beta, float *window, sdv_stream_t stream);

/*
 * sdv_gdn_verify_prep_k -- sdv_gdn_prepare_k and sdv_gdn_verify_k in one
 * launch (Flash-Next plan, "2.1 Gated DeltaNet": the conv, q/k norm and gates
 * feed the recurrence; Red Lite dev45, "What it is": the per-row preparation
 * kernels ahead of the state kernel).  Each workgroup prepares the inputs of
 * its own value rows; y, the snapshots and the window equal those of the two
 * separate calls bit for bit.  The prepared q, k, v, g, beta are not written.
 *   S_in, snaps, y  as sdv_gdn_verify_k;  qkv, hist, conv_w, a, b, A_log, dt_bias,
 *   conv_act, eps, window  as sdv_gdn_prepare_k.
 * Dk = Dv in {64, 128}; Hv a multiple of Hk.  No output may overlap an input or
 * another output.  Errors: EINVAL, EWIDTH, ELAYOUT, ERANGE (eps), EALIAS, EHIP.
 */
SDV_API int sdv_gdn_verify_prep_k(const float *S_in, const float *qkv, const float *hist, const float *conv_w,
                                  const float *a, const float *b, const float *A_log, const float *dt_bias, int k,
                                  int Hv, int Hk, int Dk, int Dv, int conv_act, float eps, float *window, float *y,
                                  float *const *snaps, sdv_stream_t stream);

/*
 * sdv_gdn_layer -- one layer's buffers for sdv_gdn_verify_prep_k_layers: the
 * pointer arguments of one sdv_gdn_verify_prep_k call, with the same meaning
 * and sizes (snaps[0..k-1] are used).
 */
typedef struct sdv_gdn_layer {
  const float *S_in, *qkv, *hist, *conv_w, *a, *b, *A_log, *dt_bias;
  float *window, *y;
  float *snaps[SDV_MAX_ROWS];
} sdv_gdn_layer;

/*
 * sdv_gdn_layers_table -- check L layers for sdv_gdn_verify_prep_k_layers and
 * copy them into a caller-owned device table (a blocking copy).
 *   layers       host array [L], 1 <= L <= 65535: each layer is checked as
 *                sdv_gdn_verify_prep_k checks its pointers, and no output of any
 *                layer (y, window, snaps) may overlap an input or output of any
 *                layer, or the table
 *   k, Hv, Hk, Dk, Dv  the layers' shape, as sdv_gdn_verify_prep_k
 *   table        device buffer, 16-byte aligned, of at least
 *                L * sizeof(sdv_gdn_layer) = table_bytes
 * Errors: EINVAL, EWIDTH, ELAYOUT, EALIAS, EHIP.
 */
SDV_API int sdv_gdn_layers_table(const sdv_gdn_layer *layers, int L, int k, int Hv, int Hk, int Dk, int Dv,
                                 void *table, size_t table_bytes);

/*
 * sdv_gdn_verify_prep_k_layers -- sdv_gdn_verify_prep_k over L independent
 * layers of one shape in one launch: a measurement form, which shows the
 * recurrence's bandwidth without the ramp of each launch (Flash-Next plan,
 * "2.1 Gated DeltaNet").  In a model each layer's input depends on the layer
 * before, so layers run one sdv_gdn_verify_prep_k call each.  Every layer's y,
 * snapshots and window equal its own sdv_gdn_verify_prep_k call's bit for bit.
 *   table    device table written by sdv_gdn_layers_table with the same L, k,
 *            Hv, Hk, Dk, Dv (its pointers are not checked again)
 *   conv_act, eps  as sdv_gdn_verify_prep_k, for every layer
 * Errors: EINVAL, EWIDTH, ELAYOUT, ERANGE (eps), EHIP.
 */
SDV_API int sdv_gdn_verify_prep_k_layers(const void *table, int L, int k, int Hv, int Hk, int Dk, int Dv,
                                         int conv_act, float eps, sdv_stream_t stream);

/*
 * sdv_gdn_gated_norm_k -- the GDN output before its projection (Flash-Next plan,
 * "2.1 Gated DeltaNet": y scaled by its reciprocal RMS, times act(gate); "5.1": sigmoid gate
 * for this model; Red Lite dev45 "What it is": the tail norm).
 *   y, z     device fp32 [k][Hv][Dv]: the recurrence output and the gate projection
 *   w        device fp32 [Dv]: the norm weight
 *   gate_act SDV_GATE_SIGMOID or SDV_GATE_SILU
 *   out      device fp32 [k][Hv][Dv] = y / sqrt(mean_Dv(y^2) + eps) * w * act(z)
 * Dv in {64, 128}.  Errors: EINVAL, EWIDTH, ELAYOUT, ERANGE (eps), EALIAS, EHIP.
 */
SDV_API int sdv_gdn_gated_norm_k(const float *y, const float *z, const float *w, int k, int Hv, int Dv,
                                 int gate_act, float eps, float *out, sdv_stream_t stream);

/*
 * sdv_gdn_verify_prep_norm_k -- sdv_gdn_verify_prep_k and sdv_gdn_gated_norm_k
 * in one launch (Flash-Next plan, "2.1 Gated DeltaNet": preparation,
 * recurrence and the gated RMSNorm tail of one layer).  The last of each
 * head's workgroups to finish applies that head's norm; y, the
 * snapshots, the window and out equal those of the two separate calls bit
 * for bit.  A workgroup counts itself in only after all of its stores have
 * completed, snapshots included, so at the 48-head layer shape the two
 * separate launches are faster.
 *   S_in ... snaps  as sdv_gdn_verify_prep_k (y is still written);
 *   z, norm_w, gate_act, norm_eps, out  as sdv_gdn_gated_norm_k's z, w,
 *   gate_act, eps, out;
 *   counters  device int32 [Hv], owned by the caller: all zero before the
 *             first call, and every completed call leaves them zero.
 *             Calls that overlap in time must not share counters.
 * Dk = Dv in {64, 128}.  No output may overlap an input or another output.
 * Errors: EINVAL, EWIDTH, ELAYOUT, ERANGE (eps, norm_eps), EALIAS, EHIP.
 */
SDV_API int sdv_gdn_verify_prep_norm_k(const float *S_in, const float *qkv, const float *hist, const float *conv_w,
                                       const float *a, const float *b, const float *A_log, const float *dt_bias,
                                       int k, int Hv, int Hk, int Dk, int Dv, int conv_act, float eps,
                                       float *window, float *y, float *const *snaps, const float *z,
                                       const float *norm_w, int gate_act, float norm_eps, float *out,
                                       int32_t *counters, sdv_stream_t stream);

/*
 * sdv_verify_accept_workspace_bytes -- device workspace needed by
 * sdv_verify_accept_k for k rows of V logits (0 for k outside 1..SDV_MAX_ROWS
 * or V < 1).
 */
SDV_API size_t sdv_verify_accept_workspace_bytes(int k, int V);

/*
 * sdv_verify_accept_k -- acceptance of a verified block: the token sampled from
 * each row and the number of leading drafts accepted (Red Lite dev45,
 * "Acceptance": draft t stands when it equals the token sampled from row
 * t-1's logits, so the output distribution is that of plain decoding for any
 * sampler; dev45b: a draft that matches the end-of-answer token is refused, so
 * that token never enters the state).
 *   logits    device fp32 [k][V]: row t's next-token logits (row 0 follows the
 *             pending token, row t > 0 follows draft t)
 *   noise     device fp32 [k][V] Gumbel(0, 1) noise, or NULL for greedy
 *   inv_temp  1 / temperature (used with noise): a row's scores are
 *             fp32(fp32(logits * inv_temp) + noise), each operation rounded
 *   drafts    device int32 [k - 1]: the tokens of rows 1..k-1 (NULL allowed for k = 1)
 *   eos       end-of-answer token id, or -1 for none
 *   tokens    device int32 [k] out: row t's sample = the index of its largest
 *             score, ties to the lower index; NaN scores never win; -1 if a row
 *             has no number
 *   accepted  device int32 [1] out: n in 0..k-1, the count of leading drafts
 *             that equal the token sampled from the previous row and are not
 *             eos.  Rows 0..n stay in the state (sdv_gdn_rollback with j = n + 1)
 *             and tokens[0..n] are emitted, tokens[n] becoming the next pending token.
 *   workspace device, at least sdv_verify_accept_workspace_bytes(k, V) bytes,
 *             overwritten (scratch between the call's two launches)
 * Results are exact (integer keys), independent of launch shape.
 * Errors: EINVAL (null, misaligned, workspace too small), EWIDTH, ERANGE (V outside
 * 1..2^30, or inv_temp not finite and positive when noise is given), EALIAS, EHIP.
 */
SDV_API int sdv_verify_accept_k(const float *logits, const float *noise, float inv_temp, const int32_t *drafts,
                                int k, int V, int eos, int32_t *tokens, int32_t *accepted, void *workspace,
                                size_t workspace_bytes, sdv_stream_t stream);

/*
 * sdv_verify_accept_k_noalloc -- sdv_verify_accept_k without a caller
 * workspace and without any allocation, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is a file-scope device
 * array of sdv_verify_accept_scratch_bytes() bytes (1 MiB), one per GPU,
 * held until the process ends; its address on a device is looked up once,
 * on that device's first call.  Arguments, results and errors are those of
 * sdv_verify_accept_k; in addition, sizes whose workspace
 * (sdv_verify_accept_workspace_bytes(k, V)) exceeds the scratch are
 * rejected with SDV_ERANGE before any launch: with 4,096-logit chunks,
 * k * ceil(V / 4096) <= 131072 (every width at a 16.7M-token vocabulary).
 * The scratch keeps the last call's contents and needs no clearing (each
 * call writes every entry it reads).  Calls that overlap in time on one GPU
 * share the array and race: serialise them (one stream, or events).
 */
SDV_API int sdv_verify_accept_k_noalloc(const float *logits, const float *noise, float inv_temp,
                                        const int32_t *drafts, int k, int V, int eos, int32_t *tokens,
                                        int32_t *accepted, sdv_stream_t stream);

/* Bytes of the built-in scratch of sdv_verify_accept_k_noalloc. */
SDV_API size_t sdv_verify_accept_scratch_bytes(void);

/* Static text for a status code. */
SDV_API const char *sdv_status_string(int status);

/* Message describing the calling thread's most recent failed call ("" if none). */
SDV_API const char *sdv_last_error(void);

/* Library version and build target, e.g. "sdv 0.1 gfx950". */
SDV_API const char *sdv_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* SDV_H */
