// C ABI of libsdv: argument validation (host only, before any launch) and
// dispatch to the kernels.  Declarations and contracts: include/sdv.h.

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "common.h"

namespace sdv {
hipError_t q4_launch(const sdv_q4t& W, int mode, const void* act, int act_dtype, bool gather,
                     const int32_t* union_ids, const int32_t* n_union, const int32_t* pair_off,
                     const int32_t* pair_row, const int32_t* pair_slot, int k, int topk, float* out,
                     const sdv_q4t* shared, const void* shared_act, float* shared_out, hipStream_t st);
size_t q4_lds_bytes_for(int K, int act_dtype, int k, bool gather, int fmt);
size_t q4t_codes_bytes(int E, int N, int K, int fused);
size_t q8_0t_codes_bytes(int E, int N, int K, int fused);
size_t q3t_codes_bytes(int E, int N, int K, int fused);
hipError_t q3_repack_launch(const sdv_q3& src, int fused, void* tcodes, uint32_t* tsb, hipStream_t st);
hipError_t q8_0_repack_launch(const sdv_q8_0& src, int fused, void* tcodes, uint32_t* tsb, hipStream_t st);
size_t q4t_sb_bytes(int E, int N, int K, int fused);
hipError_t q4_repack_launch(const sdv_q4& src, int fused, void* tcodes, uint32_t* tsb, hipStream_t st);
hipError_t route_launch(const float* logits, int k, int E, int topk, int mode, int renorm,
                        int32_t* idx, float* w, int32_t* union_ids, int32_t* n_union,
                        int32_t* pair_off, int32_t* pair_row, int32_t* pair_slot, hipStream_t st);
hipError_t combine_launch(const float* partial, const float* w, const float* shared_out,
                          const float* shared_logit, int k, int topk, int H, float* y,
                          hipStream_t st);
hipError_t combine_sliced_launch(const float* partial, const int32_t* idx, const float* w,
                                 const float* shared_logit, int S, int k, int topk, int H, int has_shared,
                                 float* y, hipStream_t st);
int expert_slices(int I);
size_t expert_lds_bytes(int k, int H, int fmt);
size_t expert_partial_bytes(int k, int topk, int H, int I);
bool route_in_experts(int k, int E);
size_t route_experts_lds_bytes(int k, int E, int H);
hipError_t moe_route_experts_launch(const float* logits, int mode, int renorm, const sdv_q4t& gu,
                                    const sdv_q4t& dn, const sdv_q4t* sgu, const sdv_q4t* sdn, const void* x, int k,
                                    int topk, int32_t* idx, float* w, int32_t* union_ids, int32_t* n_union,
                                    int32_t* pair_off, int32_t* pair_row, int32_t* pair_slot, float* partial,
                                    hipStream_t st);
hipError_t moe_experts_launch(const sdv_q4t& gu, const sdv_q4t& dn, const sdv_q4t* sgu, const sdv_q4t* sdn,
                              const void* x, const int32_t* union_ids, const int32_t* n_union,
                              const int32_t* pair_off, const int32_t* pair_row, const int32_t* pair_slot, int k,
                              int topk, float* partial, hipStream_t st);
hipError_t gdn_prepare_launch(const float* qkv, const float* hist, const float* conv_w, const float* ga,
                              const float* gb, const float* A_log, const float* dt_bias, int k, int Hv, int Hk,
                              int Dk, int Dv, int conv_act, float eps, float* q, float* kk, float* v, float* g,
                              float* beta, float* window, hipStream_t st);
hipError_t gdn_gated_norm_launch(const float* y, const float* z, const float* w, int k, int Hv, int Dv,
                                 int gate_act, float eps, float* out, hipStream_t st);
size_t accept_workspace_bytes(int k, int V);
hipError_t accept_launch(const float* logits, const float* noise, float inv_temp, const int32_t* drafts, int k,
                         int V, int eos, int32_t* tokens, int32_t* accepted, void* workspace, hipStream_t st);
int dense_multi_max();
hipError_t dense_multi_launch(const sdv_q4t* Ws, int nmulti, int mode, const void* act, int act_dtype, int k,
                              float* const* outs, hipStream_t st);
size_t accept_scratch_bytes();
hipError_t accept_noalloc_launch(const float* logits, const float* noise, float inv_temp, const int32_t* drafts,
                                 int k, int V, int eos, int32_t* tokens, int32_t* accepted, hipStream_t st);
hipError_t gdn_launch(const float* S_in, const float* q, const float* kk, const float* v,
                      const float* g, const float* beta, int k, int Hv, int Hk, int Dk, int Dv,
                      float* y, float* const* snaps, hipStream_t st);
hipError_t gdn_verify_prep_layers_launch(const sdv_gdn_layer* table, int L, int k, int Hv, int Hk, int D,
                                         int conv_act, float eps, hipStream_t st);
hipError_t gdn_verify_prep_launch(const float* S_in, const float* qkv, const float* hist, const float* conv_w,
                                  const float* ga, const float* gb, const float* A_log, const float* dt_bias, int k,
                                  int Hv, int Hk, int D, int conv_act, float eps, float* window, float* y,
                                  float* const* snaps, hipStream_t st, const float* nz = nullptr,
                                  const float* nw = nullptr, int gate_act = 0, float neps = 0.0f,
                                  float* out = nullptr, int32_t* cnt = nullptr);
}  // namespace sdv

namespace {

// LDS available to one workgroup on gfx950.
constexpr size_t kMaxLds = 160 * 1024;
constexpr int kMaxExpertInter = 1024;  // fused expert path: at most 8 slices of 128

thread_local char g_err[256] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return SDV_OK;
}

// Appends to the message of the last failure.
void fail_note(const char* fmt, ...) {
  const size_t n = strlen(g_err);
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err + n, sizeof g_err - n, fmt, ap);
  va_end(ap);
}

struct Range {
  const void* p;
  size_t bytes;
  const char* name;
};

bool overlap(const Range& a, const Range& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + a.bytes;
  const uintptr_t b0 = (uintptr_t)b.p, b1 = b0 + b.bytes;
  return a0 < b1 && b0 < a1;
}

// Every output must be disjoint from every input and from the other outputs.
int check_alias(const Range* outs, int nout, const Range* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlap(outs[i], ins[j]))
        return fail(SDV_EALIAS, "output %s overlaps input %s", outs[i].name, ins[j].name);
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j]))
        return fail(SDV_EALIAS, "outputs %s and %s overlap", outs[i].name, outs[j].name);
  }
  return SDV_OK;
}

int check_ptr(const void* p, const char* name) {
  if (!p) return fail(SDV_EINVAL, "%s is NULL", name);
  if ((uintptr_t)p % 16) return fail(SDV_EINVAL, "%s is not 16-byte aligned", name);
  return SDV_OK;
}

// names of the snapshot arguments, for error messages
const char* const kSnapNames[SDV_MAX_ROWS] = {
    "snaps[0]", "snaps[1]", "snaps[2]", "snaps[3]", "snaps[4]", "snaps[5]", "snaps[6]", "snaps[7]", "snaps[8]",
    "snaps[9]", "snaps[10]", "snaps[11]", "snaps[12]", "snaps[13]", "snaps[14]", "snaps[15]", "snaps[16]",
    "snaps[17]", "snaps[18]", "snaps[19]", "snaps[20]", "snaps[21]", "snaps[22]", "snaps[23]", "snaps[24]",
    "snaps[25]", "snaps[26]", "snaps[27]", "snaps[28]", "snaps[29]", "snaps[30]", "snaps[31]"};
static_assert(SDV_MAX_ROWS == 32, "one snapshot name per row");

int check_width(int k) {
  if (k < 1 || k > SDV_MAX_ROWS) return fail(SDV_EWIDTH, "k=%d outside 1..%d", k, SDV_MAX_ROWS);
  return SDV_OK;
}

int check_q4(const sdv_q4* W, const char* what) {
  if (!W) return fail(SDV_EINVAL, "%s descriptor is NULL", what);
  if (W->group != SDV_GROUP) return fail(SDV_ELAYOUT, "%s group=%d, only 64 is supported", what, W->group);
  if (W->K <= 0 || W->K % SDV_GROUP) return fail(SDV_ELAYOUT, "%s K=%d is not a positive multiple of 64", what, W->K);
  if (W->N <= 0 || W->E <= 0) return fail(SDV_EINVAL, "%s E=%d N=%d must be positive", what, W->E, W->N);
  int st;
  if ((st = check_ptr(W->codes, "codes"))) return st;
  if ((st = check_ptr(W->scales, "scales"))) return st;
  if ((st = check_ptr(W->biases, "biases"))) return st;
  return SDV_OK;
}

size_t q4_codes_bytes(const sdv_q4& W) { return (size_t)W.E * W.N * (W.K / 8) * 4; }
size_t q4_sb_bytes(const sdv_q4& W) { return (size_t)W.E * W.N * (W.K / 64) * 2; }

int check_q4t(const sdv_q4t* W, const char* what) {
  if (!W) return fail(SDV_EINVAL, "%s descriptor is NULL", what);
  if (W->group != SDV_GROUP) return fail(SDV_ELAYOUT, "%s group=%d, only 64 is supported", what, W->group);
  if (W->K <= 0 || W->K % SDV_GROUP) return fail(SDV_ELAYOUT, "%s K=%d is not a positive multiple of 64", what, W->K);
  if (W->N <= 0 || W->E <= 0) return fail(SDV_EINVAL, "%s E=%d N=%d must be positive", what, W->E, W->N);
  if (W->fused_gateup != 0 && W->fused_gateup != 1)
    return fail(SDV_ELAYOUT, "%s fused_gateup=%d must be 0 or 1", what, W->fused_gateup);
  if (W->fused_gateup && (W->N % 2)) return fail(SDV_ELAYOUT, "%s fused gate/up needs an even N", what);
  if (W->format != SDV_FMT_AFFINE_Q4 && W->format != SDV_FMT_Q8_0 && W->format != SDV_FMT_AFFINE_Q3)
    return fail(SDV_ELAYOUT, "%s format=%d is not a known weight format", what, W->format);
  int st;
  if ((st = check_ptr(W->codes, "codes"))) return st;
  if ((st = check_ptr(W->sb, "sb"))) return st;
  return SDV_OK;
}

// The product mode must match the tile layout ("rejects unsupported layouts").
int check_mode_layout(int mode, const sdv_q4t& W) {
  if (mode == SDV_MODE_GATEUP_SWIGLU && !W.fused_gateup)
    return fail(SDV_ELAYOUT, "gate/up SwiGLU needs a weight repacked with fused_gateup=1");
  if (mode == SDV_MODE_PLAIN && W.fused_gateup)
    return fail(SDV_ELAYOUT, "a plain product needs a weight repacked with fused_gateup=0");
  return SDV_OK;
}

int check_mode(int mode, int act_dtype, int N) {
  if (mode != SDV_MODE_PLAIN && mode != SDV_MODE_GATEUP_SWIGLU)
    return fail(SDV_EINVAL, "unknown mode %d", mode);
  if (act_dtype != SDV_ACT_BF16 && act_dtype != SDV_ACT_F32)
    return fail(SDV_EINVAL, "unknown activation type %d", act_dtype);
  if (mode == SDV_MODE_GATEUP_SWIGLU && (N % 2))
    return fail(SDV_ELAYOUT, "fused gate/up needs an even N (got %d)", N);
  return SDV_OK;
}

// Tiled code bytes of a weight in its format.
size_t tiled_codes_bytes(const sdv_q4t& W) {
  if (W.format == SDV_FMT_Q8_0) return sdv::q8_0t_codes_bytes(W.E, W.N, W.K, W.fused_gateup);
  if (W.format == SDV_FMT_AFFINE_Q3) return sdv::q3t_codes_bytes(W.E, W.N, W.K, W.fused_gateup);
  return sdv::q4t_codes_bytes(W.E, W.N, W.K, W.fused_gateup);
}

int check_lds(const sdv_q4t& W, int act_dtype, int k, bool gather) {
  const int cap = act_dtype == SDV_ACT_F32 ? 3 * k : k;
  const size_t lds = sdv::q4_lds_bytes_for(W.K, act_dtype, k, gather, W.format);
  if (lds > kMaxLds)
    return fail(SDV_ELAYOUT, "K=%d with %d activation rows needs %zu bytes of LDS (max %zu)", W.K, cap,
                lds, kMaxLds);
  return SDV_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SDV_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

const char* sdv_status_string(int status) {
  switch (status) {
    case SDV_OK: return "ok";
    case SDV_EINVAL: return "invalid argument";
    case SDV_EWIDTH: return "unsupported row width";
    case SDV_ELAYOUT: return "unsupported layout";
    case SDV_ERANGE: return "value out of range";
    case SDV_EALIAS: return "output aliases another buffer";
    case SDV_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* sdv_last_error(void) { return g_err; }

const char* sdv_build_info(void) { return "sdv 0.1 gfx950"; }

size_t sdv_q4t_codes_bytes(int E, int N, int K, int fused_gateup) {
  if (E <= 0 || N <= 0 || K <= 0 || K % SDV_GROUP) return 0;
  return sdv::q4t_codes_bytes(E, N, K, fused_gateup ? 1 : 0);
}

size_t sdv_q4t_sb_bytes(int E, int N, int K, int fused_gateup) {
  if (E <= 0 || N <= 0 || K <= 0 || K % SDV_GROUP) return 0;
  return sdv::q4t_sb_bytes(E, N, K, fused_gateup ? 1 : 0);
}

int sdv_q4_repack(const sdv_q4* src, int fused_gateup, void* codes_out, uint32_t* sb_out, sdv_stream_t stream) {
  int st;
  if ((st = check_q4(src, "src"))) return st;
  if (fused_gateup != 0 && fused_gateup != 1) return fail(SDV_ELAYOUT, "fused_gateup=%d must be 0 or 1", fused_gateup);
  if (fused_gateup && (src->N % 2)) return fail(SDV_ELAYOUT, "fused gate/up needs an even N (got %d)", src->N);
  if ((st = check_ptr(codes_out, "codes_out"))) return st;
  if ((st = check_ptr(sb_out, "sb_out"))) return st;
  Range outs[] = {{codes_out, sdv::q4t_codes_bytes(src->E, src->N, src->K, fused_gateup), "codes_out"},
                  {sb_out, sdv::q4t_sb_bytes(src->E, src->N, src->K, fused_gateup), "sb_out"}};
  Range ins[] = {{src->codes, q4_codes_bytes(*src), "codes"},
                 {src->scales, q4_sb_bytes(*src), "scales"},
                 {src->biases, q4_sb_bytes(*src), "biases"}};
  if ((st = check_alias(outs, 2, ins, 3))) return st;
  return hip_status(sdv::q4_repack_launch(*src, fused_gateup, codes_out, sb_out, (hipStream_t)stream),
                    "sdv_q4_repack launch");
}

size_t sdv_q8_0t_codes_bytes(int E, int N, int K, int fused_gateup) {
  if (E <= 0 || N <= 0 || K <= 0 || K % SDV_GROUP) return 0;
  return sdv::q8_0t_codes_bytes(E, N, K, fused_gateup ? 1 : 0);
}

int sdv_q8_0_repack(const sdv_q8_0* src, int fused_gateup, void* codes_out, uint32_t* sb_out, sdv_stream_t stream) {
  int st;
  if (!src) return fail(SDV_EINVAL, "src descriptor is NULL");
  if (src->K <= 0 || src->K % SDV_GROUP) return fail(SDV_ELAYOUT, "src K=%d is not a positive multiple of 64", src->K);
  if (src->N <= 0 || src->E <= 0) return fail(SDV_EINVAL, "src E=%d N=%d must be positive", src->E, src->N);
  if (fused_gateup != 0 && fused_gateup != 1) return fail(SDV_ELAYOUT, "fused_gateup=%d must be 0 or 1", fused_gateup);
  if (fused_gateup && (src->N % 2)) return fail(SDV_ELAYOUT, "fused gate/up needs an even N (got %d)", src->N);
  if ((st = check_ptr(src->qs, "qs"))) return st;
  if ((st = check_ptr(src->d, "d"))) return st;
  if ((st = check_ptr(codes_out, "codes_out"))) return st;
  if ((st = check_ptr(sb_out, "sb_out"))) return st;
  const size_t elems = (size_t)src->E * src->N * src->K;
  Range outs[] = {{codes_out, sdv::q8_0t_codes_bytes(src->E, src->N, src->K, fused_gateup), "codes_out"},
                  {sb_out, sdv::q4t_sb_bytes(src->E, src->N, src->K, fused_gateup), "sb_out"}};
  Range ins[] = {{src->qs, elems, "qs"}, {src->d, elems / 32 * 2, "d"}};
  if ((st = check_alias(outs, 2, ins, 2))) return st;
  return hip_status(sdv::q8_0_repack_launch(*src, fused_gateup, codes_out, sb_out, (hipStream_t)stream),
                    "sdv_q8_0_repack launch");
}

size_t sdv_q3t_codes_bytes(int E, int N, int K, int fused_gateup) {
  if (E <= 0 || N <= 0 || K <= 0 || K % SDV_GROUP) return 0;
  return sdv::q3t_codes_bytes(E, N, K, fused_gateup ? 1 : 0);
}

int sdv_q3_repack(const sdv_q3* src, int fused_gateup, void* codes_out, uint32_t* sb_out, sdv_stream_t stream) {
  int st;
  if (!src) return fail(SDV_EINVAL, "src descriptor is NULL");
  if (src->K <= 0 || src->K % SDV_GROUP) return fail(SDV_ELAYOUT, "src K=%d is not a positive multiple of 64", src->K);
  if (src->N <= 0 || src->E <= 0) return fail(SDV_EINVAL, "src E=%d N=%d must be positive", src->E, src->N);
  if (fused_gateup != 0 && fused_gateup != 1) return fail(SDV_ELAYOUT, "fused_gateup=%d must be 0 or 1", fused_gateup);
  if (fused_gateup && (src->N % 2)) return fail(SDV_ELAYOUT, "fused gate/up needs an even N (got %d)", src->N);
  const void* ptrs[] = {src->codes, src->scales, src->biases, codes_out, sb_out};
  const char* names[] = {"codes", "scales", "biases", "codes_out", "sb_out"};
  for (int i = 0; i < 5; ++i)
    if ((st = check_ptr(ptrs[i], names[i]))) return st;
  const size_t rows = (size_t)src->E * src->N;
  Range outs[] = {{codes_out, sdv::q3t_codes_bytes(src->E, src->N, src->K, fused_gateup), "codes_out"},
                  {sb_out, sdv::q4t_sb_bytes(src->E, src->N, src->K, fused_gateup), "sb_out"}};
  Range ins[] = {{src->codes, rows * 3 * src->K / 8, "codes"},
                 {src->scales, rows * (src->K / 64) * 2, "scales"},
                 {src->biases, rows * (src->K / 64) * 2, "biases"}};
  if ((st = check_alias(outs, 2, ins, 3))) return st;
  return hip_status(sdv::q3_repack_launch(*src, fused_gateup, codes_out, sb_out, (hipStream_t)stream),
                    "sdv_q3_repack launch");
}

int sdv_qmv_k(const sdv_q4t* W, const void* act, int act_dtype, int k, int mode, float* y,
              sdv_stream_t stream) {
  int st;
  if ((st = check_q4t(W, "W"))) return st;
  if (W->E != 1) return fail(SDV_EINVAL, "dense product needs E=1 (got %d)", W->E);
  if ((st = check_width(k))) return st;
  if ((st = check_mode(mode, act_dtype, W->N))) return st;
  if ((st = check_mode_layout(mode, *W))) return st;
  if ((st = check_ptr(act, "act"))) return st;
  if ((st = check_ptr(y, "y"))) return st;
  if ((st = check_lds(*W, act_dtype, k, false))) return st;
  const size_t act_bytes = (size_t)k * W->K * (act_dtype == SDV_ACT_F32 ? 4 : 2);
  const size_t n_out = mode == SDV_MODE_PLAIN ? W->N : W->N / 2;
  Range outs[] = {{y, (size_t)k * n_out * 4, "y"}};
  Range ins[] = {{W->codes, tiled_codes_bytes(*W), "codes"},
                 {W->sb, sdv::q4t_sb_bytes(W->E, W->N, W->K, W->fused_gateup), "sb"},
                 {act, act_bytes, "act"}};
  if ((st = check_alias(outs, 1, ins, 3))) return st;
  return hip_status(sdv::q4_launch(*W, mode, act, act_dtype, false, nullptr, nullptr, nullptr,
                                   nullptr, nullptr, k, 1, y, nullptr, nullptr, nullptr,
                                   (hipStream_t)stream),
                    "sdv_qmv_k launch");
}

int sdv_qmv_k_multi(const sdv_q4t* W, int nw, const void* act, int act_dtype, int k, int mode, float* const* y,
                    sdv_stream_t stream) {
  int st;
  if (!W) return fail(SDV_EINVAL, "W is NULL");
  if (!y) return fail(SDV_EINVAL, "y is NULL");
  if (nw < 1 || nw > sdv::dense_multi_max())
    return fail(SDV_ERANGE, "nw=%d outside 1..%d", nw, sdv::dense_multi_max());
  if ((st = check_width(k))) return st;
  if ((st = check_ptr(act, "act"))) return st;
  const sdv_q4t& W0 = W[0];
  const size_t act_bytes = (size_t)k * W0.K * (act_dtype == SDV_ACT_F32 ? 4 : 2);
  const size_t n_out = mode == SDV_MODE_PLAIN ? W0.N : W0.N / 2;
  // every weight: a valid dense descriptor of W[0]'s shape, format and layout
  Range ins[2 * 16 + 1];
  Range outs[16];
  for (int m = 0; m < nw; ++m) {
    if ((st = check_q4t(&W[m], "W[m]"))) return st;
    if (W[m].E != 1) return fail(SDV_EINVAL, "dense product needs E=1 (W[%d] has %d)", m, W[m].E);
    if (W[m].N != W0.N || W[m].K != W0.K || W[m].format != W0.format || W[m].fused_gateup != W0.fused_gateup)
      return fail(SDV_ELAYOUT, "W[%d] differs from W[0] in shape, format or layout", m);
    if ((st = check_ptr(y[m], "y[m]"))) return st;
    ins[2 * m] = {W[m].codes, tiled_codes_bytes(W[m]), "codes"};
    ins[2 * m + 1] = {W[m].sb, sdv::q4t_sb_bytes(1, W[m].N, W[m].K, W[m].fused_gateup), "sb"};
    outs[m] = {y[m], (size_t)k * n_out * 4, "y[m]"};
  }
  ins[2 * nw] = {act, act_bytes, "act"};
  if ((st = check_mode(mode, act_dtype, W0.N))) return st;
  if ((st = check_mode_layout(mode, W0))) return st;
  if ((st = check_lds(W0, act_dtype, k, false))) return st;
  if ((st = check_alias(outs, nw, ins, 2 * nw + 1))) return st;
  return hip_status(sdv::dense_multi_launch(W, nw, mode, act, act_dtype, k, y, (hipStream_t)stream),
                    "sdv_qmv_k_multi launch");
}

int sdv_moe_route_k(const float* logits, int k, int E, int topk, int score_mode, int renorm,
                    int32_t* idx, float* w, int32_t* union_ids, int32_t* n_union,
                    int32_t* pair_off, int32_t* pair_row, int32_t* pair_slot,
                    sdv_stream_t stream) {
  int st;
  if ((st = check_width(k))) return st;
  if (E < 1 || E > SDV_MAX_EXPERTS) return fail(SDV_ERANGE, "E=%d outside 1..%d", E, SDV_MAX_EXPERTS);
  if (topk < 1 || topk > SDV_MAX_TOPK || topk > E)
    return fail(SDV_ERANGE, "topk=%d outside 1..min(E,%d)", topk, SDV_MAX_TOPK);
  if (score_mode != SDV_ROUTE_SOFTMAX && score_mode != SDV_ROUTE_SIGMOID)
    return fail(SDV_EINVAL, "unknown score mode %d", score_mode);
  const void* ptrs[] = {logits, idx, w, union_ids, n_union, pair_off, pair_row, pair_slot};
  const char* names[] = {"logits", "idx", "w", "union_ids", "n_union", "pair_off", "pair_row", "pair_slot"};
  for (int i = 0; i < 8; ++i)
    if ((st = check_ptr(ptrs[i], names[i]))) return st;
  const size_t kt = (size_t)k * topk;
  Range outs[] = {{idx, kt * 4, "idx"},           {w, kt * 4, "w"},
                  {union_ids, kt * 4, "union_ids"}, {n_union, 4, "n_union"},
                  {pair_off, (kt + 1) * 4, "pair_off"}, {pair_row, kt * 4, "pair_row"},
                  {pair_slot, kt * 4, "pair_slot"}};
  Range ins[] = {{logits, (size_t)k * E * 4, "logits"}};
  if ((st = check_alias(outs, 7, ins, 1))) return st;
  return hip_status(sdv::route_launch(logits, k, E, topk, score_mode, renorm, idx, w, union_ids,
                                      n_union, pair_off, pair_row, pair_slot, (hipStream_t)stream),
                    "sdv_moe_route_k launch");
}

int sdv_gather_qmv_k(const sdv_q4t* bank, int mode, const void* act, int act_dtype,
                     const int32_t* union_ids, const int32_t* n_union, const int32_t* pair_off,
                     const int32_t* pair_row, const int32_t* pair_slot, int k, int topk,
                     float* out, const sdv_q4t* shared, const void* shared_act, float* shared_out,
                     sdv_stream_t stream) {
  int st;
  if ((st = check_q4t(bank, "bank"))) return st;
  if ((st = check_width(k))) return st;
  if (topk < 1 || topk > SDV_MAX_TOPK || topk > bank->E)
    return fail(SDV_ERANGE, "topk=%d outside 1..min(E,%d)", topk, SDV_MAX_TOPK);
  if ((st = check_mode(mode, act_dtype, bank->N))) return st;
  if ((st = check_mode_layout(mode, *bank))) return st;
  if ((st = check_lds(*bank, act_dtype, k, true))) return st;
  const void* ptrs[] = {act, union_ids, n_union, pair_off, pair_row, pair_slot, out};
  const char* names[] = {"act", "union_ids", "n_union", "pair_off", "pair_row", "pair_slot", "out"};
  for (int i = 0; i < 7; ++i)
    if ((st = check_ptr(ptrs[i], names[i]))) return st;
  if (shared) {
    if ((st = check_q4t(shared, "shared"))) return st;
    if (shared->E != 1) return fail(SDV_EINVAL, "shared expert needs E=1 (got %d)", shared->E);
    if (shared->N != bank->N || shared->K != bank->K || shared->fused_gateup != bank->fused_gateup ||
        shared->format != bank->format)
      return fail(SDV_ELAYOUT,
                  "shared expert geometry (N=%d K=%d fused=%d format=%d) differs from the bank's (N=%d K=%d fused=%d format=%d)",
                  shared->N, shared->K, shared->fused_gateup, shared->format, bank->N, bank->K, bank->fused_gateup,
                  bank->format);
    if ((st = check_ptr(shared_act, "shared_act"))) return st;
    if ((st = check_ptr(shared_out, "shared_out"))) return st;
  } else if (shared_act || shared_out) {
    return fail(SDV_EINVAL, "shared_act/shared_out given without a shared expert");
  }
  const size_t kt = (size_t)k * topk;
  const size_t act_bytes = act_dtype == SDV_ACT_F32 ? kt * bank->K * 4 : (size_t)k * bank->K * 2;
  const size_t n_out = mode == SDV_MODE_PLAIN ? bank->N : bank->N / 2;
  const size_t sh_act_bytes = shared ? (size_t)k * bank->K * (act_dtype == SDV_ACT_F32 ? 4 : 2) : 0;
  Range outs[] = {{out, kt * n_out * 4, "out"}, {shared_out, shared ? (size_t)k * n_out * 4 : 0, "shared_out"}};
  Range ins[] = {{bank->codes, tiled_codes_bytes(*bank), "codes"},
                 {bank->sb, sdv::q4t_sb_bytes(bank->E, bank->N, bank->K, bank->fused_gateup), "sb"},
                 {act, act_bytes, "act"},
                 {union_ids, kt * 4, "union_ids"},
                 {n_union, 4, "n_union"},
                 {pair_off, (kt + 1) * 4, "pair_off"},
                 {pair_row, kt * 4, "pair_row"},
                 {pair_slot, kt * 4, "pair_slot"},
                 {shared ? shared->codes : nullptr, shared ? tiled_codes_bytes(*shared) : 0, "shared codes"},
                 {shared ? shared->sb : nullptr, shared ? sdv::q4t_sb_bytes(1, bank->N, bank->K, bank->fused_gateup) : 0,
                  "shared sb"},
                 {shared_act, sh_act_bytes, "shared_act"}};
  if ((st = check_alias(outs, 2, ins, 11))) return st;
  return hip_status(sdv::q4_launch(*bank, mode, act, act_dtype, true, union_ids, n_union, pair_off,
                                   pair_row, pair_slot, k, topk, out, shared, shared_act, shared_out,
                                   (hipStream_t)stream),
                    "sdv_gather_qmv_k launch");
}

size_t sdv_moe_experts_partial_bytes(int k, int topk, int H, int I) {
  if (k < 1 || k > SDV_MAX_ROWS || topk < 1 || topk > SDV_MAX_TOPK || H <= 0 || I <= 0 || H % SDV_GROUP ||
      I % SDV_GROUP)
    return 0;
  return sdv::expert_partial_bytes(k, topk, H, I);
}

}  // extern "C"

namespace {

// The checks sdv_moe_experts_k and sdv_moe_route_experts_k share: weights,
// shapes, widths, LDS and the partial output's size (in *pbytes).
int check_experts(const sdv_q4t* gate_up, const sdv_q4t* down, const sdv_q4t* shared_gate_up,
                  const sdv_q4t* shared_down, int k, int topk, size_t lds_extra_for_route, size_t* pbytes_out,
                  bool q4_only) {
  int st;
  if ((st = check_q4t(gate_up, "gate_up"))) return st;
  if ((st = check_q4t(down, "down"))) return st;
  if (!gate_up->fused_gateup) return fail(SDV_ELAYOUT, "gate_up must be repacked with fused_gateup=1");
  const int fmt = gate_up->format;
  if (down->format != fmt || (shared_gate_up && shared_gate_up->format != fmt) ||
      (shared_down && shared_down->format != fmt))
    return fail(SDV_ELAYOUT, "the fused expert kernel needs one weight format for all four weights");
  if (q4_only && fmt != SDV_FMT_AFFINE_Q4)
    return fail(SDV_ELAYOUT, "the router dispatch inside the expert kernel takes affine Q4 weights; "
                "route with sdv_moe_route_k and call sdv_moe_experts_k for Q8_0 and Q3");
  if (down->fused_gateup) return fail(SDV_ELAYOUT, "down must be repacked with fused_gateup=0");
  const int H = gate_up->K, I = gate_up->N / 2;
  if (down->E != gate_up->E || down->N != H || down->K != I)
    return fail(SDV_ELAYOUT, "down is E=%d N=%d K=%d, expected E=%d N=%d K=%d (gate_up E=%d N=2I=%d K=H=%d)",
                down->E, down->N, down->K, gate_up->E, H, I, gate_up->E, gate_up->N, H);
  if (I % SDV_GROUP) return fail(SDV_ELAYOUT, "intermediate size %d is not a multiple of 64", I);
  if (I > kMaxExpertInter) return fail(SDV_ERANGE, "intermediate size %d above %d (8 slices)", I, kMaxExpertInter);
  if ((st = check_width(k))) return st;
  if (topk < 1 || topk > SDV_MAX_TOPK || topk > gate_up->E)
    return fail(SDV_ERANGE, "topk=%d outside 1..min(E,%d)", topk, SDV_MAX_TOPK);
  if ((shared_gate_up == nullptr) != (shared_down == nullptr))
    return fail(SDV_EINVAL, "give both shared expert weights or neither");
  if (shared_gate_up) {
    if ((st = check_q4t(shared_gate_up, "shared_gate_up"))) return st;
    if ((st = check_q4t(shared_down, "shared_down"))) return st;
    if (shared_gate_up->E != 1 || shared_down->E != 1)
      return fail(SDV_EINVAL, "shared expert weights need E=1");
    if (shared_gate_up->N != gate_up->N || shared_gate_up->K != H || !shared_gate_up->fused_gateup ||
        shared_down->N != H || shared_down->K != I || shared_down->fused_gateup)
      return fail(SDV_ELAYOUT, "shared expert geometry differs from the routed experts'");
  }
  size_t lds = sdv::expert_lds_bytes(k, H, fmt);
  if (lds_extra_for_route > lds) lds = lds_extra_for_route;
  // the kernel's static LDS (row maps and the in-kernel routing's outputs)
  // takes at most kExpertStaticLds of the workgroup's LDS
  constexpr size_t kExpertStaticLds = 4096;
  if (lds > kMaxLds - kExpertStaticLds)
    return fail(SDV_ELAYOUT, "H=%d with k=%d needs %zu bytes of LDS (max %zu)", H, k, lds, kMaxLds - kExpertStaticLds);
  const size_t pbytes = sdv::expert_partial_bytes(k, topk, H, I);
  if (pbytes >= 0x7FFFFFF0u) return fail(SDV_ERANGE, "partial output of %zu bytes exceeds 2 GiB", pbytes);
  *pbytes_out = pbytes;
  return SDV_OK;
}

// Ranges of an expert call's weights (for the alias checks).
int expert_weight_ranges(const sdv_q4t* gate_up, const sdv_q4t* down, const sdv_q4t* shared_gate_up,
                         const sdv_q4t* shared_down, Range* r) {
  const int H = gate_up->K, I = gate_up->N / 2;
  r[0] = {gate_up->codes, tiled_codes_bytes(*gate_up), "gate_up codes"};
  r[1] = {gate_up->sb, sdv::q4t_sb_bytes(gate_up->E, gate_up->N, H, 1), "gate_up sb"};
  r[2] = {down->codes, tiled_codes_bytes(*down), "down codes"};
  r[3] = {down->sb, sdv::q4t_sb_bytes(down->E, H, I, 0), "down sb"};
  r[4] = {shared_gate_up ? shared_gate_up->codes : nullptr, shared_gate_up ? tiled_codes_bytes(*shared_gate_up) : 0,
          "shared_gate_up codes"};
  r[5] = {shared_gate_up ? shared_gate_up->sb : nullptr, shared_gate_up ? sdv::q4t_sb_bytes(1, 2 * I, H, 1) : 0,
          "shared_gate_up sb"};
  r[6] = {shared_down ? shared_down->codes : nullptr, shared_down ? tiled_codes_bytes(*shared_down) : 0,
          "shared_down codes"};
  r[7] = {shared_down ? shared_down->sb : nullptr, shared_down ? sdv::q4t_sb_bytes(1, H, I, 0) : 0, "shared_down sb"};
  return 8;
}

}  // namespace

extern "C" {

int sdv_moe_experts_k(const sdv_q4t* gate_up, const sdv_q4t* down, const void* x, const int32_t* union_ids,
                      const int32_t* n_union, const int32_t* pair_off, const int32_t* pair_row,
                      const int32_t* pair_slot, int k, int topk, const sdv_q4t* shared_gate_up,
                      const sdv_q4t* shared_down, float* partial, sdv_stream_t stream) {
  int st;
  size_t pbytes = 0;
  if ((st = check_experts(gate_up, down, shared_gate_up, shared_down, k, topk, 0, &pbytes, false))) return st;
  const int H = gate_up->K;
  const void* ptrs[] = {x, union_ids, n_union, pair_off, pair_row, pair_slot, partial};
  const char* names[] = {"x", "union_ids", "n_union", "pair_off", "pair_row", "pair_slot", "partial"};
  for (int i = 0; i < 7; ++i)
    if ((st = check_ptr(ptrs[i], names[i]))) return st;
  const size_t kt = (size_t)k * topk;
  Range outs[] = {{partial, pbytes, "partial"}};
  Range ins[14];
  expert_weight_ranges(gate_up, down, shared_gate_up, shared_down, ins);
  ins[8] = {x, (size_t)k * H * 2, "x"};
  ins[9] = {union_ids, kt * 4, "union_ids"};
  ins[10] = {n_union, 4, "n_union"};
  ins[11] = {pair_off, (kt + 1) * 4, "pair_off"};
  ins[12] = {pair_row, kt * 4, "pair_row"};
  ins[13] = {pair_slot, kt * 4, "pair_slot"};
  if ((st = check_alias(outs, 1, ins, 14))) return st;
  return hip_status(sdv::moe_experts_launch(*gate_up, *down, shared_gate_up, shared_down, x, union_ids, n_union,
                                            pair_off, pair_row, pair_slot, k, topk, partial, (hipStream_t)stream),
                    "sdv_moe_experts_k launch");
}

int sdv_moe_route_experts_k(const float* logits, int score_mode, int renorm, const sdv_q4t* gate_up,
                            const sdv_q4t* down, const void* x, int k, int topk, const sdv_q4t* shared_gate_up,
                            const sdv_q4t* shared_down, int32_t* idx, float* w, int32_t* union_ids, int32_t* n_union,
                            int32_t* pair_off, int32_t* pair_row, int32_t* pair_slot, float* partial,
                            sdv_stream_t stream) {
  int st;
  if ((st = check_q4t(gate_up, "gate_up"))) return st;
  const int E = gate_up->E;
  if (E > SDV_MAX_EXPERTS) return fail(SDV_ERANGE, "E=%d above %d", E, SDV_MAX_EXPERTS);
  if (score_mode != SDV_ROUTE_SOFTMAX && score_mode != SDV_ROUTE_SIGMOID)
    return fail(SDV_EINVAL, "unknown score mode %d", score_mode);
  size_t pbytes = 0;
  const size_t route_lds = sdv::route_in_experts(k, E) ? sdv::route_experts_lds_bytes(k, E, gate_up->K) : 0;
  if ((st = check_experts(gate_up, down, shared_gate_up, shared_down, k, topk, route_lds, &pbytes, true))) return st;
  const int H = gate_up->K;
  const void* ptrs[] = {logits, x, idx, w, union_ids, n_union, pair_off, pair_row, pair_slot, partial};
  const char* names[] = {"logits", "x", "idx", "w", "union_ids", "n_union", "pair_off", "pair_row", "pair_slot",
                         "partial"};
  for (int i = 0; i < 10; ++i)
    if ((st = check_ptr(ptrs[i], names[i]))) return st;
  const size_t kt = (size_t)k * topk;
  Range outs[] = {{idx, kt * 4, "idx"},           {w, kt * 4, "w"},
                  {union_ids, kt * 4, "union_ids"}, {n_union, 4, "n_union"},
                  {pair_off, (kt + 1) * 4, "pair_off"}, {pair_row, kt * 4, "pair_row"},
                  {pair_slot, kt * 4, "pair_slot"}, {partial, pbytes, "partial"}};
  Range ins[10];
  expert_weight_ranges(gate_up, down, shared_gate_up, shared_down, ins);
  ins[8] = {x, (size_t)k * H * 2, "x"};
  ins[9] = {logits, (size_t)k * E * 4, "logits"};
  if ((st = check_alias(outs, 8, ins, 10))) return st;
  return hip_status(sdv::moe_route_experts_launch(logits, score_mode, renorm, *gate_up, *down, shared_gate_up,
                                                  shared_down, x, k, topk, idx, w, union_ids, n_union, pair_off,
                                                  pair_row, pair_slot, partial, (hipStream_t)stream),
                    "sdv_moe_route_experts_k launch");
}

int sdv_moe_combine_sliced_k(const float* partial, const int32_t* idx, const float* w, const float* shared_logit,
                             int k, int topk, int H, int I, int has_shared, float* y, sdv_stream_t stream) {
  int st;
  if ((st = check_width(k))) return st;
  if (topk < 1 || topk > SDV_MAX_TOPK) return fail(SDV_ERANGE, "topk=%d outside 1..%d", topk, SDV_MAX_TOPK);
  if (H <= 0 || H % SDV_GROUP || I <= 0 || I % SDV_GROUP)
    return fail(SDV_EINVAL, "H=%d and I=%d must be positive multiples of 64", H, I);
  if (I > kMaxExpertInter) return fail(SDV_ERANGE, "I=%d above %d (8 slices)", I, kMaxExpertInter);
  if (has_shared != 0 && has_shared != 1) return fail(SDV_EINVAL, "has_shared=%d must be 0 or 1", has_shared);
  if (shared_logit && !has_shared) return fail(SDV_EINVAL, "shared_logit given without a shared expert");
  const void* ptrs[] = {partial, idx, w, y};
  const char* names[] = {"partial", "idx", "w", "y"};
  for (int i = 0; i < 4; ++i)
    if ((st = check_ptr(ptrs[i], names[i]))) return st;
  if (shared_logit && (st = check_ptr(shared_logit, "shared_logit"))) return st;
  const size_t kt = (size_t)k * topk;
  Range outs[] = {{y, (size_t)k * H * 4, "y"}};
  Range ins[] = {{partial, sdv::expert_partial_bytes(k, topk, H, I), "partial"},
                 {idx, kt * 4, "idx"},
                 {w, kt * 4, "w"},
                 {shared_logit, shared_logit ? (size_t)k * 4 : 0, "shared_logit"}};
  if ((st = check_alias(outs, 1, ins, 4))) return st;
  return hip_status(sdv::combine_sliced_launch(partial, idx, w, shared_logit, sdv::expert_slices(I), k, topk, H,
                                               has_shared, y, (hipStream_t)stream),
                    "sdv_moe_combine_sliced_k launch");
}

int sdv_moe_combine_k(const float* partial, const float* w, const float* shared_out,
                      const float* shared_logit, int k, int topk, int H, float* y,
                      sdv_stream_t stream) {
  int st;
  if ((st = check_width(k))) return st;
  if (topk < 1 || topk > SDV_MAX_TOPK) return fail(SDV_ERANGE, "topk=%d outside 1..%d", topk, SDV_MAX_TOPK);
  if (H < 4 || H % 4) return fail(SDV_EINVAL, "H=%d must be a positive multiple of 4", H);
  if ((st = check_ptr(partial, "partial"))) return st;
  if ((st = check_ptr(w, "w"))) return st;
  if ((st = check_ptr(y, "y"))) return st;
  if (shared_out && (st = check_ptr(shared_out, "shared_out"))) return st;
  if (shared_logit && !shared_out) return fail(SDV_EINVAL, "shared_logit given without shared_out");
  if (shared_logit && (st = check_ptr(shared_logit, "shared_logit"))) return st;
  Range outs[] = {{y, (size_t)k * H * 4, "y"}};
  Range ins[] = {{partial, (size_t)k * topk * H * 4, "partial"},
                 {w, (size_t)k * topk * 4, "w"},
                 {shared_out, shared_out ? (size_t)k * H * 4 : 0, "shared_out"},
                 {shared_logit, shared_logit ? (size_t)k * 4 : 0, "shared_logit"}};
  if ((st = check_alias(outs, 1, ins, 4))) return st;
  return hip_status(sdv::combine_launch(partial, w, shared_out, shared_logit, k, topk, H, y,
                                        (hipStream_t)stream),
                    "sdv_moe_combine_k launch");
}

int sdv_gdn_verify_k(const float* S_in, const float* q, const float* kk, const float* v,
                     const float* g, const float* beta, int k, int Hv, int Hk, int Dk, int Dv,
                     float* y, float* const* snaps, sdv_stream_t stream) {
  int st;
  if ((st = check_width(k))) return st;
  if (Dk != 64 && Dk != 128) return fail(SDV_ELAYOUT, "Dk=%d, only 64 and 128 are supported", Dk);
  if (Hv < 1 || Hk < 1 || Dv < 1) return fail(SDV_EINVAL, "Hv=%d Hk=%d Dv=%d must be positive", Hv, Hk, Dv);
  if (Hv % Hk) return fail(SDV_ELAYOUT, "Hv=%d is not a multiple of Hk=%d", Hv, Hk);
  if ((long)Hv * Dv > (1L << 26)) return fail(SDV_EINVAL, "Hv*Dv=%ld too large", (long)Hv * Dv);
  const void* ptrs[] = {S_in, q, kk, v, g, beta, y};
  const char* names[] = {"S_in", "q", "kk", "v", "g", "beta", "y"};
  for (int i = 0; i < 7; ++i)
    if ((st = check_ptr(ptrs[i], names[i]))) return st;
  if (!snaps) return fail(SDV_EINVAL, "snaps is NULL");
  const size_t state = (size_t)Hv * Dv * Dk * 4;
  Range ins[] = {{S_in, state, "S_in"},
                 {q, (size_t)k * Hk * Dk * 4, "q"},
                 {kk, (size_t)k * Hk * Dk * 4, "kk"},
                 {v, (size_t)k * Hv * Dv * 4, "v"},
                 {g, (size_t)k * Hv * 4, "g"},
                 {beta, (size_t)k * Hv * 4, "beta"}};
  Range outs[SDV_MAX_ROWS + 1];
  outs[0] = {y, (size_t)k * Hv * Dv * 4, "y"};
  for (int t = 0; t < k; ++t) {
    if ((st = check_ptr(snaps[t], kSnapNames[t]))) return st;
    outs[t + 1] = {snaps[t], state, kSnapNames[t]};
  }
  if ((st = check_alias(outs, k + 1, ins, 6))) return st;
  return hip_status(sdv::gdn_launch(S_in, q, kk, v, g, beta, k, Hv, Hk, Dk, Dv, y, snaps,
                                    (hipStream_t)stream),
                    "sdv_gdn_verify_k launch");
}

int sdv_gdn_rollback(int k, int j, int* selected_slot) {
  int st;
  if (!selected_slot) return fail(SDV_EINVAL, "selected_slot is NULL");
  if ((st = check_width(k))) return st;
  if (j < 0 || j > k) return fail(SDV_ERANGE, "accepted prefix %d outside 0..%d", j, k);
  *selected_slot = j;
  return ok();
}

int sdv_gdn_rollback_copy(float* dst, const float* S_in, float* const* snaps, int k, int j,
                          size_t state_elems, sdv_stream_t stream) {
  int st, slot = 0;
  if ((st = sdv_gdn_rollback(k, j, &slot))) return st;
  if ((st = check_ptr(dst, "dst"))) return st;
  if (state_elems == 0) return fail(SDV_EINVAL, "state_elems is 0");
  const float* src = nullptr;
  if (slot == 0) {
    src = S_in;
  } else {
    if (!snaps) return fail(SDV_EINVAL, "snaps is NULL");
    src = snaps[slot - 1];
  }
  if ((st = check_ptr(src, slot == 0 ? "S_in" : "selected snapshot"))) return st;
  if (src == dst) return ok();
  Range a{dst, state_elems * 4, "dst"}, b{src, state_elems * 4, "source"};
  if (overlap(a, b)) return fail(SDV_EALIAS, "dst partially overlaps the selected state");
  return hip_status(hipMemcpyAsync(dst, src, state_elems * 4, hipMemcpyDeviceToDevice, (hipStream_t)stream),
                    "sdv_gdn_rollback_copy");
}

size_t sdv_verify_accept_workspace_bytes(int k, int V) {
  if (k < 1 || k > SDV_MAX_ROWS || V < 1 || V > (1 << 30)) return 0;
  return sdv::accept_workspace_bytes(k, V);
}

int sdv_verify_accept_k(const float* logits, const float* noise, float inv_temp, const int32_t* drafts, int k,
                        int V, int eos, int32_t* tokens, int32_t* accepted, void* workspace,
                        size_t workspace_bytes, sdv_stream_t stream) {
  int st;
  if ((st = check_width(k))) return st;
  if (V < 1 || V > (1 << 30)) return fail(SDV_ERANGE, "V=%d outside 1..2^30", V);
  if ((st = check_ptr(logits, "logits"))) return st;
  if (noise) {
    if ((st = check_ptr(noise, "noise"))) return st;
    if (!(inv_temp > 0.0f && inv_temp <= 3.4e38f))
      return fail(SDV_ERANGE, "inv_temp=%g must be finite and positive", (double)inv_temp);
  }
  if (k > 1 && (st = check_ptr(drafts, "drafts"))) return st;
  if ((st = check_ptr(tokens, "tokens"))) return st;
  if ((st = check_ptr(accepted, "accepted"))) return st;
  if ((st = check_ptr(workspace, "workspace"))) return st;
  const size_t need = sdv::accept_workspace_bytes(k, V);
  if (workspace_bytes < need)
    return fail(SDV_EINVAL, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  const size_t lbytes = (size_t)k * V * 4;
  Range outs[] = {{tokens, (size_t)k * 4, "tokens"}, {accepted, 4, "accepted"}, {workspace, need, "workspace"}};
  Range ins[] = {{logits, lbytes, "logits"},
                 {noise, noise ? lbytes : 0, "noise"},
                 {drafts, k > 1 ? (size_t)(k - 1) * 4 : 0, "drafts"}};
  if ((st = check_alias(outs, 3, ins, 3))) return st;
  return hip_status(sdv::accept_launch(logits, noise, inv_temp, k > 1 ? drafts : nullptr, k, V, eos, tokens,
                                       accepted, workspace, (hipStream_t)stream),
                    "sdv_verify_accept_k launch");
}

int sdv_verify_accept_k_noalloc(const float* logits, const float* noise, float inv_temp, const int32_t* drafts,
                                int k, int V, int eos, int32_t* tokens, int32_t* accepted, sdv_stream_t stream) {
  int st;
  if ((st = check_width(k))) return st;
  if (V < 1 || V > (1 << 30)) return fail(SDV_ERANGE, "V=%d outside 1..2^30", V);
  const size_t need = sdv::accept_workspace_bytes(k, V);
  if (need > sdv::accept_scratch_bytes())
    return fail(SDV_ERANGE, "k=%d rows of V=%d logits need %zu bytes of workspace, more than the %zu of the "
                "built-in scratch (use sdv_verify_accept_k with a caller workspace)",
                k, V, need, sdv::accept_scratch_bytes());
  if ((st = check_ptr(logits, "logits"))) return st;
  if (noise) {
    if ((st = check_ptr(noise, "noise"))) return st;
    if (!(inv_temp > 0.0f && inv_temp <= 3.4e38f))
      return fail(SDV_ERANGE, "inv_temp=%g must be finite and positive", (double)inv_temp);
  }
  if (k > 1 && (st = check_ptr(drafts, "drafts"))) return st;
  if ((st = check_ptr(tokens, "tokens"))) return st;
  if ((st = check_ptr(accepted, "accepted"))) return st;
  const size_t lbytes = (size_t)k * V * 4;
  Range outs[] = {{tokens, (size_t)k * 4, "tokens"}, {accepted, 4, "accepted"}};
  Range ins[] = {{logits, lbytes, "logits"},
                 {noise, noise ? lbytes : 0, "noise"},
                 {drafts, k > 1 ? (size_t)(k - 1) * 4 : 0, "drafts"}};
  if ((st = check_alias(outs, 2, ins, 3))) return st;
  return hip_status(sdv::accept_noalloc_launch(logits, noise, inv_temp, k > 1 ? drafts : nullptr, k, V, eos, tokens,
                                               accepted, (hipStream_t)stream),
                    "sdv_verify_accept_k_noalloc launch");
}

size_t sdv_verify_accept_scratch_bytes(void) { return sdv::accept_scratch_bytes(); }

int sdv_gdn_prepare_k(const float* qkv, const float* hist, const float* conv_w, const float* a, const float* b,
                      const float* A_log, const float* dt_bias, int k, int Hv, int Hk, int Dk, int Dv, int conv_act,
                      float eps, float* q, float* kk, float* v, float* g, float* beta, float* window,
                      sdv_stream_t stream) {
  int st;
  if ((st = check_width(k))) return st;
  if (Hv <= 0 || Hk <= 0) return fail(SDV_EINVAL, "Hv=%d Hk=%d must be positive", Hv, Hk);
  if (Hv % Hk) return fail(SDV_ELAYOUT, "Hv=%d is not a multiple of Hk=%d", Hv, Hk);
  if (Dk != Dv || (Dk != 64 && Dk != 128))
    return fail(SDV_ELAYOUT, "Dk=%d Dv=%d: the preparation needs Dk = Dv in {64, 128}", Dk, Dv);
  if (conv_act != SDV_CONV_NONE && conv_act != SDV_CONV_SILU) return fail(SDV_EINVAL, "conv_act=%d", conv_act);
  if (!(eps >= 0.0f && eps <= 3.4e38f)) return fail(SDV_ERANGE, "eps=%g must be finite and >= 0", (double)eps);
  const struct {
    const void* p;
    const char* n;
  } ptrs[] = {{qkv, "qkv"}, {hist, "hist"}, {conv_w, "conv_w"}, {a, "a"}, {b, "b"}, {A_log, "A_log"},
              {dt_bias, "dt_bias"}, {q, "q"}, {kk, "kk"}, {v, "v"}, {g, "g"}, {beta, "beta"}, {window, "window"}};
  for (const auto& pt : ptrs)
    if ((st = check_ptr(pt.p, pt.n))) return st;
  const size_t C = 2 * (size_t)Hk * Dk + (size_t)Hv * Dv;
  Range outs[] = {{q, (size_t)k * Hk * Dk * 4, "q"}, {kk, (size_t)k * Hk * Dk * 4, "kk"},
                  {v, (size_t)k * Hv * Dv * 4, "v"}, {g, (size_t)k * Hv * 4, "g"}, {beta, (size_t)k * Hv * 4, "beta"},
                  {window, (size_t)(k + 3) * C * 4, "window"}};
  Range ins[] = {{qkv, (size_t)k * C * 4, "qkv"}, {hist, 3 * C * 4, "hist"}, {conv_w, C * 16, "conv_w"},
                 {a, (size_t)k * Hv * 4, "a"}, {b, (size_t)k * Hv * 4, "b"}, {A_log, (size_t)Hv * 4, "A_log"},
                 {dt_bias, (size_t)Hv * 4, "dt_bias"}};
  if ((st = check_alias(outs, 6, ins, 7))) return st;
  return hip_status(sdv::gdn_prepare_launch(qkv, hist, conv_w, a, b, A_log, dt_bias, k, Hv, Hk, Dk, Dv, conv_act,
                                            eps, q, kk, v, g, beta, window, (hipStream_t)stream),
                    "sdv_gdn_prepare_k launch");
}

}  // extern "C"

namespace {

// The checks of the preparation + recurrence call; fills the output and
// input ranges for the alias check (outs: y, window, snapshots; ins: 8).
int check_verify_prep(const float* S_in, const float* qkv, const float* hist, const float* conv_w, const float* a,
                      const float* b, const float* A_log, const float* dt_bias, int k, int Hv, int Hk, int Dk,
                      int Dv, int conv_act, float eps, float* window, float* y, float* const* snaps, Range* outs,
                      Range* ins) {
  int st;
  if ((st = check_width(k))) return st;
  if (Hv <= 0 || Hk <= 0) return fail(SDV_EINVAL, "Hv=%d Hk=%d must be positive", Hv, Hk);
  if (Hv % Hk) return fail(SDV_ELAYOUT, "Hv=%d is not a multiple of Hk=%d", Hv, Hk);
  if (Dk != Dv || (Dk != 64 && Dk != 128))
    return fail(SDV_ELAYOUT, "Dk=%d Dv=%d: the preparation needs Dk = Dv in {64, 128}", Dk, Dv);
  if ((long)Hv * Dv > (1L << 26)) return fail(SDV_EINVAL, "Hv*Dv=%ld too large", (long)Hv * Dv);
  if (conv_act != SDV_CONV_NONE && conv_act != SDV_CONV_SILU) return fail(SDV_EINVAL, "conv_act=%d", conv_act);
  if (!(eps >= 0.0f && eps <= 3.4e38f)) return fail(SDV_ERANGE, "eps=%g must be finite and >= 0", (double)eps);
  const struct {
    const void* p;
    const char* n;
  } ptrs[] = {{S_in, "S_in"}, {qkv, "qkv"}, {hist, "hist"}, {conv_w, "conv_w"}, {a, "a"}, {b, "b"},
              {A_log, "A_log"}, {dt_bias, "dt_bias"}, {window, "window"}, {y, "y"}};
  for (const auto& pt : ptrs)
    if ((st = check_ptr(pt.p, pt.n))) return st;
  if (!snaps) return fail(SDV_EINVAL, "snaps is NULL");
  const size_t C = 2 * (size_t)Hk * Dk + (size_t)Hv * Dv;
  const size_t state = (size_t)Hv * Dv * Dk * 4;
  ins[0] = {S_in, state, "S_in"};
  ins[1] = {qkv, (size_t)k * C * 4, "qkv"};
  ins[2] = {hist, 3 * C * 4, "hist"};
  ins[3] = {conv_w, C * 16, "conv_w"};
  ins[4] = {a, (size_t)k * Hv * 4, "a"};
  ins[5] = {b, (size_t)k * Hv * 4, "b"};
  ins[6] = {A_log, (size_t)Hv * 4, "A_log"};
  ins[7] = {dt_bias, (size_t)Hv * 4, "dt_bias"};
  outs[0] = {y, (size_t)k * Hv * Dv * 4, "y"};
  outs[1] = {window, (size_t)(k + 3) * C * 4, "window"};
  for (int t = 0; t < k; ++t) {
    if ((st = check_ptr(snaps[t], kSnapNames[t]))) return st;
    outs[t + 2] = {snaps[t], state, kSnapNames[t]};
  }
  return SDV_OK;
}

}  // namespace

extern "C" {

int sdv_gdn_verify_prep_k(const float* S_in, const float* qkv, const float* hist, const float* conv_w,
                          const float* a, const float* b, const float* A_log, const float* dt_bias, int k, int Hv,
                          int Hk, int Dk, int Dv, int conv_act, float eps, float* window, float* y,
                          float* const* snaps, sdv_stream_t stream) {
  int st;
  Range outs[SDV_MAX_ROWS + 2], ins[8];
  if ((st = check_verify_prep(S_in, qkv, hist, conv_w, a, b, A_log, dt_bias, k, Hv, Hk, Dk, Dv, conv_act, eps,
                              window, y, snaps, outs, ins)))
    return st;
  if ((st = check_alias(outs, k + 2, ins, 8))) return st;
  return hip_status(sdv::gdn_verify_prep_launch(S_in, qkv, hist, conv_w, a, b, A_log, dt_bias, k, Hv, Hk, Dk,
                                                conv_act, eps, window, y, snaps, (hipStream_t)stream),
                    "sdv_gdn_verify_prep_k launch");
}

int sdv_gdn_layers_table(const sdv_gdn_layer* layers, int L, int k, int Hv, int Hk, int Dk, int Dv, void* table,
                         size_t table_bytes) {
  int st;
  if (!layers) return fail(SDV_EINVAL, "layers is NULL");
  if (L < 1 || L > 65535) return fail(SDV_EINVAL, "L=%d outside 1..65535", L);
  if ((st = check_ptr(table, "table"))) return st;
  const size_t need = (size_t)L * sizeof(sdv_gdn_layer);
  if (table_bytes < need) return fail(SDV_EINVAL, "table has %zu bytes, %d layers need %zu", table_bytes, L, need);
  if ((st = check_width(k))) return st;
  std::vector<Range> outs((size_t)L * (k + 2) + 1), ins((size_t)L * 8);
  for (int l = 0; l < L; ++l) {
    const sdv_gdn_layer& g = layers[l];
    if ((st = check_verify_prep(g.S_in, g.qkv, g.hist, g.conv_w, g.a, g.b, g.A_log, g.dt_bias, k, Hv, Hk, Dk, Dv,
                                SDV_CONV_NONE, 0.0f, g.window, g.y, g.snaps, &outs[(size_t)l * (k + 2)],
                                &ins[(size_t)l * 8]))) {
      fail_note(" (layer %d)", l);
      return st;
    }
  }
  outs.back() = {table, need, "table"};
  if ((st = check_alias(outs.data(), (int)outs.size(), ins.data(), (int)ins.size()))) return st;
  return hip_status(hipMemcpy(table, layers, need, hipMemcpyHostToDevice), "sdv_gdn_layers_table copy");
}

int sdv_gdn_verify_prep_k_layers(const void* table, int L, int k, int Hv, int Hk, int Dk, int Dv, int conv_act,
                                 float eps, sdv_stream_t stream) {
  int st;
  if ((st = check_ptr(table, "table"))) return st;
  if (L < 1 || L > 65535) return fail(SDV_EINVAL, "L=%d outside 1..65535", L);
  if ((st = check_width(k))) return st;
  if (Hv <= 0 || Hk <= 0) return fail(SDV_EINVAL, "Hv=%d Hk=%d must be positive", Hv, Hk);
  if (Hv % Hk) return fail(SDV_ELAYOUT, "Hv=%d is not a multiple of Hk=%d", Hv, Hk);
  if (Dk != Dv || (Dk != 64 && Dk != 128))
    return fail(SDV_ELAYOUT, "Dk=%d Dv=%d: the preparation needs Dk = Dv in {64, 128}", Dk, Dv);
  if ((long)Hv * Dv > (1L << 26)) return fail(SDV_EINVAL, "Hv*Dv=%ld too large", (long)Hv * Dv);
  if (conv_act != SDV_CONV_NONE && conv_act != SDV_CONV_SILU) return fail(SDV_EINVAL, "conv_act=%d", conv_act);
  if (!(eps >= 0.0f && eps <= 3.4e38f)) return fail(SDV_ERANGE, "eps=%g must be finite and >= 0", (double)eps);
  return hip_status(sdv::gdn_verify_prep_layers_launch(static_cast<const sdv_gdn_layer*>(table), L, k, Hv, Hk, Dk,
                                                       conv_act, eps, (hipStream_t)stream),
                    "sdv_gdn_verify_prep_k_layers launch");
}

int sdv_gdn_verify_prep_norm_k(const float* S_in, const float* qkv, const float* hist, const float* conv_w,
                               const float* a, const float* b, const float* A_log, const float* dt_bias, int k,
                               int Hv, int Hk, int Dk, int Dv, int conv_act, float eps, float* window, float* y,
                               float* const* snaps, const float* z, const float* norm_w, int gate_act,
                               float norm_eps, float* out, int32_t* counters, sdv_stream_t stream) {
  int st;
  Range outs[SDV_MAX_ROWS + 4], ins[11];
  if ((st = check_verify_prep(S_in, qkv, hist, conv_w, a, b, A_log, dt_bias, k, Hv, Hk, Dk, Dv, conv_act, eps,
                              window, y, snaps, outs, ins)))
    return st;
  if (gate_act != SDV_GATE_SIGMOID && gate_act != SDV_GATE_SILU) return fail(SDV_EINVAL, "gate_act=%d", gate_act);
  if (!(norm_eps >= 0.0f && norm_eps <= 3.4e38f))
    return fail(SDV_ERANGE, "norm_eps=%g must be finite and >= 0", (double)norm_eps);
  if ((st = check_ptr(z, "z"))) return st;
  if ((st = check_ptr(norm_w, "norm_w"))) return st;
  if ((st = check_ptr(out, "out"))) return st;
  if (!counters) return fail(SDV_EINVAL, "counters is NULL");
  if ((uintptr_t)counters % 4) return fail(SDV_EINVAL, "counters is not 4-byte aligned");
  const size_t n = (size_t)k * Hv * Dv * 4;
  outs[k + 2] = {out, n, "out"};
  outs[k + 3] = {counters, (size_t)Hv * 4, "counters"};
  ins[8] = {z, n, "z"};
  ins[9] = {norm_w, (size_t)Dv * 4, "norm_w"};
  if ((st = check_alias(outs, k + 4, ins, 10))) return st;
  return hip_status(sdv::gdn_verify_prep_launch(S_in, qkv, hist, conv_w, a, b, A_log, dt_bias, k, Hv, Hk, Dk,
                                                conv_act, eps, window, y, snaps, (hipStream_t)stream, z, norm_w,
                                                gate_act, norm_eps, out, counters),
                    "sdv_gdn_verify_prep_norm_k launch");
}

int sdv_gdn_gated_norm_k(const float* y, const float* z, const float* w, int k, int Hv, int Dv, int gate_act,
                         float eps, float* out, sdv_stream_t stream) {
  int st;
  if ((st = check_width(k))) return st;
  if (Hv <= 0) return fail(SDV_EINVAL, "Hv=%d must be positive", Hv);
  if (Dv != 64 && Dv != 128) return fail(SDV_ELAYOUT, "Dv=%d: the output norm needs Dv in {64, 128}", Dv);
  if (gate_act != SDV_GATE_SIGMOID && gate_act != SDV_GATE_SILU) return fail(SDV_EINVAL, "gate_act=%d", gate_act);
  if (!(eps >= 0.0f && eps <= 3.4e38f)) return fail(SDV_ERANGE, "eps=%g must be finite and >= 0", (double)eps);
  if ((st = check_ptr(y, "y"))) return st;
  if ((st = check_ptr(z, "z"))) return st;
  if ((st = check_ptr(w, "w"))) return st;
  if ((st = check_ptr(out, "out"))) return st;
  const size_t n = (size_t)k * Hv * Dv * 4;
  Range outs[] = {{out, n, "out"}};
  Range ins[] = {{y, n, "y"}, {z, n, "z"}, {w, (size_t)Dv * 4, "w"}};
  if ((st = check_alias(outs, 1, ins, 3))) return st;
  return hip_status(sdv::gdn_gated_norm_launch(y, z, w, k, Hv, Dv, gate_act, eps, out, (hipStream_t)stream),
                    "sdv_gdn_gated_norm_k launch");
}

}  // extern "C"
