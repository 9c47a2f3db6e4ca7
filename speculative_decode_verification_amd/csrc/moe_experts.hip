// Fused expert MLP over the union of the rows' experts: for each (expert,
// 128-wide slice of the intermediate dimension) one workgroup runs the fused
// gate/up product with SwiGLU for that slice and then the down product over
// the same slice of its K dimension, writing one partial output per slice.
//
// The method reads each union expert's packed weights once for all rows routed
// to it, gate and up read together, then the gathered down projection
// (mere.run transfer report, "Exact verification kernels and benchmark
// admission"; Red Lite dev45, "What it is"; Flash-Next plan "2.3 MoE").
// Splitting the intermediate dimension into slices keeps SwiGLU's output in
// LDS (no round trip through HBM, no second launch) and lets each wave's load
// stream run on from the gate/up weights into the down weights, so the
// down-projection loads are in flight while the gate/up tail computes.  The
// slices' partial sums are added in slice order by the combine, so every
// output row depends only on its own activation row and the weights: width-k
// rows equal width-1 rows bit for bit.
//
// Workgroup (unit u, slice j), 8 waves:
//   phase A  wave w streams fused gate/up tile 8j + w (16 gate + 16 up
//            weight rows) over all H / 64 groups; its SwiGLU outputs go to
//            LDS already split into phase B's bf16 parts, with their sums.
//   phase B  wave w streams
//            down tiles w, w + 8, ... over the slice's two K groups and stores
//            each finished tile (32 outputs per row).  A 64-wide last slice
//            is padded with zero activations; its second group re-reads the
//            first group's weights, which then add exactly zero.
// Each wave's ring of 4 prefetched (codes, scale/bias) blocks (2 of Q8_0's
// 2 KB blocks) runs across the phase boundary.  Phase A is padded to a
// multiple of the ring (the padding steps re-read the tile's last block and
// compute nothing), so phase B starts at ring slot 0; every refill is
// unconditional (past the end of the stream it re-reads the last block),
// which keeps the load counter waits static.  The weights are affine Q4,
// Q8_0 or affine Q3 (the kernel is instantiated per format; only the block
// loads, the group step and the Q8_0 activation sums per 32 elements differ).
// Finished down tiles are written with five buffer stores (store i writes row
// i from the lanes of half 0 and row 4 + i from half 1; the fifth writes row
// 8); lanes without a row get an out-of-range offset, so each tile issues the
// same number of stores.

#include <atomic>

#include "q4_core.h"
#include "route_core.h"

namespace sdv {

namespace {

using namespace q4;

constexpr int kWaves = 8;
// blocks in flight per wave: 4 one-KB blocks, or 2 two-KB Q8_0 blocks (the
// same bytes and registers); a multiple of the slice's groups
template <int FMT>
constexpr int ring_of() { return FMT == SDV_FMT_Q8_0 ? 2 : 4; }
// activation sums per 64-element group: one, or one per 32-element Q8_0 block
template <int FMT>
constexpr int spg_of() { return FMT == SDV_FMT_Q8_0 ? 2 : 1; }
constexpr int kSlice = 128;      // intermediate columns per workgroup
constexpr int kSliceTiles = kSlice / 16;
constexpr uint32_t kBufferDword3 = 0x00020000u;  // raw buffer resource word 3 (gfx9 family)
constexpr int kDropOffset = 0x7FFFFFF0;          // beyond any partial buffer: the store is dropped

struct ExpertArgs {
  const uint4* gu_codes;  // fused gate/up bank [E][TA][GA][64] uint4
  const uint32_t* gu_sb;  // [E][TA][GA][32]
  const uint4* dn_codes;  // down bank [E][TB][GB][64]
  const uint32_t* dn_sb;
  const uint4* sgu_codes;  // shared expert (E = 1) or null
  const uint32_t* sgu_sb;
  const uint4* sdn_codes;
  const uint32_t* sdn_sb;
  const uint16_t* x;  // bf16 [k][H]
  const int32_t* union_ids;
  const int32_t* n_union;
  const int32_t* pair_off;
  const int32_t* pair_row;
  const int32_t* pair_slot;
  int E, H, I, k, topk;
  int TA, GA, TB, GB, S;
  float* partial;  // [S][k][topk + 1][H]
  uint32_t partial_bytes;
  int balance;     // more workgroups than compute units: issue priority from stream progress
  // the router dispatch inside the kernel (RPL > 0): its inputs, and the
  // global copies of its outputs (written by workgroup (0, 0))
  const float* logits;
  int mode, renorm;
  int32_t* r_idx;
  float* r_w;
  int32_t* r_union;
  int32_t* r_nu;
  int32_t* r_off;
  int32_t* r_row;
  int32_t* r_slot;
};

constexpr int kExpertThreads = 64 * kWaves;

// LDS scratch of the in-kernel router dispatch, at the start of the dynamic
// LDS (the x staging overwrites it after the dispatch): candidate keys, each
// wave's pool of 64 keys, row masks and counts over E, wave totals, the
// total, and per-row counts, softmax shifts and sums.
struct RouteScratchLayout {
  size_t cand, pool, rowmask, cnt, wave, total, nsel, mx, part, bytes;
};
__host__ __device__ inline RouteScratchLayout route_scratch(int E) {
  RouteScratchLayout l;
  l.cand = 0;
  l.pool = l.cand + (size_t)kPassRows * SDV_MAX_TOPK * 8;
  l.rowmask = l.pool + (size_t)kExpertThreads * 8;
  l.cnt = l.rowmask + (size_t)E * 4;
  l.wave = l.cnt + (size_t)E * 4;
  l.total = l.wave + (kExpertThreads / 64) * 4;
  l.nsel = l.total + 4;
  l.mx = l.nsel + kPassRows * 4;
  l.part = l.mx + kPassRows * 4;
  l.bytes = l.part + kPassRows * 4;
  return l;
}

struct Lds {
  size_t xs, xsum, hs, hpart, hrow, total;
};

// LDS layout: phase A's bf16 x rows and their group sums (spg per group);
// phase B's bf16 parts of h (written by phase A's epilogue, so they cannot
// share space with x rows that slower waves may still read), the per-wave
// partial group sums of h and the rows' group sums (spg per group).
__host__ __device__ inline Lds expert_lds(int k, int H, int spg) {
  Lds l;
  const size_t rsA = (size_t)H + 8, rsB = kSlice + 8;
  l.xs = 0;
  l.xsum = (size_t)(k + 1) * rsA * 2;
  l.hs = (l.xsum + (size_t)32 * (H / 64) * spg * 4 + 15) & ~(size_t)15;
  l.hpart = l.hs + (size_t)(3 * k + 1) * rsB * 2;
  l.hrow = l.hpart + (size_t)kPassRows * kSliceTiles * 4;
  l.total = l.hrow + (size_t)kPassRows * (kSlice / 64) * spg * 4;
  return l;
}

// One ring entry: the lane's code words of a (tile, group) block.  Q4: one
// 16-byte chunk of the 1 KB block; Q3: three words of the 768-byte block;
// Q8_0: two 16-byte chunks, one from each 1 KB half of the 2 KB block.
template <int FMT>
struct Blk {
  uint4 c;
};
template <>
struct Blk<SDV_FMT_Q8_0> {
  uint4 c, c2;
};

// Bytes of one (tile, group) block of the format.
template <int FMT>
constexpr int block_bytes() { return FMT == SDV_FMT_Q8_0 ? 2048 : (FMT == SDV_FMT_AFFINE_Q3 ? 768 : 1024); }

// The lane's part of the block that starts at byte address p.
template <int FMT>
__device__ __forceinline__ void load_block(Blk<FMT>& b, const unsigned char* p, int lane) {
  if constexpr (FMT == SDV_FMT_Q8_0) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
    b.c = load_nt(q + lane);  // weights: read once per call
    b.c2 = load_nt(q + 64 + lane);
  } else if constexpr (FMT == SDV_FMT_AFFINE_Q3) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(p) + lane;
    b.c = make_uint4(load_nt(w), load_nt(w + 64), load_nt(w + 128), 0u);
  } else {
    b.c = load_nt(reinterpret_cast<const uint4*>(p) + lane);
  }
}

// The group step of the format (q4_core.h): activation sums xr[i][s_idx]
// (Q4, Q3) or xr[i][2 s_idx + b] (Q8_0).
template <int ACT, int FMT>
__device__ __forceinline__ void block_mac(const Blk<FMT>& b, uint32_t sbw, const uint16_t* ap,
                                          const float* const (&xr)[5], int s_idx, float y[5], DecodeK dk) {
  if constexpr (FMT == SDV_FMT_Q8_0)
    group_mac_rows_q8<ACT>(b.c, b.c2, sbw, ap, xr, s_idx, y);
  else
    group_mac_rows<ACT, FMT>(b.c, sbw, ap, xr, s_idx, y, dk);
}

// A lane half reads elements 32 h .. of a Q4 or Q3 group, 8 h .. (every 16)
// of a Q8_0 group.
template <int FMT>
constexpr int half_offset() { return FMT == SDV_FMT_Q8_0 ? 8 : 32; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(float* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)bytes, (int)kBufferDword3);
}

// A wave's issue priority from its progress through its stream: 3 in the
// first quarter, down to 0 in the last.  Two workgroups that share a CU
// otherwise issue oldest first, and the second workgroup placed on a CU
// (which also learns its routing words later) falls behind and ends last;
// with the wave furthest behind issuing first, the two progress together
// (45.1-46.1 against 46.1-46.9 us per flashnext launch).  Used only when the
// grid is well above one workgroup per CU (balance_grid): with one workgroup
// per CU it measured slower (256-expert layers at 5 rows: 23.7-25.6 against
// 22.9-23.0 us; at 9 rows, 288 workgroups of which about 250 have a unit:
// 28.5-30.1 against 27.7-28.4 us).
// The quarters of a stream of `total` steps start at steps ceil(m total / 4),
// m = 1, 2, 3 (taken once per wave, so a round compares instead of dividing).
struct Quarters {
  int t1, t2, t3;
};
__device__ __forceinline__ Quarters quarters_of(int total) {
  return {(total + 3) >> 2, (2 * total + 3) >> 2, (3 * total + 3) >> 2};
}
__device__ __forceinline__ void prio_by_progress(int done, const Quarters& q) {
  if (done < q.t1) __builtin_amdgcn_s_setprio(3);  // wave-uniform
  else if (done < q.t2) __builtin_amdgcn_s_setprio(2);
  else if (done < q.t3) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Phase B of one wave: down tiles wave, wave + 8, ... over the slice's two
// groups.  The stream is padded to whole ring rounds, so every round is the
// same straight-line code (static load counter waits); padding steps compute
// tiles past the last one, whose stores are dropped.
template <int FMT, typename Issue>
__device__ __forceinline__ void phase_b(const ExpertArgs& a, const Blk<FMT> (&cbuf)[ring_of<FMT>()],
                                        const uint32_t (&sbuf)[ring_of<FMT>()],
                                        Issue& issue, const uint16_t* hs, const float* hrow, const int* s_dst,
                                        int nrows, int kr, int j, int wave, int lane, int s_begin, int s_end,
                                        DecodeK dk) {
  const int k = a.k, H = a.H;
  const int col = lane & 31, half = lane >> 5;
  const int rsB = kSlice + 8;
  const int slot = slot_of_arow<SDV_ACT_F32>(col, nrows);
  constexpr int kRing = ring_of<FMT>(), SPG = spg_of<FMT>();
  const uint16_t* ap = hs + (size_t)(slot >= 0 ? slot : 3 * kr) * rsB + half * half_offset<FMT>();
  const float* xr[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) xr[i] = hrow + (i < 4 ? 4 * half + i : 8) * 2 * SPG;
  const __amdgpu_buffer_rsrc_t rsrc = out_rsrc(a.partial, a.partial_bytes);
  // byte offset of the output row behind each of this lane's five
  // accumulators (rows 4 * half + i, and row 8), or -1
  int off[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int r = i < 4 ? 4 * half + i : 8;
    const int d = (r < nrows && (i < 4 || half == 0)) ? s_dst[r] : -1;
    off[i] = d >= 0 ? (int)(((size_t)j * k * (a.topk + 1) + d) * H * 4) : -1;
  }
  float y[5];
  int t = wave;
  const Quarters quarters = quarters_of(s_end);
  auto round = [&](int s0) {
    if (a.balance) prio_by_progress(s0, quarters);
#pragma unroll
    for (int i = 0; i < kRing; ++i) {
      // The slice's activations are the same for every tile; an opaque zero
      // offset (distinct per step, so never merged or hoisted, and free of
      // side effects, so the scheduler may still move it) keeps their LDS
      // reads in each step instead of holding them in registers across steps
      // (which would not fit beside the load ring).
      int z = __builtin_amdgcn_readfirstlane(s0 + i);
      asm("" : "+s"(z));
      z -= s0 + i;
      const int g = i & 1;  // ring rounds start at slot 0 and kRing is even
      if (g == 0) {
#pragma unroll
        for (int v = 0; v < 5; ++v) y[v] = 0.0f;
      }
      block_mac<SDV_ACT_F32, FMT>(cbuf[i], sbuf[i], ap + z + g * 64, xr, z + g, y, dk);
      issue(i, s0 + i + kRing);
      if (g == 1) {
        const int n = t * 32 + col;
#pragma unroll
        for (int v = 0; v < 5; ++v)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y[v]), rsrc,
                                                (off[v] >= 0 && n < H) ? off[v] + n * 4 : kDropOffset, 0, 0);
        t += kWaves;
      }
    }
  };
  // The first round is peeled: it enters with only loads outstanding, later
  // rounds with loads and stores, and separate code lets each keep exact
  // load counter waits.
  if (s_begin < s_end) round(s_begin);
  for (int s0 = s_begin + kRing; s0 < s_end; s0 += kRing) round(s0);
}

// WIDE (k > kPassRows): a unit is one pass of at most kPassRows of an
// expert's rows (pass blockIdx.z), and only those rows are staged.
// RPL > 0 (k <= kPassRows, E <= 512): every workgroup first runs the router
// dispatch itself (route_block, RPL candidates per lane) on the logits, so
// the routing needs no launch of its own; the results are identical in every
// workgroup, and workgroup (0, 0) writes them out for the combine.
template <bool WIDE, int RPL, int FMT>
__global__ __launch_bounds__(512, 4) void moe_experts_kernel(ExpertArgs a) {
  static_assert(!(WIDE && RPL > 0), "the in-kernel dispatch covers one pass of rows");
  static_assert(RPL == 0 || FMT == SDV_FMT_AFFINE_Q4, "the in-kernel dispatch is built for affine Q4 only");
  constexpr int kRing = ring_of<FMT>(), SPG = spg_of<FMT>();
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_src[kPassRows], s_dst[kPassRows];
  constexpr int kRS = RPL > 0 ? kPassRows * SDV_MAX_TOPK : 1;
  __shared__ int32_t s_r_idx[kRS], s_r_union[kRS], s_r_off[kRS + 1], s_r_row[kRS], s_r_slot[kRS], s_r_nu;
  __shared__ float s_r_w[kRS];
  const int H = a.H, GA = a.GA, GB = a.GB, k = a.k;
  const int kr = min(k, kPassRows);  // rows of the LDS staging; row kr is all zero
  const Lds L = expert_lds(kr, H, SPG);
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem + L.xs);
  float* xsum = reinterpret_cast<float*>(smem + L.xsum);
  uint16_t* hs = reinterpret_cast<uint16_t*>(smem + L.hs);
  float* hpart = reinterpret_cast<float*>(smem + L.hpart);
  float* hrow = reinterpret_cast<float*>(smem + L.hrow);
  const int rsA = H + 8, rsB = kSlice + 8;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;

  // ---- x rows: thread t stages group t % G of row t / G (its 64 elements are
  // contiguous, at element 64 t); the loads of the first k * G tasks go out
  // before anything else, since x does not depend on the routing.  All k rows
  // are staged, in x-row order; the unit's rows pick theirs through s_src.
  const int G = H >> 6;
  int nxt = k * G;
  constexpr int kThreads = kExpertThreads;
  uint4 xv[8];
  if constexpr (!WIDE) {
    const uint4* xp = reinterpret_cast<const uint4*>(a.x) + (size_t)min(tid, nxt - 1) * 8;
#pragma unroll
    for (int q = 0; q < 8; ++q) xv[q] = xp[q];
  }

  // ---- the router dispatch in the workgroup (RPL > 0)
  const int32_t* rt_union = a.union_ids;
  const int32_t* rt_nu = a.n_union;
  const int32_t* rt_off = a.pair_off;
  const int32_t* rt_row = a.pair_row;
  const int32_t* rt_slot = a.pair_slot;
  if constexpr (RPL > 0) {
    const RouteScratchLayout rl = route_scratch(a.E);
    const RouteSmem sm{s_r_idx,
                       reinterpret_cast<uint32_t*>(smem + rl.rowmask),
                       reinterpret_cast<int32_t*>(smem + rl.cnt),
                       reinterpret_cast<int32_t*>(smem + rl.wave),
                       reinterpret_cast<int32_t*>(smem + rl.total),
                       reinterpret_cast<uint64_t*>(smem + rl.cand),
                       reinterpret_cast<int32_t*>(smem + rl.nsel),
                       reinterpret_cast<float*>(smem + rl.mx),
                       reinterpret_cast<float*>(smem + rl.part),
                       reinterpret_cast<uint64_t*>(smem + rl.pool)};
    const RouteArgs ra{a.logits, k, a.E, a.topk, a.mode, a.renorm, s_r_idx, s_r_w, s_r_union, &s_r_nu,
                       s_r_off, s_r_row, s_r_slot};
    route_block<RPL, kExpertThreads>(ra, sm);
    __syncthreads();
    if (blockIdx.x == 0 && blockIdx.y == 0) {
      const int kt = k * a.topk;
      for (int t = tid; t < kt; t += kExpertThreads) {
        a.r_idx[t] = s_r_idx[t];
        a.r_w[t] = s_r_w[t];
        a.r_union[t] = s_r_union[t];
        a.r_row[t] = s_r_row[t];
        a.r_slot[t] = s_r_slot[t];
      }
      for (int t = tid; t <= kt; t += kExpertThreads) a.r_off[t] = s_r_off[t];
      if (tid == 0) *a.r_nu = s_r_nu;
    }
    rt_union = s_r_union;
    rt_nu = &s_r_nu;
    rt_off = s_r_off;
    rt_row = s_r_row;
    rt_slot = s_r_slot;
  }

  // ---- unit: a union expert's rows, or the shared expert's k rows.  The
  // routing words are loaded together before any is tested.
  // The shared expert (every row: the unit with the most staging and output)
  // takes grid row ysh, inside the first 192 workgroups in dispatch order,
  // instead of the last row: dispatched last, its workgroups shared CUs and
  // ended last (47.6-48.7 against 46.4-47.1 us per flashnext launch).  The
  // rows from ysh on shift up by one; unused units stay at the end.  Without
  // a shared expert the order is kept.
  const int ny = gridDim.y, ysh = a.sgu_codes ? min(ny - 1, 192 / (int)gridDim.x) : ny - 1;
  const int u = blockIdx.y == ysh ? ny - 1 : (int)blockIdx.y - ((int)blockIdx.y > ysh), j = blockIdx.x;
  const int pass0 = WIDE ? (int)blockIdx.z * kPassRows : 0;
  const bool shared = u == k * a.topk;
  int e = 0, p0 = 0, nrows = k;
  const uint4* guc = a.gu_codes;
  const uint32_t* gus = a.gu_sb;
  const uint4* dnc = a.dn_codes;
  const uint32_t* dns = a.dn_sb;
  if (shared) {
    if (!a.sgu_codes) return;
    guc = a.sgu_codes;
    gus = a.sgu_sb;
    dnc = a.sdn_codes;
    dns = a.sdn_sb;
    if constexpr (WIDE) {
      nrows = min(k - pass0, kPassRows);
      if (nrows <= 0) return;
    }
  } else {
    int nu = __builtin_amdgcn_readfirstlane(*rt_nu);
    int e0 = __builtin_amdgcn_readfirstlane(rt_union[u]);
    int q0 = __builtin_amdgcn_readfirstlane(rt_off[u]);
    int q1 = __builtin_amdgcn_readfirstlane(rt_off[u + 1]);
    asm volatile("" : "+s"(nu), "+s"(e0), "+s"(q0), "+s"(q1));  // all four in flight together
    if (u >= nu || e0 < 0 || e0 >= a.E) return;
    if (q0 < 0 || q1 <= q0 || q1 > k * a.topk) return;
    q0 += pass0;
    nrows = min(q1 - q0, WIDE ? kPassRows : k);
    if (nrows <= 0) return;
    e = __builtin_amdgcn_readfirstlane(e0);
    p0 = __builtin_amdgcn_readfirstlane(q0);
    nrows = __builtin_amdgcn_readfirstlane(nrows);
  }

  // ---- slice geometry and this wave's stream
  const int i0 = j * kSlice;
  const int sw = min(kSlice, a.I - i0);  // 64 or 128
  const int tilesA = sw / 16;
  const int gB0 = i0 / 64;                // first down group of the slice
  const int gBlast = a.GB - 1;
  const int nA = wave < tilesA ? GA : 0;
  const int nA8 = (nA + kRing - 1) / kRing * kRing;
  const int tilesB = wave < a.TB ? (a.TB - wave + kWaves - 1) / kWaves : 0;
  const int nB = tilesB * 2;
  const int nB8 = (nB + kRing - 1) / kRing * kRing;
  const int total = __builtin_amdgcn_readfirstlane(nA8 + nB8);
  const size_t baseA = ((size_t)e * a.TA + (size_t)j * kSliceTiles + wave) * GA;  // block of step 0
  const size_t baseB = ((size_t)e * a.TB + min(wave, a.TB - 1)) * GB;

  Blk<FMT> cbuf[kRing];
  uint32_t sbuf[kRing];
  // Load the (codes, scale/bias) block of stream step s into ring slot `slot`.
  // Steps past the end re-read the last block; a wave without blocks reads
  // the first block of its last down tile, so every wave issues the same
  // loads in the same order.
  // The block is selected without branches, so a ring round is one
  // straight-line block the compiler can schedule across steps.
  // Each phase's step-0 block as a byte address (codes) and its sb line,
  // taken once, so a refill adds a 32-bit block offset to one of two bases.
  const unsigned char* const cA = reinterpret_cast<const unsigned char*>(guc) + baseA * block_bytes<FMT>();
  const unsigned char* const cB = reinterpret_cast<const unsigned char*>(dnc) + baseB * block_bytes<FMT>();
  const uint32_t* const sA = gus + baseA * 32;
  const uint32_t* const sB = dns + baseB * 32;
  const int strideB = kWaves * GB;  // blocks from one of the wave's down tiles to its next
  auto issue = [&](int slot, int s) {
    s = max(min(s, total - 1), 0);
    const bool inA = s < nA8;                               // then nA > 0
    const int q = max(min(s - nA8, nB - 1), 0);
    // a 64-wide slice re-reads its only group
    const int off = inA ? min(s, nA - 1) : (q >> 1) * strideB + min(gB0 + (q & 1), gBlast);
    load_block<FMT>(cbuf[slot], (inA ? cA : cB) + (unsigned)off * (unsigned)block_bytes<FMT>(), lane);
    sbuf[slot] = load_nt((inA ? sA : sB) + (unsigned)off * 32u + col);
  };
  // the unit's (row, slot) pairs go out before the ring, so waiting for them
  // does not wait for the ring (loads complete in issue order)
  // (every lane loads, at a clamped index in [p0, p0 + nrows); the shared
  // unit's are not used).
  const int pq = p0 + min(tid, nrows - 1);
  const int pr = rt_row[pq], ps = rt_slot[pq];
  // WIDE: the x rows of this pass's rows only, staged in pass order (the
  // pair rows are loaded first: the x addresses depend on them)
  auto x_src = [&](int i) {  // x row of staged row i
    if (shared) return pass0 + i;
    const int r = rt_row[p0 + i];
    return min(max(r, 0), k - 1);
  };
  if constexpr (WIDE) {
    nxt = nrows * G;
    const int t = min(tid, nxt - 1), i = t / G;
    const uint4* xp = reinterpret_cast<const uint4*>(a.x) + ((size_t)x_src(i) * G + (t - i * G)) * 8;
#pragma unroll
    for (int q = 0; q < 8; ++q) xv[q] = xp[q];
  }
#pragma unroll
  for (int i = 0; i < kRing; ++i) issue(i, i);

  // ---- phase A staging (the ring loads are already in flight): the all-zero
  // rows (MFMA rows without data read them)
  for (int t = tid; t < rsA / 2; t += kThreads) reinterpret_cast<uint32_t*>(xs + (size_t)kr * rsA)[t] = 0u;
  for (int t = tid; t < rsB / 2; t += kThreads) reinterpret_cast<uint32_t*>(hs + (size_t)3 * kr * rsB)[t] = 0u;
  for (int t = tid; t < G * SPG; t += kThreads) xsum[kr * G * SPG + t] = 0.0f;
  // One task = (x row i, group g): its 8 blocks of 8 elements are stored in NU
  // order and summed in order, and the group sum adds the 8 block sums
  // pairwise ((b0 + b1) + (b2 + b3)) + ((b4 + b5) + (b6 + b7)).
  auto put = [&](int t, const uint4 (&v)[8]) {
    const int i = t / G, g = t - i * G;
    float bsum[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t e8[8] = {v[q].x & 0xFFFFu, v[q].x >> 16, v[q].y & 0xFFFFu, v[q].y >> 16,
                              v[q].z & 0xFFFFu, v[q].z >> 16, v[q].w & 0xFFFFu, v[q].w >> 16};
      float acc = 0.0f;
#pragma unroll
      for (int c = 0; c < 8; ++c) acc = acc + bf16_bits_to_f32(e8[c]);
      bsum[q] = acc;
      *reinterpret_cast<uint4*>(xs + (size_t)i * rsA + g * 64 + q * 8) = nu_pack(e8);
    }
    if constexpr (SPG == 2) {
      // Q8_0: one sum per 32-element block, each added pairwise
      xsum[(i * G + g) * 2] = (bsum[0] + bsum[1]) + (bsum[2] + bsum[3]);
      xsum[(i * G + g) * 2 + 1] = (bsum[4] + bsum[5]) + (bsum[6] + bsum[7]);
    } else {
      xsum[i * G + g] = ((bsum[0] + bsum[1]) + (bsum[2] + bsum[3])) + ((bsum[4] + bsum[5]) + (bsum[6] + bsum[7]));
    }
  };
  if (tid < nxt) put(tid, xv);
  for (int t = tid + kThreads; t < nxt; t += kThreads) {
    const int i = t / G;
    const uint4* xp = reinterpret_cast<const uint4*>(a.x) + (WIDE ? ((size_t)x_src(i) * G + (t - i * G)) : (size_t)t) * 8;
    uint4 v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = xp[q];
    put(t, v);
  }
  // the unit's rows, after the x tasks (whose loads went out first), so the
  // wait for the (row, slot) pairs overlaps that work
  if (tid < kPassRows) {
    int src = -1, dst = -1;
    if (tid < nrows) {
      if (!shared) {
        const int r = pr, s = ps;
        if (r >= 0 && r < k && s >= 0 && s < a.topk) {
          src = WIDE ? tid : r;
          dst = r * (a.topk + 1) + s;
        }
      } else {
        src = tid;
        dst = (pass0 + tid) * (a.topk + 1) + a.topk;
      }
    }
    s_src[tid] = src;
    s_dst[tid] = dst;
  }
  __syncthreads();
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): enter the stream with no load outstanding

  const DecodeK dk = decode_k();
  // ---- phase A: one fused gate/up tile over all GA groups
  {
    const int src = col < nrows ? s_src[col] : -1;
    const uint16_t* ap = xs + (size_t)(src >= 0 ? src : kr) * rsA + half * half_offset<FMT>();
    // group sums of the x row behind each accumulator (row k is all zero)
    const float* xr[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int r = i < 4 ? 4 * half + i : 8;
      const int sr = r < nrows ? s_src[r] : -1;
      xr[i] = xsum + (sr >= 0 ? sr : kr) * G * SPG;
    }
    float y[5] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    // whole rounds, then a last round whose steps past nA compute nothing
    const int nAfull = nA / kRing * kRing;
    const Quarters quarters = quarters_of(total);
    for (int s0 = 0; s0 < nAfull; s0 += kRing) {
      if (a.balance) prio_by_progress(s0, quarters);
#pragma unroll
      for (int i = 0; i < kRing; ++i) {
        const int s = s0 + i;
        block_mac<SDV_ACT_BF16, FMT>(cbuf[i], sbuf[i], ap + s * 64, xr, s, y, dk);
        issue(i, s + kRing);
      }
    }
    if (nAfull < nA8) {
#pragma unroll
      for (int i = 0; i < kRing; ++i) {
        const int s = nAfull + i;
        if (s < nA) block_mac<SDV_ACT_BF16, FMT>(cbuf[i], sbuf[i], ap + s * 64, xr, s, y, dk);
        issue(i, s + kRing);
      }
    }
    // SwiGLU of this wave's 16 intermediate columns (gate in columns 0-15,
    // the matching up rows in columns 16-31), written straight into phase
    // B's activation rows: the three bf16 parts of each value at its slot in
    // the NU order of its 8-column block, and the 16 columns' sum per row.
    // Columns past a 64-wide slice's end are zero.
    const int c16 = col & 15;
    const int n = wave * 16 + c16;                              // column in the slice
    const int hpos = (n & ~7) + ((n & 7) < 4 ? 2 * (n & 7) : 2 * (n & 7) - 7);
#pragma unroll
    for (int r = 0; r < kPassRows; ++r) {
      if (r < nrows && wave < kSliceTiles) {
        float h = 0.0f;
        if (nA > 0) {
          const float g = rows_value(y, r);
          const float up = __shfl_xor(g, 16);
          h = siluf_(g) * up;
        }
        const float sum16 = row16_sum(h);                        // lanes 0-15 and 32-47 hold columns
        if (half == rows_half(r) && col < 16) {
          const uint32_t hi = f32_to_bf16_rne(h);
          const float r1 = h - bf16_bits_to_f32(hi);
          const uint32_t mi = f32_to_bf16_rne(r1);
          const float r2 = r1 - bf16_bits_to_f32(mi);
          const uint32_t lo = f32_to_bf16_rne(r2);
          hs[(size_t)(3 * r + 0) * rsB + hpos] = (uint16_t)hi;
          hs[(size_t)(3 * r + 1) * rsB + hpos] = (uint16_t)mi;
          hs[(size_t)(3 * r + 2) * rsB + hpos] = (uint16_t)lo;
          if (col == 0) hpart[r * kSliceTiles + wave] = sum16;
        }
      }
    }
  }
  __syncthreads();  // every wave's part of h is in LDS
  // each row's group sums: the four 16-column partial sums of the group, in
  // order (Q8_0: the two of each 32-element block)
  if constexpr (SPG == 2) {
    if (tid < kPassRows * 4) {
      const int r = tid >> 2, b = tid & 3;
      const float* hp = hpart + r * kSliceTiles + 2 * b;
      hrow[r * 4 + b] = r < nrows ? hp[0] + hp[1] : 0.0f;
    }
  } else {
    if (tid < kPassRows * 2) {
      const int r = tid >> 1, g = tid & 1;
      const float* hp = hpart + r * kSliceTiles + 4 * g;
      hrow[r * 2 + g] = r < nrows ? (hp[0] + hp[1]) + (hp[2] + hp[3]) : 0.0f;
    }
  }
  __syncthreads();

  // ---- phase B: down tiles over the slice's groups
  phase_b<FMT>(a, cbuf, sbuf, issue, hs, hrow, s_dst, nrows, kr, j, wave, lane, nA8, total, dk);
}

}  // namespace

int expert_slices(int I) { return (I + kSlice - 1) / kSlice; }

// a unit stages at most min(k, kPassRows) rows (one pass of its rows)
size_t expert_lds_bytes(int k, int H, int fmt) {
  return expert_lds(k < kPassRows ? k : kPassRows, H, fmt == SDV_FMT_Q8_0 ? 2 : 1).total;
}

size_t expert_partial_bytes(int k, int topk, int H, int I) {
  return (size_t)expert_slices(I) * k * (topk + 1) * H * 4;
}

namespace {

// Raise the kernel's dynamic LDS limit once per process (the largest size
// asked for so far; the attribute is per function, not per device).
template <bool WIDE, int RPL, int FMT>
hipError_t raise_lds_limit(size_t lds) {
  static std::atomic<size_t> lds_limit{65536};
  size_t cur = lds_limit.load(std::memory_order_relaxed);
  if (lds > cur) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(moe_experts_kernel<WIDE, RPL, FMT>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    while (cur < lds && !lds_limit.compare_exchange_weak(cur, lds)) {
    }
  }
  return hipSuccess;
}

template <bool WIDE, int RPL, int FMT = SDV_FMT_AFFINE_Q4>
hipError_t launch_experts(const ExpertArgs& a, dim3 grid, size_t lds, hipStream_t st) {
  const hipError_t err = raise_lds_limit<WIDE, RPL, FMT>(lds);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((moe_experts_kernel<WIDE, RPL, FMT>), grid, dim3(kExpertThreads), lds, st, a);
  return hipGetLastError();
}

// Whether the launch takes the progress priorities: a grid over 5/4 of the
// compute units (units past the union exit at once, so a grid just above one
// workgroup per CU still leaves most CUs with one working workgroup), and
// within the two workgroups per CU that are resident at once.  With more
// rounds of workgroups, the new workgroups' high priority holds back the
// older ones that would free their slots (16 rows, 3,220 workgroups in two
// passes: 84.2-84.3 against 80.4-82.1 us).
bool balance_grid(dim3 grid) {
  const long n = (long)grid.x * grid.y * grid.z, cus = device_cus();
  return n * 4 > cus * 5 && n <= 2 * cus;
}

ExpertArgs expert_args(const sdv_q4t& gu, const sdv_q4t& dn, const sdv_q4t* sgu, const sdv_q4t* sdn, const void* x,
                       int k, int topk, float* partial) {
  ExpertArgs a{};
  a.gu_codes = static_cast<const uint4*>(gu.codes);
  a.gu_sb = gu.sb;
  a.dn_codes = static_cast<const uint4*>(dn.codes);
  a.dn_sb = dn.sb;
  a.sgu_codes = sgu ? static_cast<const uint4*>(sgu->codes) : nullptr;
  a.sgu_sb = sgu ? sgu->sb : nullptr;
  a.sdn_codes = sdn ? static_cast<const uint4*>(sdn->codes) : nullptr;
  a.sdn_sb = sdn ? sdn->sb : nullptr;
  a.x = static_cast<const uint16_t*>(x);
  a.E = gu.E;
  a.H = gu.K;
  a.I = dn.K;
  a.k = k;
  a.topk = topk;
  a.TA = (a.I + 15) / 16;
  a.GA = a.H / 64;
  a.TB = (a.H + 31) / 32;
  a.GB = a.I / 64;
  a.S = expert_slices(a.I);
  a.partial = partial;
  a.partial_bytes = (uint32_t)expert_partial_bytes(k, topk, a.H, a.I);
  return a;
}

}  // namespace

hipError_t moe_experts_launch(const sdv_q4t& gu, const sdv_q4t& dn, const sdv_q4t* sgu, const sdv_q4t* sdn,
                              const void* x, const int32_t* union_ids, const int32_t* n_union,
                              const int32_t* pair_off, const int32_t* pair_row, const int32_t* pair_slot, int k,
                              int topk, float* partial, hipStream_t st) {
  ExpertArgs a = expert_args(gu, dn, sgu, sdn, x, k, topk, partial);
  a.union_ids = union_ids;
  a.n_union = n_union;
  a.pair_off = pair_off;
  a.pair_row = pair_row;
  a.pair_slot = pair_slot;
  const size_t lds = expert_lds_bytes(k, a.H, gu.format);
  const int units = k * topk + (sgu ? 1 : 0);
  // every width takes the pass form: a unit stages only its own x rows,
  // after its pair loads (about 1.1 rows per routed unit at nine rows,
  // instead of all k)
  const int passes = (k + kPassRows - 1) / kPassRows;
  const dim3 grid(a.S, units, passes);
  a.balance = balance_grid(grid);
  switch (gu.format) {
    case SDV_FMT_AFFINE_Q4: return launch_experts<true, 0, SDV_FMT_AFFINE_Q4>(a, grid, lds, st);
    case SDV_FMT_Q8_0: return launch_experts<true, 0, SDV_FMT_Q8_0>(a, grid, lds, st);
    case SDV_FMT_AFFINE_Q3: return launch_experts<true, 0, SDV_FMT_AFFINE_Q3>(a, grid, lds, st);
    default: return hipErrorInvalidValue;
  }
}

// Whether the router dispatch runs inside the expert kernel: one pass of
// rows and at most one expert per thread of its workgroup.
bool route_in_experts(int k, int E) { return k <= kPassRows && E <= kExpertThreads; }

size_t route_experts_lds_bytes(int k, int E, int H) {
  const size_t a = expert_lds_bytes(k, H, SDV_FMT_AFFINE_Q4), b = route_scratch(E).bytes;
  return a > b ? a : b;
}

hipError_t route_launch(const float* logits, int k, int E, int topk, int mode, int renorm, int32_t* idx, float* w,
                        int32_t* union_ids, int32_t* n_union, int32_t* pair_off, int32_t* pair_row,
                        int32_t* pair_slot, hipStream_t st);

hipError_t moe_route_experts_launch(const float* logits, int mode, int renorm, const sdv_q4t& gu,
                                    const sdv_q4t& dn, const sdv_q4t* sgu, const sdv_q4t* sdn, const void* x, int k,
                                    int topk, int32_t* idx, float* w, int32_t* union_ids, int32_t* n_union,
                                    int32_t* pair_off, int32_t* pair_row, int32_t* pair_slot, float* partial,
                                    hipStream_t st) {
  const int E = gu.E;
  if (!route_in_experts(k, E)) {
    // two launches: the router dispatch, then the experts reading its outputs
    const hipError_t e = route_launch(logits, k, E, topk, mode, renorm, idx, w, union_ids, n_union, pair_off,
                                      pair_row, pair_slot, st);
    if (e != hipSuccess) return e;
    return moe_experts_launch(gu, dn, sgu, sdn, x, union_ids, n_union, pair_off, pair_row, pair_slot, k, topk,
                              partial, st);
  }
  ExpertArgs a = expert_args(gu, dn, sgu, sdn, x, k, topk, partial);
  a.logits = logits;
  a.mode = mode;
  a.renorm = renorm;
  a.r_idx = idx;
  a.r_w = w;
  a.r_union = union_ids;
  a.r_nu = n_union;
  a.r_off = pair_off;
  a.r_row = pair_row;
  a.r_slot = pair_slot;
  const size_t lds = route_experts_lds_bytes(k, E, a.H);
  const dim3 grid(a.S, k * topk + (sgu ? 1 : 0));
  a.balance = balance_grid(grid);
  const int per_lane = (E + 63) / 64;
  if (per_lane <= 1) return launch_experts<false, 1>(a, grid, lds, st);
  if (per_lane <= 2) return launch_experts<false, 2>(a, grid, lds, st);
  if (per_lane <= 4) return launch_experts<false, 4>(a, grid, lds, st);
  return launch_experts<false, 8>(a, grid, lds, st);
}

}  // namespace sdv
