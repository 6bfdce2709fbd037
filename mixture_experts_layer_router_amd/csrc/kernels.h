// Host-side launchers of the gfx950 kernels (internal interface between the
// C ABI in api.hip and the kernel translation units).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

enum WFmt { W_BF16 = 0, W_FP8_B128 = 1, W_MXFP8 = 2 };
enum AFmt { A_NONE = 0, A_FP8_1X128 = 1, A_MXFP8_1X32 = 2 };

// ------------------------------------------------------------------ routing
struct RouteParams {
  int H, E, G, TG, K;
  float scale;
};
// Small-T router logits: one workgroup per expert row.  T <= kRouteGemvMaxT.
constexpr int kRouteGemvMaxT = 8;
hipError_t launch_route_logits(const uint16_t* x, int T, const uint16_t* wr, const RouteParams& p,
                               float* logits, hipStream_t s);
// Top-k over precomputed fp32 logits [T][E] (bias added here).  The logits
// may come as nslice partial sums at stride slice_stride (elements), added in
// slice order.
hipError_t launch_topk(const float* logits, int T, const float* bias, const RouteParams& p, int* ids,
                       float* w, hipStream_t s, int nslice = 1, long slice_stride = 0);
constexpr int kRouterMaxSplit = 16;  // K slices of the batched router GEMM

// Batched routing in one launch (route_fused.hip): optional stage M RMSNorm,
// router, top-k, the routed-format input and per-block expert counts, one
// workgroup per kRouteBlock tokens.
constexpr int kRouteBlock = 16;
struct RouteFusedParams {
  const uint16_t* h;      // bf16 [T][H]: the layer input x, or the pre-norm h when gamma is set
  const uint16_t* gamma;  // bf16 [H] norm weight, or null (no norm)
  float eps;
  int T, H;
  const uint16_t* wr;     // bf16 [E][H]
  const float* bias;      // fp32 [E] or null
  RouteParams rp;
  int* ids;               // [T][K]
  float* w;               // [T][K]
  uint16_t* x_out;        // bf16 [T][H] normalised x (or a copy of x), or null
  int afmt;               // format of xq / xqs
  void* xq;               // codes u8 [T][H] in afmt (FP8_1X128 / MXFP8_1X32), or null
  void* xqs;              // their scales
  int* hist;              // int32 [ceil(T/kRouteBlock)][E] slot counts per block, or null
  // K split: each block of kRouteBlock tokens is routed by `slices` workgroups
  // over contiguous ranges of H; they hand their partial logits over in
  // `part` (fp32 [blocks][slices][kRouteBlock][E]) and the last one (per the
  // counter of the block in `ctr`, zero between calls) adds them in slice order
  int slices;             // 1: no split
  float* part;
  unsigned* ctr;
};
hipError_t launch_route_fused(const RouteFusedParams& p, hipStream_t s);
// Stage M alone: x = bf16 RMSNorm(h) * gamma (the rounding of route_fused).
hipError_t launch_rmsnorm_rows(const uint16_t* h, const uint16_t* gamma, float eps, int T, int H, uint16_t* x,
                               hipStream_t s);

// ------------------------------------------------------------------ dispatch
// ids [TK]; writes offsets [E+1], perm_src [TK], inv_pos [TK]; when tiles is
// non-null also the grouped-GEMM tile list for row tiles of `bm` rows:
// tiles[2i] = expert, tiles[2i+1] = row offset in the segment; ntiles[0] = count.
// hist: int32 scratch of permute_hist_ints(TK, E) entries.
constexpr size_t permute_hist_ints(int TK, int E) { return size_t((TK + 1023) / 1024) * size_t(E); }
hipError_t launch_permute(const int* ids, int TK, int E, int* hist, int* offsets, int* perm_src, int* inv_pos,
                          int* tiles, int* ntiles, int bm, hipStream_t s);
// The scatter alone, with counts given as hist rows of `fine` slots each
// (fine <= 1024; row i counts slots [i*fine, (i+1)*fine)).
hipError_t launch_permute_scatter(const int* ids, int TK, int E, const int* hist, int fine, int* offsets,
                                  int* perm_src, int* inv_pos, int* tiles, int* ntiles, int bm, hipStream_t s);
hipError_t launch_validate_dispatch(const int* ids, int TK, int E, const int* offsets, const int* perm, const int* inv,
                                   const int* tiles, const int* ntiles, int maxt, int bm, int* flags, hipStream_t s);
hipError_t launch_build_tiles(const int* offsets, int E, int rows, int bm, int* tiles, int* ntiles, hipStream_t s);
constexpr int kGemmBM = 128;   // rows per tile of the 128-row grouped GEMM (gemm.hip)
constexpr int kGemm2BM = 256;  // main rows per tile of the large-tile grouped GEMM (gemm2.hip)
inline int max_tiles(int rows, int E, int bm) { return (rows + bm - 1) / bm + E; }
// Rows one tile of the large-tile kernel can hold: its 256 main rows plus one
// extra 32-row MFMA block, which the waves compute against the B operands
// they already hold.
constexpr int kGemm2Rows = 288;
// Number of tiles and row offset step of one expert's grouped-GEMM tiles.
// 128-row kernel: ceil(cnt / bm) tiles of bm rows.  Large-tile kernel: an
// expert of at most kGemm2Rows rows is one tile (so the 256 +- 16 rows of a
// flat 2,048-token layer stream each weight panel once, where a 256-row tile
// plus a 16-row tail streamed it twice: a tail tile is bound by its weight
// loads, not its MFMAs); larger experts get ceil(cnt / kGemm2Rows) tiles that
// share the rows evenly in multiples of 32 (one MFMA row block), so 600 rows
// run as 224 + 224 + 152.  Every tile holds at least one row; where an even
// split cannot guarantee that, the tiles fall back to 256-row steps.
__host__ __device__ inline int tile_split(int cnt, int bm, int* step) {
  if (cnt <= 0) {
    *step = bm;
    return 0;
  }
  if (bm != kGemm2BM) {
    *step = bm;
    return (cnt + bm - 1) / bm;
  }
  const int n = (cnt + kGemm2Rows - 1) / kGemm2Rows;
  if (n == 1) {
    *step = kGemm2Rows;
    return 1;
  }
  const int h = ((cnt + n - 1) / n + 31) / 32 * 32;
  if ((n - 1) * h < cnt) {
    *step = h;
    return n;
  }
  *step = bm;
  return (cnt + bm - 1) / bm;
}
__host__ __device__ inline int tile_count(int cnt, int bm) {
  int step;
  return tile_split(cnt, bm, &step);
}
__host__ __device__ inline int tile_step(int cnt, int bm) {
  int step;
  tile_split(cnt, bm, &step);
  return step;
}

// ------------------------------------------------------------------ quantisers
// Row r of the output reads input row (row_map ? row_map[r] / row_div : r).
// in: bf16 (in_f32 = false) or fp32.  Modes:
//   A_NONE: copy as bf16 to q (as uint16) [rows][H]
//   A_FP8_1X128 / A_MXFP8_1X32: codes u8 to q, scales to qs
// When deq_out is non-null the dequantised values (code * scale, or the
// bf16/fp32 value itself for A_NONE) are written there as fp32 instead.
hipError_t launch_quant_rows(const void* in, bool in_f32, int rows, int H, const int* row_map, int row_div,
                             int afmt, void* q, void* qs, float* deq_out, hipStream_t s);

// codes u8 [rows][H] + scales (afmt layout) -> fp32 code * scale
hipError_t launch_dequant_rows(const uint8_t* q, const void* qs, int afmt, int rows, int H, float* out, hipStream_t s);

// ------------------------------------------------------------------ grouped GEMM (MFMA)
enum Epi { EPI_F32 = 0, EPI_BF16 = 1, EPI_GATEUP = 2 };
struct GemmParams {
  // A: rows of K elements; bf16 for W_BF16, e4m3 codes otherwise
  const void* A;
  long lda;          // elements
  const void* As;    // A scales (fp32 [rows][K/128] or e8m0 [rows][K/32]); null for bf16
  const int* a_map;  // optional gather: physical row = a_map[r] / a_div
  int a_div;
  // B: per group [N][K] (gate in B0, up in B1 for EPI_GATEUP)
  const void* B0;
  const void* B1;
  long b_stride;  // elements per group
  const void* B0s;
  const void* B1s;
  long bs_stride;  // scale elements per group
  int N;           // output columns (h columns for EPI_GATEUP)
  int K;
  // rows: segments seg[g]..seg[g+1] (seg null: one group of M rows)
  const int* seg;
  int M;
  const int* tiles;  // device tile list (null: tiles are 0..ceil(M/BM)-1 of group 0)
  const int* ntiles;
  int max_tiles;
  // output
  void* C;
  long ldc;
  void* Cs;       // scales of quantised h (EPI_GATEUP with out_afmt != A_NONE)
  int out_afmt;   // EPI_GATEUP: A_NONE -> bf16 h; else quantised h
  float* C_f32;   // EPI_GATEUP only: if non-null, h is written as fp32 here instead
  // EPI_F32 only: the K steps are split into ksplit slices (0 or 1: none); slice
  // z writes its partial product to C + z * c_split (elements)
  int ksplit;
  long c_split;
  // rows per tile the tile list was built for: kGemm2BM selects the large-tile
  // kernel (gemm2.hip), anything else the 128-row kernel (gemm.hip).  Without
  // a tile list the launcher picks the kernel (gemm2_chosen).
  int bm;
};
constexpr int kGemmMaxK = 8192;  // FP8_B128 GEMM: K (elements) <= this
hipError_t launch_gemm(int wfmt, int epi, const GemmParams& p, hipStream_t s);
// large-tile kernel: bf16, and MXFP8 with K a multiple of 512
bool gemm2_serves(int wfmt, int K, int epi, int out_afmt, int ksplit);
// whether launch_gemm runs p on the large-tile kernel: with a tile list when it
// was built for kGemm2BM; without one when that kernel serves the format and
// its tiles still fill the chip
bool gemm2_chosen(int wfmt, int epi, const GemmParams& p);
hipError_t launch_gemm2(int wfmt, int epi, const GemmParams& p, hipStream_t s);
// two bf16-output GEMMs of the large-tile kernel in one launch, p1's tiles
// first (both must be ones gemm2_chosen picks)
hipError_t launch_gemm2_dual(int wf1, const GemmParams& p1, int wf2, const GemmParams& p2, hipStream_t s);
// rows per tile of an expert FFN's two GEMMs (gate/up with K = H, down with K = I)
inline int ffn_tile_rows(int wfmt, int H, int I) {
  return (wfmt == W_BF16 || (wfmt == W_MXFP8 && H % 512 == 0 && I % 512 == 0)) ? kGemm2BM : kGemmBM;
}

// ------------------------------------------------------------------ small-batch GEMV FFN
struct GemvUpParams {
  int wfmt;
  const void* x;      // bf16 [T][H] (x_f32 false) or fp32 dequantised [T][H]
  bool x_f32;
  int T, H;
  // routed slots (T*K of them): expert = ids[slot], token = slot / K
  const int* ids;     // null: no routed slots
  int K;
  const void *g, *u, *gs, *us;  // routed weights
  int I;
  float* h;           // fp32 [T*K][I]
  // shared expert on every token
  const void *sg, *su, *sgs, *sus;
  int swfmt;
  int Is;
  float* hs;          // fp32 [T][Is]
  const void* xs;     // x for the shared expert (may differ in quantisation)
  bool xs_f32;
  // per-slot rows when the routed slots are "rows" of an explicit segment
  // list (moe_expert_ffn): expert of row r from seg; token = r
  const int* seg;
  int E;
};
hipError_t launch_gemv_gate_up(const GemvUpParams& p, hipStream_t s);

struct GemvDownParams {
  int wfmt, swfmt;
  int T, H, K, I, Is;
  const int* ids;      // [T][K] experts (null: only the shared part / explicit seg mode)
  const float* w;      // [T][K] routing weights (combine mode)
  const float* h;      // fp32 [T*K][I] (routed)
  const float* hs;     // fp32 [T][Is] (shared) or null
  const void *d, *ds;  // routed down [E][H][I] + scales
  const void *sd, *sds;
  // combine mode: out bf16 [T][H] = sum_j w*Y_j + S.  Per-row mode (out null):
  // y fp32 [rows][H] = h_row . Wd_e, expert from seg (or shared when seg null
  // and ids null)
  uint16_t* out;
  float* y;
  int rows;
  const int* seg;
  int E;
  const float* ys_add;  // combine mode: fp32 [T][H] added before the rounding (shared output), or null
};
hipError_t launch_gemv_down(const GemvDownParams& p, hipStream_t s);

// Small-T layer in four launches whose dependencies are hidden behind
// independent work (no device-wide synchronisation inside a launch):
//   stage 1: router logits || shared gate/up
//   stage 2: top-k || shared down (-> ysh)
//   then routed gate/up (launch_gemv_gate_up) and routed down + combine
//   (launch_gemv_down with ys_add = ysh).
struct DecodeParams {
  const uint16_t* x;  // bf16 [T][H] (router input; the pre-norm h when gamma is set)
  const uint16_t* gamma;  // single launch only: stage M norm weight bf16 [H], or null (must be null
                          // when T * H * 2 > kFusedXLdsMax: x is then read already normalised)
  float eps;
  uint16_t* x_out;        // single launch only: the normalised x, bf16 [T][H], or null
  int T, H;
  const uint16_t* wr;
  const float* bias;
  RouteParams rp;
  float* logits;  // [T][E]
  int* ids;       // [T][K]
  float* w;       // [T][K]
  // shared expert (Is = 0: none)
  int swfmt;
  const void* xs;  // shared-expert input: bf16 or fp32 dequantised
  bool xs_f32;
  const void *sg, *su, *sgs, *sus, *sd, *sds;
  int Is;
  float* hs;   // fp32 [T][Is]
  float* ysh;  // fp32 [T][H]
};
hipError_t launch_decode_stage1(const DecodeParams& p, hipStream_t s);
hipError_t launch_decode_stage2(const DecodeParams& p, hipStream_t s);

// Small-T layer (T <= kRouteGemvMaxT) with bf16 activations and one weight
// format for routed and shared experts, in one persistent launch (decode.hip): router, top-k, shared
// and routed gate/up, down + combine, ordered by work queues and completion
// counters in `ctr` (kFusedCtrBytes, zero before the first launch; every
// launch leaves its queues and counters zero again; the sticky error word,
// the epoch word and the tagged router logits are kept).  d.xs must be
// d.x (bf16); d.swfmt must equal wfmt; d.ysh is unused.
struct FusedDecodeParams {
  DecodeParams d;
  int wfmt, I;
  const void *g, *u, *gs, *us, *dn, *dns;  // routed experts
  float* h;        // fp32 [T*K][I]
  uint16_t* out;   // bf16 [T][H]
  unsigned* ctr;   // counter block
};
constexpr int kFusedCtrBytes = 49152;
constexpr int kFusedErrorWord = 0;  // ctr[0] != 0: a bounded wait gave up (never expected)
constexpr int kFusedEpochWord = 1;  // ctr[1]: launches so far modulo 0xffffffff, never reset
constexpr int kFusedTagOff = 24576;  // bytes: tagged router logits, 64-bit [T][E]
// bytes: the batched router's per-block counters (K split), after the tagged
// logits; zero between calls (the last workgroup of a block resets its word)
constexpr int kRouteCtrOff = 40960;
constexpr int kRouteCtrMax = (kFusedCtrBytes - kRouteCtrOff) / 4;
constexpr int kFusedXLdsMax = 65536;  // bytes of x (T * H bf16) the launch stages in LDS; above, x is read from L2
hipError_t launch_fused_decode(const FusedDecodeParams& p, hipStream_t s);

// ------------------------------------------------------------------ combine
// out[t] = bf16(sum_j w[t][j] * y_perm[inv_pos[t*K+j]] + y_shared[t]).
hipError_t launch_combine(const void* y_perm, bool y_bf16, const int* inv_pos, const float* w,
                          const void* y_shared, bool ys_bf16, int T, int K, int H, uint16_t* out,
                          hipStream_t s);

// ------------------------------------------------------------------ backward (backward.hip)
// C (+)= sum_k A(m, k) B(k, n), bf16 operands, fp32 accumulate, 64 x 64 tiles.
//   NN (tn false): rows m of the groups' segments (tile list of 64-row tiles,
//     or rows 0..rows-1 of one group), A[m][k] row-major (row gathered through
//     a_map[seg0 + m] / a_div when set), B of group e at B + e * b_stride
//     stored [k][n]; npass = 2 adds A1 (K1 columns) times B1.  C rows are the
//     A rows: C[(seg0 + m) * ldc + n].
//   TN (tn true): per group e, C_e[m][n] = sum over the group's segment rows
//     k of P[k][m] Q[k][n]; P = A0 (row k at a_map[k] / a_div when set), Q = B0
//     (row k at b_map[k] / b_div when set); C_e at C + e * c_stride.  Without
//     seg, one group over rows 0..rows-1.
struct BwdGemmParams {
  const uint16_t* A0;
  const uint16_t* A1;
  long lda;
  const int* a_map;
  int a_div;
  const uint16_t* B0;
  const uint16_t* B1;
  long ldb, b_stride;
  const int* b_map;
  int b_div;
  int npass;
  int M, N, K, K1;
  int rows;
  const int* seg;
  const int* tiles;
  const int* ntiles;
  int max_tiles;
  void* C;
  long ldc, c_stride;
};
hipError_t launch_bwd_gemm(bool tn, bool out_bf16, const BwdGemmParams& p, int n_groups, hipStream_t s);
hipError_t launch_swiglu_fwd(const float* g, const float* u, long n, uint16_t* h, hipStream_t s);
hipError_t launch_swiglu_bwd(const float* g, const float* u, const float* dh, long n, uint16_t* dg, uint16_t* du,
                             hipStream_t s);
hipError_t launch_combine_bwd(const uint16_t* dy, const float* Y, const int* inv_pos, const float* w, int T, int K,
                              int H, float* dw, uint16_t* dY, hipStream_t s);
hipError_t launch_router_bwd(const float* logits, const float* bias, const int* ids, const float* dw, int T, int E,
                             int K, float scale, float* dl, uint16_t* dl_bf, hipStream_t s);
hipError_t launch_dx_sum(const float* dXr, const int* inv_pos, int K, const float* dXs, const float* dXw, int T, int H,
                         uint16_t* dx, hipStream_t s);
hipError_t launch_colsum(const float* dl, int T, int E, float* out, hipStream_t s);

// ------------------------------------------------------------------ diagnostics
hipError_t launch_e4m3_decode(const uint8_t* codes, float* out, int n, hipStream_t s);
hipError_t launch_e4m3_encode(const float* in, uint8_t* codes, int n, hipStream_t s);

}  // namespace moe
