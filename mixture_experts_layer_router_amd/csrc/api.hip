// C ABI of the MoE layer library: host-side validation, workspace planning,
// path selection and kernel orchestration.  Declarations and the contract of
// every entry point are in include/moe.h.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/moe.h"
#include "common.h"
#include "kernels.h"

using namespace moe;

namespace {

constexpr int kGemvMaxT = 4;       // moe_forward: T <= this runs the GEMV path
constexpr int kGemvMaxRows = 16;   // moe_expert_ffn: rows <= this runs the GEMV path
constexpr size_t kAlign = 256;

size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// test hook: MOE_FORCE_PATH=gemv|gemm|staged (staged: the GEMV path with the
// small-T layer in separate launches instead of the single-launch kernel)
int forced_path() {
  const char* s = getenv("MOE_FORCE_PATH");
  if (!s) return 0;
  if (!strcmp(s, "gemv")) return 1;
  if (!strcmp(s, "gemm")) return 2;
  if (!strcmp(s, "staged")) return 3;
  return 0;
}

bool gemm_pair(int wf, int af) {
  return (wf == W_BF16 && af == A_NONE) || (wf == W_FP8_B128 && af == A_FP8_1X128) ||
         (wf == W_MXFP8 && af == A_MXFP8_1X32);
}
bool any_pair(int wf, int af) {
  return gemm_pair(wf, af) || (wf == W_FP8_B128 && af == A_NONE) || (wf == W_MXFP8 && af == A_NONE);
}

moe_status check_cfg(const moe_config* c) {
  if (!c) return MOE_EINVAL;
  if (c->hidden <= 0 || c->inter <= 0 || c->shared_inter < 0 || c->n_experts <= 0 || c->n_groups <= 0)
    return MOE_EINVAL;
  if (c->n_experts % c->n_groups != 0) return MOE_EINVAL;
  if (c->topk_groups < 1 || c->topk_groups > c->n_groups) return MOE_EINVAL;
  const int cand = c->topk_groups * (c->n_experts / c->n_groups);
  if (c->topk < 1 || c->topk > cand || c->topk > 16) return MOE_EINVAL;
  if (!isfinite(c->route_scale)) return MOE_EINVAL;
  for (int f : {c->routed_wfmt, c->shared_wfmt})
    if (f < 0 || f > 2) return MOE_EINVAL;
  for (int f : {c->routed_afmt, c->shared_afmt})
    if (f < 0 || f > 2) return MOE_EINVAL;
  if (c->n_experts > 256 || c->n_groups > 64) return MOE_EUNSUPPORTED;
  if (c->hidden % 128 || c->inter % 128 || c->shared_inter % 128) return MOE_EALIGN;
  if (!any_pair(c->routed_wfmt, c->routed_afmt)) return MOE_EUNSUPPORTED;
  // the FP8_B128 GEMM stages all K steps' weight scales in LDS
  for (int f : {c->routed_wfmt, c->shared_wfmt})
    if (f == W_FP8_B128 && (c->hidden > kGemmMaxK || c->inter > kGemmMaxK || c->shared_inter > kGemmMaxK))
      return MOE_EUNSUPPORTED;
  if (c->shared_inter > 0 && !any_pair(c->shared_wfmt, c->shared_afmt)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

moe_status check_weights(const moe_ffn_weights* w, int wfmt) {
  if (!w || !w->gate || !w->up || !w->down) return MOE_EINVAL;
  if (wfmt != W_BF16 && (!w->gate_s || !w->up_s || !w->down_s)) return MOE_EINVAL;
  for (const void* p : {w->gate, w->up, w->down})
    if (!aligned16(p)) return MOE_EALIGN;
  if (wfmt != W_BF16)
    for (const void* p : {w->gate_s, w->up_s, w->down_s})
      if (!aligned16(p)) return MOE_EALIGN;
  return MOE_OK;
}

size_t act_scale_bytes(int afmt, size_t rows, int cols) {
  if (afmt == A_FP8_1X128) return rows * (cols / 128) * 4;
  if (afmt == A_MXFP8_1X32) return rows * (cols / 32);
  return 0;
}
// bytes of an activation matrix [rows][cols] in the GEMM path
size_t act_bytes(int afmt, size_t rows, int cols) {
  return afmt == A_NONE ? rows * cols * 2 : rows * cols;
}
size_t wscale_stride(int wfmt, int N, int K) {  // scale elements per expert
  if (wfmt == W_FP8_B128) return size_t(N / 128) * (K / 128);
  if (wfmt == W_MXFP8) return size_t(N) * (K / 32);
  return 0;
}

struct Ws {
  size_t counter, logits, ids, w, offsets, perm, inv, hist, tiles, ntiles;
  size_t xq, xqs, xs2, xs2s;  // routed-format x, shared-format x
  size_t xn, rhist;           // normalised x (bf16), per-block expert counts of the fused router
  size_t h, hs, hsh, hshs;    // routed h (+scales), shared h (+scales)
  size_t yperm, ysh;
  size_t total;
};

Ws plan(const moe_config* c, int Tm) {
  const size_t T = size_t(std::max(Tm, 1)), K = c->topk, E = c->n_experts, H = c->hidden, I = c->inter,
               Is = c->shared_inter;
  const size_t TK = T * K;
  Ws s{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o += up(std::max<size_t>(bytes, 16));
    return at;
  };
  s.counter = take(kFusedCtrBytes);  // must stay at offset 0 (documented in moe.h)
  s.logits = take(T * E * 4 * (T > size_t(kRouteGemvMaxT) ? kRouterMaxSplit : 1));  // split-K slices
  s.ids = take(TK * 4);
  s.w = take(TK * 4);
  s.offsets = take((E + 1) * 4);
  s.perm = take(TK * 4);
  s.inv = take(TK * 4);
  s.hist = take(permute_hist_ints(int(TK), int(E)) * 4);
  s.tiles = take(size_t(2) * max_tiles(int(TK), int(E), kGemmBM) * 4);
  s.ntiles = take(16);
  // x in the routed activation format: quantised rows (up to TK rows for
  // moe_expert_ffn) or fp32 dequantised rows for the GEMV path
  s.xq = take(TK * H * 4);
  s.xqs = take(std::max(act_scale_bytes(A_FP8_1X128, TK, int(H)), act_scale_bytes(A_MXFP8_1X32, TK, int(H))));
  s.xs2 = take(T * H * 4);
  s.xs2s = take(std::max(act_scale_bytes(A_FP8_1X128, T, int(H)), act_scale_bytes(A_MXFP8_1X32, T, int(H))));
  s.h = take(TK * I * 4);
  s.hs = take(std::max(act_scale_bytes(A_FP8_1X128, TK, int(I)), act_scale_bytes(A_MXFP8_1X32, TK, int(I))));
  if (Is) {
    s.hsh = take(T * Is * 4);
    s.hshs = take(std::max(act_scale_bytes(A_FP8_1X128, T, int(Is)), act_scale_bytes(A_MXFP8_1X32, T, int(Is))));
    s.ysh = take(T * H * 4);
  }
  s.yperm = take(TK * H * 2);
  s.xn = take(T * H * 2);
  s.rhist = take(((T + kRouteBlock - 1) / kRouteBlock) * E * 4);
  s.total = o;
  return s;
}

template <class P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<uint8_t*>(ws) + off);
}

RouteParams route_params(const moe_config* c) {
  return RouteParams{c->hidden, c->n_experts, c->n_groups, c->topk_groups, c->topk, c->route_scale};
}

#define HIP_TRY(expr)                             \
  do {                                            \
    if ((expr) != hipSuccess) return MOE_EHIP;    \
  } while (0)

// Optional launch trace for measurement: when armed, every kernel launch of
// the entry points is bracketed by two caller-owned events recorded on the
// launch stream.  Not thread-safe; meant for one benchmarking thread.
struct Trace {
  hipEvent_t* ev = nullptr;
  int max = 0;
  int n = 0;
  const char* names[128] = {};
} g_trace;

// Second stream of the batched path, per device, for a shared expert too
// small to fill the chip: its FFN needs only x, so it runs beside the routing,
// dispatch and routed experts and joins back before the combine.  Created on
// first use (default priority, non-blocking); the mutex keeps each call's
// fork and join enqueues together when several host threads call in.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
SideStream g_side[64];

// the side stream of the device that `caller` runs on, or null if it cannot be had
SideStream* side_stream(hipStream_t caller) {
  int dev = 0, cur = 0;
  if (hipStreamGetDevice(caller, &dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  SideStream& ss = g_side[dev];
  if (!ss.s) {
    if (hipGetDevice(&cur) != hipSuccess || hipSetDevice(dev) != hipSuccess) return nullptr;
    hipStream_t s = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    bool ok = hipStreamCreateWithFlags(&s, hipStreamNonBlocking) == hipSuccess;
    ok = ok && hipEventCreateWithFlags(&f, hipEventDisableTiming) == hipSuccess;
    ok = ok && hipEventCreateWithFlags(&j, hipEventDisableTiming) == hipSuccess;
    if (ok) {
      ss.fork = f;
      ss.join = j;
      ss.s = s;
    } else {
      if (j) (void)hipEventDestroy(j);
      if (f) (void)hipEventDestroy(f);
      if (s) (void)hipStreamDestroy(s);
    }
    (void)hipSetDevice(cur);
    if (!ok) return nullptr;
  }
  return &ss;
}

// Joins the side stream back into the caller's stream when it goes out of
// scope, so a call that returns early after the fork (a failed launch) still
// leaves the caller's stream ordered after the side stream's work on x and
// the workspace.  join() does it early, before the combine.
struct SideJoin {
  SideStream* side = nullptr;
  hipStream_t caller = nullptr;
  hipError_t join() {
    if (!side) return hipSuccess;
    SideStream* s = side;
    side = nullptr;
    const hipError_t e = hipEventRecord(s->join, s->s);
    const hipError_t f = hipStreamWaitEvent(caller, s->join, 0);
    return e != hipSuccess ? e : f;
  }
  ~SideJoin() { (void)join(); }
};

template <class F>
hipError_t traced(const char* name, hipStream_t s, F&& f) {
  if (!g_trace.ev || 2 * g_trace.n + 1 >= g_trace.max || g_trace.n >= 128) return f();
  if (hipEventRecord(g_trace.ev[2 * g_trace.n], s) != hipSuccess) return hipErrorUnknown;
  const hipError_t e = f();
  if (hipEventRecord(g_trace.ev[2 * g_trace.n + 1], s) != hipSuccess) return hipErrorUnknown;
  g_trace.names[g_trace.n++] = name;
  return e;
}
#define LAUNCH(name, expr) HIP_TRY(traced(name, s_, [&] { return (expr); }))

// stage M: the norm weight (null: no norm), its eps, and where the caller
// wants the normalised x (null: nowhere)
struct NormArgs {
  const uint16_t* gamma = nullptr;
  float eps = 0.f;
  uint16_t* x_out = nullptr;
};

moe_status do_route(const moe_config* c, const uint16_t* x, int T, const uint16_t* wr, const float* bias, int* ids,
                    float* w, void* ws, const Ws& L, hipStream_t s) {
  const RouteParams rp = route_params(c);
  hipStream_t s_ = s;
  if (T <= kRouteGemvMaxT) {
    LAUNCH("route_logits", launch_route_logits(x, T, wr, rp, at<float>(ws, L.logits), s));
    LAUNCH("topk", launch_topk(at<float>(ws, L.logits), T, bias, rp, ids, w, s));
    return MOE_OK;
  }
  RouteFusedParams rf{};
  rf.h = x;
  rf.T = T;
  rf.H = c->hidden;
  rf.wr = wr;
  rf.bias = bias;
  rf.rp = rp;
  rf.ids = ids;
  rf.w = w;
  rf.slices = 1;
  LAUNCH("route_fused", launch_route_fused(rf, s));
  return MOE_OK;
}

// H slices of the batched router per block of kRouteBlock tokens: about one
// workgroup per CU in all, at most 8, and at least 4 column blocks of 128 per
// slice (half the workgroup's waves busy); 1 beyond the counters' capacity.
// The partial logits fit the logits region: blocks x slices <= T for T > 8.
int route_slices(int T, int H) {
  const int blocks = (T + kRouteBlock - 1) / kRouteBlock;
  if (blocks > kRouteCtrMax) return 1;
  const int want = (256 + blocks - 1) / blocks;
  return std::max(1, std::min({want, 8, (H / 128) / 4}));
}

// The batched routing stack: stage M (if any), router, top-k, the routed
// input in its activation format and the per-block counts in one launch
// (route_fused.hip), then the stable scatter (offsets, perm_src, inv_pos and,
// with `tiles`, the grouped-GEMM tile list of bm-row tiles).
moe_status route_dispatch(const moe_config* c, const uint16_t* h, int T, const NormArgs& nm, const uint16_t* wr,
                          const float* bias, int* ids, float* w, int* off, int* perm, int* inv, uint16_t* x_out,
                          void* xq, void* xqs, int* tiles, int* ntiles, int bm, void* ws, const Ws& L, hipStream_t s) {
  hipStream_t s_ = s;
  RouteFusedParams rf{};
  rf.h = h;
  rf.gamma = nm.gamma;
  rf.eps = nm.eps;
  rf.T = T;
  rf.H = c->hidden;
  rf.wr = wr;
  rf.bias = bias;
  rf.rp = route_params(c);
  rf.ids = ids;
  rf.w = w;
  rf.x_out = x_out;
  rf.afmt = c->routed_afmt;
  rf.xq = c->routed_afmt != A_NONE ? xq : nullptr;
  rf.xqs = xqs;
  rf.hist = at<int>(ws, L.rhist);
  rf.slices = route_slices(T, c->hidden);
  rf.part = at<float>(ws, L.logits);
  rf.ctr = at<unsigned>(ws, L.counter + kRouteCtrOff);
  LAUNCH("route_fused", launch_route_fused(rf, s));
  LAUNCH("permute", launch_permute_scatter(ids, T * c->topk, c->n_experts, rf.hist, kRouteBlock * c->topk, off, perm,
                                           inv, tiles, ntiles, bm, s));
  return MOE_OK;
}

// GEMM-path FFN on rows already laid out per segment (or all rows for the
// shared expert).  A: activation rows in `afmt` (bf16 when A_NONE); a_map
// gathers rows.  Output: y (fp32 or bf16) [rows][H].
// The two GEMMs of an expert FFN: gate/up (with SiLU * up and h in the
// activation format) into h, and down from h into y.
void ffn_gemm_params(const moe_config* c, bool routed, const void* A, const void* As, const int* a_map, int a_div,
                     int rows, const int* seg, const int* tiles, const int* ntiles, int maxt, int bm,
                     const moe_ffn_weights* W, void* h, void* hs, void* y, GemmParams* gp, GemmParams* dp) {
  const int wf = routed ? c->routed_wfmt : c->shared_wfmt;
  const int af = routed ? c->routed_afmt : c->shared_afmt;
  const int I = routed ? c->inter : c->shared_inter;
  const int H = c->hidden;
  GemmParams g{};
  g.A = A;
  g.lda = H;
  g.As = As;
  g.a_map = a_map;
  g.a_div = a_div;
  g.B0 = W->gate;
  g.B1 = W->up;
  g.b_stride = long(I) * H;
  g.B0s = W->gate_s;
  g.B1s = W->up_s;
  g.bs_stride = long(wscale_stride(wf, I, H));
  g.N = I;
  g.K = H;
  g.seg = seg;
  g.M = rows;
  g.tiles = tiles;
  g.ntiles = ntiles;
  g.max_tiles = maxt;
  g.bm = bm;
  g.C = h;
  g.ldc = I;
  g.Cs = hs;
  g.out_afmt = af;
  GemmParams d{};
  d.A = h;
  d.lda = I;
  d.As = hs;
  d.B0 = W->down;
  d.b_stride = long(H) * I;
  d.B0s = W->down_s;
  d.bs_stride = long(wscale_stride(wf, H, I));
  d.N = H;
  d.K = I;
  d.seg = seg;
  d.M = rows;
  d.tiles = tiles;
  d.ntiles = ntiles;
  d.max_tiles = maxt;
  d.bm = bm;
  d.C = y;
  d.ldc = H;
  *gp = g;
  *dp = d;
}

moe_status gemm_ffn(const moe_config* c, bool routed, const void* A, const void* As, const int* a_map, int a_div,
                    int rows, const int* seg, const int* tiles, const int* ntiles, int maxt, int bm,
                    const moe_ffn_weights* W, void* h, void* hs, void* y, bool y_bf16, hipStream_t s) {
  const int wf = routed ? c->routed_wfmt : c->shared_wfmt;
  hipStream_t s_ = s;
  GemmParams g, d;
  ffn_gemm_params(c, routed, A, As, a_map, a_div, rows, seg, tiles, ntiles, maxt, bm, W, h, hs, y, &g, &d);
  LAUNCH(routed ? "gemm_gate_up_routed" : "gemm_gate_up_shared", launch_gemm(wf, EPI_GATEUP, g, s));
  LAUNCH(routed ? "gemm_down_routed" : "gemm_down_shared", launch_gemm(wf, y_bf16 ? EPI_BF16 : EPI_F32, d, s));
  return MOE_OK;
}

// The batched shared FFN on all T rows of x, on stream s, using only its own
// workspace regions (x quantised into xs2 in the shared activation format,
// h in hsh, y in ysh); *ysh gets the output rows, bf16 like Y_perm.
moe_status shared_ffn(const moe_config* cfg, const uint16_t* x, int T, const moe_ffn_weights* shared, void* ws,
                      const Ws& L, float** ysh, hipStream_t s) {
  hipStream_t s_ = s;
  const int H = cfg->hidden, saf = cfg->shared_afmt;
  const void* xs = x;
  const void* xss = nullptr;
  if (saf != A_NONE) {
    LAUNCH("quant_rows_shared", launch_quant_rows(x, false, T, H, nullptr, 1, saf, at<void>(ws, L.xs2),
                                                  at<void>(ws, L.xs2s), nullptr, s));
    xs = at<void>(ws, L.xs2);
    xss = at<void>(ws, L.xs2s);
  }
  *ysh = at<float>(ws, L.ysh);
  return gemm_ffn(cfg, false, xs, xss, nullptr, 1, T, nullptr, nullptr, nullptr, 0,
                  ffn_tile_rows(cfg->shared_wfmt, H, cfg->shared_inter), shared, at<void>(ws, L.hsh),
                  at<void>(ws, L.hshs), *ysh, true, s);
}

// moe_forward on a given workspace.  side_ok: a shared expert too small to
// fill the chip may run on the side stream (created on first use); false
// keeps every launch on the caller's stream.
// nm: stage M before the router (nm.gamma null: x is the layer input as given).
moe_status forward_impl(const moe_config* cfg, const uint16_t* x, int32_t T, const uint16_t* w_router,
                        const float* bias, const moe_ffn_weights* routed, const moe_ffn_weights* shared, uint16_t* out,
                        int32_t* topk_ids_out, float* topk_w_out, void* ws, size_t ws_bytes, hipStream_t stream,
                        bool side_ok, const NormArgs& nm = NormArgs{}) {
  hipStream_t s_ = stream;
  moe_status st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !routed || !out || !ws) return MOE_EINVAL;
  const bool has_shared = cfg->shared_inter > 0;
  if (has_shared && !shared) return MOE_EINVAL;
  if ((st = check_weights(routed, cfg->routed_wfmt)) != MOE_OK) return st;
  if (has_shared && (st = check_weights(shared, cfg->shared_wfmt)) != MOE_OK) return st;
  for (const void* p : {(const void*)x, (const void*)w_router, (const void*)out, (const void*)ws})
    if (!aligned16(p)) return MOE_EALIGN;
  if (nm.gamma && (!aligned16(nm.gamma) || (nm.x_out && !aligned16(nm.x_out)) || !(nm.eps >= 0.f)))
    return nm.eps >= 0.f ? MOE_EALIGN : MOE_EINVAL;
  const Ws L = plan(cfg, T);
  if (ws_bytes < L.total) return MOE_EWORKSPACE;

  const int H = cfg->hidden, K = cfg->topk, E = cfg->n_experts, TK = T * K;
  const bool norm = nm.gamma != nullptr;
  uint16_t* xn = norm ? (nm.x_out ? nm.x_out : at<uint16_t>(ws, L.xn)) : nullptr;  // normalised x
  const int raf = cfg->routed_afmt, saf = cfg->shared_afmt;
  int* ids = topk_ids_out ? topk_ids_out : at<int>(ws, L.ids);
  float* w = topk_w_out ? topk_w_out : at<float>(ws, L.w);
  const int fp = forced_path();
  const bool pairs_ok = gemm_pair(cfg->routed_wfmt, raf) && (!has_shared || gemm_pair(cfg->shared_wfmt, saf));
  if (fp == 2 && !pairs_ok) return MOE_EUNSUPPORTED;
  const bool gemv = fp == 1 || fp == 3 || (fp != 2 && T <= kGemvMaxT) || !pairs_ok;

  // T <= 8 with bf16 activations and one weight format: the single launch
  // (unless a test forces the GEMM or the staged launches)
  const bool single = fp != 2 && fp != 3 && T <= kRouteGemvMaxT && raf == A_NONE && H % 8 == 0 &&
                      (!has_shared || (saf == A_NONE && cfg->shared_wfmt == cfg->routed_wfmt));
  if (single) {
    // x staged in LDS (with the norm applied there) up to kFusedXLdsMax bytes;
    // above, the launch reads x from L2, normalised first by its own launch
    NormArgs snm = nm;
    if (norm && size_t(T) * H * 2 > size_t(kFusedXLdsMax)) {
      LAUNCH("rmsnorm", launch_rmsnorm_rows(x, nm.gamma, nm.eps, T, H, xn, stream));
      x = xn;
      snm = NormArgs{};
    }
    // small T, bf16 activations: the whole layer in one persistent launch
    FusedDecodeParams fp_{};
    DecodeParams& dp = fp_.d;
    dp.x = x;
    dp.T = T;
    dp.H = H;
    dp.wr = w_router;
    dp.bias = bias;
    dp.rp = route_params(cfg);
    dp.logits = at<float>(ws, L.logits);
    dp.ids = ids;
    dp.w = w;
    dp.swfmt = has_shared ? cfg->shared_wfmt : W_BF16;
    if (has_shared) {
      dp.xs = x;
      dp.sg = shared->gate; dp.su = shared->up; dp.sgs = shared->gate_s; dp.sus = shared->up_s;
      dp.sd = shared->down; dp.sds = shared->down_s;
      dp.Is = cfg->shared_inter;
      dp.hs = at<float>(ws, L.hsh);
    }
    fp_.wfmt = cfg->routed_wfmt;
    fp_.I = cfg->inter;
    fp_.g = routed->gate; fp_.u = routed->up; fp_.gs = routed->gate_s; fp_.us = routed->up_s;
    fp_.dn = routed->down; fp_.dns = routed->down_s;
    fp_.h = at<float>(ws, L.h);
    fp_.out = out;
    fp_.ctr = at<unsigned>(ws, L.counter);
    dp.gamma = snm.gamma;
    dp.eps = snm.eps;
    dp.x_out = snm.x_out;
    LAUNCH("decode_fused", launch_fused_decode(fp_, stream));
    return MOE_OK;
  }

  if (norm && gemv) {  // the launches below read x: normalise it first
    LAUNCH("rmsnorm", launch_rmsnorm_rows(x, nm.gamma, nm.eps, T, H, xn, stream));
    x = xn;
  }

  if (gemv && T <= kRouteGemvMaxT) {
    // small T: router || shared gate/up, then top-k || shared down, then the
    // routed experts; the kernel boundaries are the only synchronisation
    const void* xs = x;
    bool xs32 = false;
    if (has_shared && saf != A_NONE) {
      LAUNCH("quant_rows", launch_quant_rows(x, false, T, H, nullptr, 1, saf, nullptr, nullptr, at<float>(ws, L.xs2), stream));
      xs = at<float>(ws, L.xs2);
      xs32 = true;
    }
    DecodeParams dp{};
    dp.x = x;
    dp.T = T;
    dp.H = H;
    dp.wr = w_router;
    dp.bias = bias;
    dp.rp = route_params(cfg);
    dp.logits = at<float>(ws, L.logits);
    dp.ids = ids;
    dp.w = w;
    dp.swfmt = has_shared ? cfg->shared_wfmt : W_BF16;
    if (has_shared) {
      dp.xs = xs;
      dp.xs_f32 = xs32;
      dp.sg = shared->gate; dp.su = shared->up; dp.sgs = shared->gate_s; dp.sus = shared->up_s;
      dp.sd = shared->down; dp.sds = shared->down_s;
      dp.Is = cfg->shared_inter;
      dp.hs = at<float>(ws, L.hsh);
      dp.ysh = at<float>(ws, L.ysh);
    }
    LAUNCH("decode_router_shared_up", launch_decode_stage1(dp, stream));
    if (has_shared && saf != A_NONE)
      LAUNCH("quant_rows", launch_quant_rows(dp.hs, true, T, cfg->shared_inter, nullptr, 1, saf, nullptr, nullptr, dp.hs, stream));
    LAUNCH("decode_topk_shared_down", launch_decode_stage2(dp, stream));
    const void* xr = x;
    bool xr32 = false;
    if (raf != A_NONE) {
      if (saf == raf && has_shared) {
        xr = xs;
      } else {
        LAUNCH("quant_rows", launch_quant_rows(x, false, T, H, nullptr, 1, raf, nullptr, nullptr, at<float>(ws, L.xq), stream));
        xr = at<float>(ws, L.xq);
      }
      xr32 = true;
    }
    float* h = at<float>(ws, L.h);
    GemvUpParams u{};
    u.wfmt = cfg->routed_wfmt;
    u.swfmt = cfg->routed_wfmt;
    u.x = xr;
    u.x_f32 = xr32;
    u.T = T;
    u.H = H;
    u.ids = ids;
    u.K = K;
    u.g = routed->gate; u.u = routed->up; u.gs = routed->gate_s; u.us = routed->up_s;
    u.I = cfg->inter;
    u.h = h;
    u.E = E;
    LAUNCH("gemv_gate_up", launch_gemv_gate_up(u, stream));
    if (raf != A_NONE) LAUNCH("quant_rows", launch_quant_rows(h, true, TK, cfg->inter, nullptr, 1, raf, nullptr, nullptr, h, stream));
    GemvDownParams d{};
    d.wfmt = cfg->routed_wfmt;
    d.swfmt = cfg->routed_wfmt;
    d.T = T;
    d.H = H;
    d.K = K;
    d.I = cfg->inter;
    d.ids = ids;
    d.w = w;
    d.h = h;
    d.d = routed->down; d.ds = routed->down_s;
    d.out = out;
    d.E = E;
    d.ys_add = has_shared ? dp.ysh : nullptr;
    LAUNCH("gemv_down_combine", launch_gemv_down(d, stream));
    return MOE_OK;
  }

  // batched path, shared expert whose gate/up grid fills at most half the
  // CUs (128-row tiles, 128 output columns each): it forks onto the side
  // stream before the routing.  A larger one stays in order on the caller's
  // stream: beside the routed GEMMs it measured slower (their tiles take the
  // same CUs).
  std::unique_lock<std::mutex> side_lock(g_side_mu, std::defer_lock);
  SideStream* side = nullptr;
  SideJoin joiner;  // declared after the lock: it joins before the lock is released
  float* ysh = nullptr;
  // the shared FFN forks onto the side stream as soon as its input exists:
  // at once without a norm, after the fused router (which writes xn) with one
  const bool fork = !gemv && has_shared && side_ok &&
                    long((T + kGemmBM - 1) / kGemmBM) * ((cfg->shared_inter + 127) / 128) < 128;
  auto fork_shared = [&](const uint16_t* xs_in) -> moe_status {
    side_lock.lock();
    side = side_stream(stream);
    if (side) {
      HIP_TRY(hipEventRecord(side->fork, stream));
      HIP_TRY(hipStreamWaitEvent(side->s, side->fork, 0));
      joiner.side = side;
      joiner.caller = stream;
      return shared_ffn(cfg, xs_in, T, shared, ws, L, &ysh, side->s);
    }
    return MOE_OK;
  };
  if (fork && !norm && (st = fork_shared(x)) != MOE_OK) return st;

  if (gemv) {
    if ((st = do_route(cfg, x, T, w_router, bias, ids, w, ws, L, stream)) != MOE_OK) return st;
  }

  if (gemv) {  // T > kRouteGemvMaxT on the GEMV path: routed + shared gate/up in one launch
    const void* xr = x;
    bool xr32 = false;
    if (raf != A_NONE) {
      LAUNCH("quant_rows", launch_quant_rows(x, false, T, H, nullptr, 1, raf, nullptr, nullptr, at<float>(ws, L.xq), stream));
      xr = at<float>(ws, L.xq);
      xr32 = true;
    }
    const void* xs = x;
    bool xs32 = false;
    if (has_shared && saf != A_NONE) {
      if (saf == raf) {
        xs = xr;
      } else {
        LAUNCH("quant_rows", launch_quant_rows(x, false, T, H, nullptr, 1, saf, nullptr, nullptr, at<float>(ws, L.xs2), stream));
        xs = at<float>(ws, L.xs2);
      }
      xs32 = true;
    }
    float* h = at<float>(ws, L.h);
    float* hs = has_shared ? at<float>(ws, L.hsh) : nullptr;
    GemvUpParams u{};
    u.wfmt = cfg->routed_wfmt;
    u.swfmt = has_shared ? cfg->shared_wfmt : cfg->routed_wfmt;
    u.x = xr;
    u.x_f32 = xr32;
    u.T = T;
    u.H = H;
    u.ids = ids;
    u.K = K;
    u.g = routed->gate; u.u = routed->up; u.gs = routed->gate_s; u.us = routed->up_s;
    u.I = cfg->inter;
    u.h = h;
    if (has_shared) {
      u.sg = shared->gate; u.su = shared->up; u.sgs = shared->gate_s; u.sus = shared->up_s;
      u.Is = cfg->shared_inter;
      u.hs = hs;
      u.xs = xs;
      u.xs_f32 = xs32;
    }
    u.E = E;
    LAUNCH("gemv_gate_up", launch_gemv_gate_up(u, stream));
    if (raf != A_NONE) LAUNCH("quant_rows", launch_quant_rows(h, true, TK, cfg->inter, nullptr, 1, raf, nullptr, nullptr, h, stream));
    if (has_shared && saf != A_NONE)
      LAUNCH("quant_rows", launch_quant_rows(hs, true, T, cfg->shared_inter, nullptr, 1, saf, nullptr, nullptr, hs, stream));
    GemvDownParams d{};
    d.wfmt = cfg->routed_wfmt;
    d.swfmt = u.swfmt;
    d.T = T;
    d.H = H;
    d.K = K;
    d.I = cfg->inter;
    d.Is = cfg->shared_inter;
    d.ids = ids;
    d.w = w;
    d.h = h;
    d.hs = hs;
    d.d = routed->down; d.ds = routed->down_s;
    if (has_shared) { d.sd = shared->down; d.sds = shared->down_s; }
    d.out = out;
    d.E = E;
    LAUNCH("gemv_down_combine", launch_gemv_down(d, stream));
    return MOE_OK;
  }

  // batched path: routing stack (fused router + scatter), routed GEMMs,
  // shared GEMMs (side stream or in order), combine
  int* off = at<int>(ws, L.offsets);
  int* perm = at<int>(ws, L.perm);
  int* inv = at<int>(ws, L.inv);
  int* tiles = at<int>(ws, L.tiles);
  int* ntiles = at<int>(ws, L.ntiles);
  const int rbm = ffn_tile_rows(cfg->routed_wfmt, H, cfg->inter);
  if ((st = route_dispatch(cfg, x, T, nm, w_router, bias, ids, w, off, perm, inv, xn, at<void>(ws, L.xq),
                           at<void>(ws, L.xqs), tiles, ntiles, rbm, ws, L, stream)) != MOE_OK)
    return st;
  const uint16_t* xin = norm ? xn : x;  // the layer input x
  if (fork && norm && (st = fork_shared(xin)) != MOE_OK) return st;
  const void* xa = xin;
  const void* xas = nullptr;
  if (raf != A_NONE) {
    xa = at<void>(ws, L.xq);
    xas = at<void>(ws, L.xqs);
  }
  // shared expert in order on the caller's stream: its input
  const void* xs = xin;
  const void* xss = nullptr;
  if (has_shared && !side && saf != A_NONE) {
    if (saf == raf) {
      xs = xa;
      xss = xas;
    } else {
      LAUNCH("quant_rows", launch_quant_rows(xin, false, T, H, nullptr, 1, saf, at<void>(ws, L.xs2), at<void>(ws, L.xs2s),
                                nullptr, stream));
      xs = at<void>(ws, L.xs2);
      xss = at<void>(ws, L.xs2s);
    }
  }
  GemmParams rg, rd, sgp, sdp;
  ffn_gemm_params(cfg, true, xa, xas, perm, K, TK, off, tiles, ntiles, max_tiles(TK, E, rbm), rbm, routed,
                  at<void>(ws, L.h), at<void>(ws, L.hs), at<void>(ws, L.yperm), &rg, &rd);
  if (has_shared && !side) {
    ysh = at<float>(ws, L.ysh);
    ffn_gemm_params(cfg, false, xs, xss, nullptr, 1, T, nullptr, nullptr, nullptr, 0,
                    ffn_tile_rows(cfg->shared_wfmt, H, cfg->shared_inter), shared, at<void>(ws, L.hsh),
                    at<void>(ws, L.hshs), ysh, &sgp, &sdp);
  }
  // Both down GEMMs on the large-tile kernel (the 2,048-token MXFP8 layer:
  // 3.5 waves of routed tiles, 0.875 of shared ones): one launch, the
  // shared tiles first, so each GEMM's partial last wave is filled with the
  // other's tiles.
  const int swf = cfg->shared_wfmt, rwf = cfg->routed_wfmt;
  const bool dual = has_shared && !side && gemm2_chosen(rwf, EPI_BF16, rd) && gemm2_chosen(swf, EPI_BF16, sdp);
  LAUNCH("gemm_gate_up_routed", launch_gemm(rwf, EPI_GATEUP, rg, stream));
  if (dual) {
    LAUNCH("gemm_gate_up_shared", launch_gemm(swf, EPI_GATEUP, sgp, stream));
    LAUNCH("gemm_down_shared_routed", launch_gemm2_dual(swf, sdp, rwf, rd, stream));
  } else {
    LAUNCH("gemm_down_routed", launch_gemm(rwf, EPI_BF16, rd, stream));
    if (has_shared && !side) {
      LAUNCH("gemm_gate_up_shared", launch_gemm(swf, EPI_GATEUP, sgp, stream));
      LAUNCH("gemm_down_shared", launch_gemm(swf, EPI_BF16, sdp, stream));
    }
  }
  HIP_TRY(joiner.join());
  // Y_perm and the shared output are bf16 here (the combine sums in fp32 and rounds once)
  LAUNCH("combine", launch_combine(at<void>(ws, L.yperm), true, inv, w, ysh, true, T, K, H, out, stream));
  return MOE_OK;
}

// Workspace of moe_forward_noalloc: a file-scope device array, one copy per
// GPU, held from the library's first use on that GPU until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory: host
// code uses only the address hipGetSymbolAddress gives for the current
// device (g_scratch), never the name.
constexpr size_t kScratchBytes = size_t(32) << 20;
static_assert(kScratchBytes >= size_t(kFusedCtrBytes), "scratch holds the counter block");
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

struct ScratchDev {
  void* ptr = nullptr;
};
std::mutex g_scratch_mu;
ScratchDev g_scratch[64];

// zero-fills n 16-byte words at p (a kernel, not a memset: callers may be
// under graph capture)
__global__ void zero_words_kernel(i32x4* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = i32x4{0, 0, 0, 0};
}

// The scratch address on the device of `stream`, set up on first use: the
// symbol is resolved with that device current and its counter block (which
// the single-launch path needs zero before its first launch) is cleared on
// `stream`.  Null if the device cannot be had.
void* scratch_for(hipStream_t stream) {
  int dev = 0, cur = 0;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  ScratchDev& sd = g_scratch[dev];
  if (sd.ptr) return sd.ptr;
  if (hipGetDevice(&cur) != hipSuccess || hipSetDevice(dev) != hipSuccess) return nullptr;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  (void)hipSetDevice(cur);
  if (e != hipSuccess || !p) return nullptr;
  const int n = kFusedCtrBytes / 16;
  hipLaunchKernelGGL(zero_words_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, static_cast<i32x4*>(p), n);
  if (hipGetLastError() != hipSuccess) return nullptr;
  sd.ptr = p;
  return p;
}

// ------------------------------------------------------------------ backward
struct BwdWs {
  size_t logits, ids, w, off, perm, inv, hist, tiles, ntiles;
  size_t G, U, h, Y, dw, dY, dh, dg, du, dXr;
  size_t Gs, Us, hs, dhs, dgs, dus, dXs;
  size_t dl, dlb, dXw;
  size_t total;
};

BwdWs bwd_plan(const moe_config* c, int Tm) {
  const size_t T = size_t(std::max(Tm, 1)), K = c->topk, E = c->n_experts, H = c->hidden, I = c->inter,
               Is = c->shared_inter, TK = T * K;
  BwdWs s{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o += up(std::max<size_t>(bytes, 16));
    return at;
  };
  s.logits = take(T * E * 4);
  s.ids = take(TK * 4);
  s.w = take(TK * 4);
  s.off = take((E + 1) * 4);
  s.perm = take(TK * 4);
  s.inv = take(TK * 4);
  s.hist = take(permute_hist_ints(int(TK), int(E)) * 4);
  s.tiles = take(size_t(2) * max_tiles(int(TK), int(E), kGemmBM) * 4);
  s.ntiles = take(16);
  s.G = take(TK * I * 4);
  s.U = take(TK * I * 4);
  s.h = take(TK * I * 2);
  s.Y = take(TK * H * 4);
  s.dw = take(TK * 4);
  s.dY = take(TK * H * 2);
  s.dh = take(TK * I * 4);
  s.dg = take(TK * I * 2);
  s.du = take(TK * I * 2);
  s.dXr = take(TK * H * 4);
  if (Is) {
    s.Gs = take(T * Is * 4);
    s.Us = take(T * Is * 4);
    s.hs = take(T * Is * 2);
    s.dhs = take(T * Is * 4);
    s.dgs = take(T * Is * 2);
    s.dus = take(T * Is * 2);
    s.dXs = take(T * H * 4);
  }
  s.dl = take(T * E * 4);
  s.dlb = take(T * E * 2);
  s.dXw = take(T * H * 4);
  s.total = o;
  return s;
}

bool bwd_supported(const moe_config* c) {
  return c->routed_wfmt == W_BF16 && c->routed_afmt == A_NONE &&
         (c->shared_inter == 0 || (c->shared_wfmt == W_BF16 && c->shared_afmt == A_NONE));
}

// the recomputed forward of one FFN on rows already laid out (routed: per
// segment, gathered from x through perm / K; shared: all T rows): G, U fp32,
// h = SiLU(G) U bf16, and (routed) Y = h Wd^T fp32
moe_status bwd_ffn_forward(const moe_config* c, bool routed, const uint16_t* x, int rows, const int* perm,
                           const int* off, const int* tiles, const int* ntiles, const moe_ffn_weights* W, float* G,
                           float* U, uint16_t* h, float* Y, hipStream_t s) {
  hipStream_t s_ = s;
  const int H = c->hidden, I = routed ? c->inter : c->shared_inter, E = c->n_experts;
  for (int k = 0; k < 2; ++k) {
    GemmParams g{};
    g.A = x;
    g.lda = H;
    g.a_map = routed ? perm : nullptr;
    g.a_div = routed ? c->topk : 1;
    g.B0 = k ? W->up : W->gate;
    g.b_stride = long(I) * H;
    g.N = I;
    g.K = H;
    g.seg = routed ? off : nullptr;
    g.M = rows;
    g.tiles = routed ? tiles : nullptr;
    g.ntiles = routed ? ntiles : nullptr;
    g.max_tiles = routed ? max_tiles(rows, E, kGemmBM) : 0;
    g.bm = kGemmBM;
    g.C = k ? U : G;
    g.ldc = I;
    LAUNCH(k ? "bwd_up_fwd" : "bwd_gate_fwd", launch_gemm(W_BF16, EPI_F32, g, s));
  }
  LAUNCH("bwd_swiglu_fwd", launch_swiglu_fwd(G, U, long(rows) * I, h, s));
  if (Y) {
    GemmParams d{};
    d.A = h;
    d.lda = I;
    d.B0 = W->down;
    d.b_stride = long(H) * I;
    d.N = H;
    d.K = I;
    d.seg = off;
    d.M = rows;
    d.tiles = tiles;
    d.ntiles = ntiles;
    d.max_tiles = max_tiles(rows, E, kGemmBM);
    d.bm = kGemmBM;
    d.C = Y;
    d.ldc = H;
    LAUNCH("bwd_down_fwd", launch_gemm(W_BF16, EPI_F32, d, s));
  }
  return MOE_OK;
}

// dh, then dg / du, then dX (two passes) and the three weight gradients of
// one FFN, from dY (bf16, rows laid out as the FFN's rows)
moe_status bwd_ffn_backward(const moe_config* c, bool routed, const uint16_t* x, int rows, const int* perm,
                            const int* off, const int* tiles, const int* ntiles, const moe_ffn_weights* W,
                            const moe_ffn_grads* D, const float* G, const float* U, const uint16_t* h,
                            const uint16_t* dY, float* dh, uint16_t* dg, uint16_t* du, float* dX, hipStream_t s) {
  hipStream_t s_ = s;
  const int H = c->hidden, I = routed ? c->inter : c->shared_inter, E = c->n_experts;
  const int ngroups = routed ? E : 1;
  BwdGemmParams n{};  // dh = dY Wd: A = dY [rows][H], B = Wd [H][I]
  n.A0 = dY;
  n.lda = H;
  n.B0 = static_cast<const uint16_t*>(W->down);
  n.ldb = I;
  n.b_stride = long(H) * I;
  n.npass = 1;
  n.N = I;
  n.K = H;
  n.rows = rows;
  n.seg = routed ? off : nullptr;
  n.tiles = routed ? tiles : nullptr;  // 128-row tiles (the forward's list)
  n.ntiles = routed ? ntiles : nullptr;
  n.max_tiles = routed ? max_tiles(rows, E, kGemmBM) : 0;
  n.C = dh;
  n.ldc = I;
  LAUNCH("bwd_dh", launch_bwd_gemm(false, false, n, 1, s));
  LAUNCH("bwd_swiglu", launch_swiglu_bwd(G, U, dh, long(rows) * I, dg, du, s));
  BwdGemmParams x2 = n;  // dX = dg Wg + du Wu: A = dg / du [rows][I], B = Wg / Wu [I][H]
  x2.A0 = dg;
  x2.A1 = du;
  x2.lda = I;
  x2.B0 = static_cast<const uint16_t*>(W->gate);
  x2.B1 = static_cast<const uint16_t*>(W->up);
  x2.ldb = H;
  x2.b_stride = long(I) * H;
  x2.npass = 2;
  x2.N = H;
  x2.K = I;
  x2.K1 = I;
  x2.C = dX;
  x2.ldc = H;
  LAUNCH("bwd_dx", launch_bwd_gemm(false, false, x2, 1, s));
  BwdGemmParams t{};  // dWd[e] = dY_e^T h_e: P = dY [rows][H], Q = h [rows][I]
  t.A0 = dY;
  t.lda = H;
  t.B0 = h;
  t.ldb = I;
  t.npass = 1;
  t.M = H;
  t.N = I;
  t.rows = rows;
  t.seg = routed ? off : nullptr;
  t.C = D->down;
  t.ldc = I;
  t.c_stride = long(H) * I;
  LAUNCH("bwd_ddown", launch_bwd_gemm(true, true, t, ngroups, s));
  for (int k = 0; k < 2; ++k) {  // dWg[e] = dg_e^T X_e, dWu[e] = du_e^T X_e: P = dg / du [rows][I], Q = x rows
    BwdGemmParams q{};
    q.A0 = k ? du : dg;
    q.lda = I;
    q.B0 = x;
    q.ldb = H;
    q.b_map = routed ? perm : nullptr;
    q.b_div = routed ? c->topk : 1;
    q.npass = 1;
    q.M = I;
    q.N = H;
    q.rows = rows;
    q.seg = routed ? off : nullptr;
    q.C = k ? D->up : D->gate;
    q.ldc = H;
    q.c_stride = long(I) * H;
    LAUNCH(k ? "bwd_dup" : "bwd_dgate", launch_bwd_gemm(true, true, q, ngroups, s));
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int32_t st) {
  switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: configuration not implemented";
    case MOE_EALIGN: return "MOE_EALIGN: pointer or dimension misaligned";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace too small";
    case MOE_EHIP: return "MOE_EHIP: HIP launch failed";
    case MOE_EWAIT: return "MOE_EWAIT: a bounded wait of the single-launch path gave up (NaN output rows)";
    default: return "unknown moe_status";
  }
}

moe_status moe_workspace_size(const moe_config* cfg, int32_t max_tokens, size_t* bytes) {
  if (!bytes || max_tokens < 0) return MOE_EINVAL;
  moe_status st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  *bytes = plan(cfg, max_tokens).total;
  return MOE_OK;
}

moe_status moe_route(const moe_config* cfg, const uint16_t* x, int32_t T, const uint16_t* w_router, const float* bias,
                     int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !topk_ids || !topk_w || !ws) return MOE_EINVAL;
  for (const void* p : {(const void*)x, (const void*)w_router, (const void*)ws})
    if (!aligned16(p)) return MOE_EALIGN;
  const Ws L = plan(cfg, T);
  if (ws_bytes < L.total) return MOE_EWORKSPACE;
  return do_route(cfg, x, T, w_router, bias, topk_ids, topk_w, ws, L, stream);
}

moe_status moe_permute(const moe_config* cfg, const int32_t* topk_ids, int32_t T, const uint16_t* x,
                       int32_t* expert_offsets, int32_t* perm_src, int32_t* inv_pos, void* x_perm,
                       void* x_perm_scale, void* ws, size_t ws_bytes, hipStream_t stream) {
  hipStream_t s_ = stream;
  moe_status st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!topk_ids || !expert_offsets || !perm_src || !inv_pos || !ws) return MOE_EINVAL;
  if (x_perm && !x) return MOE_EINVAL;
  if (x_perm && cfg->routed_afmt != A_NONE && !x_perm_scale) return MOE_EINVAL;
  if (!aligned16(ws) || (x && !aligned16(x)) || (x_perm && !aligned16(x_perm))) return MOE_EALIGN;
  const Ws L = plan(cfg, T);
  if (ws_bytes < L.total) return MOE_EWORKSPACE;
  const int TK = T * cfg->topk;
  LAUNCH("permute", launch_permute(topk_ids, TK, cfg->n_experts, at<int>(ws, L.hist), expert_offsets, perm_src, inv_pos, nullptr, nullptr, kGemmBM,
                         stream));
  if (x_perm)
    LAUNCH("quant_rows", launch_quant_rows(x, false, TK, cfg->hidden, perm_src, cfg->topk, cfg->routed_afmt, x_perm, x_perm_scale,
                              nullptr, stream));
  return MOE_OK;
}

moe_status moe_expert_ffn(const moe_config* cfg, int32_t which, const void* x, const void* x_scale, int32_t rows,
                          const int32_t* seg_offsets, const moe_ffn_weights* W, float* y, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  hipStream_t s_ = stream;
  moe_status st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (which != 0 && which != 1) return MOE_EINVAL;
  const bool routed = which == 0;
  if (!routed && cfg->shared_inter == 0) return MOE_EINVAL;
  if (rows < 0) return MOE_EINVAL;
  if (rows == 0) return MOE_OK;
  if (!x || !W || !y || !ws || (routed && !seg_offsets)) return MOE_EINVAL;
  const int wf = routed ? cfg->routed_wfmt : cfg->shared_wfmt;
  const int af = routed ? cfg->routed_afmt : cfg->shared_afmt;
  if ((st = check_weights(W, wf)) != MOE_OK) return st;
  if (x_scale && af == A_NONE) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(y) || !aligned16(ws) || (x_scale && !aligned16(x_scale))) return MOE_EALIGN;
  // rows <= max_tokens*K for routed, <= max_tokens for shared: size the plan accordingly
  const int Tm = routed ? (rows + cfg->topk - 1) / cfg->topk : rows;
  const Ws L = plan(cfg, Tm);
  if (ws_bytes < L.total) return MOE_EWORKSPACE;
  const int H = cfg->hidden, I = routed ? cfg->inter : cfg->shared_inter, E = cfg->n_experts;
  const int fp = forced_path();
  const bool gemv = fp == 1 || (fp != 2 && rows <= kGemvMaxRows) || !gemm_pair(wf, af);
  if (fp == 2 && !gemm_pair(wf, af)) return MOE_EUNSUPPORTED;

  if (gemv) {
    const void* xin = x;
    bool xf32 = false;
    if (x_scale) {  // pre-quantised rows: dequantise to fp32
      LAUNCH("dequant_rows", launch_dequant_rows(static_cast<const uint8_t*>(x), x_scale, af, rows, H, at<float>(ws, L.xq), stream));
      xin = at<float>(ws, L.xq);
      xf32 = true;
    } else if (af != A_NONE) {
      LAUNCH("quant_rows", launch_quant_rows(x, false, rows, H, nullptr, 1, af, nullptr, nullptr, at<float>(ws, L.xq), stream));
      xin = at<float>(ws, L.xq);
      xf32 = true;
    }
    float* h = at<float>(ws, routed ? L.h : L.hsh);
    GemvUpParams u{};
    u.T = rows;
    u.H = H;
    u.E = E;
    if (routed) {
      u.wfmt = wf;
      u.swfmt = wf;
      u.x = xin;
      u.x_f32 = xf32;
      u.seg = seg_offsets;
      u.g = W->gate; u.u = W->up; u.gs = W->gate_s; u.us = W->up_s;
      u.I = I;
      u.h = h;
    } else {
      u.wfmt = wf;
      u.swfmt = wf;
      u.xs = xin;
      u.xs_f32 = xf32;
      u.sg = W->gate; u.su = W->up; u.sgs = W->gate_s; u.sus = W->up_s;
      u.Is = I;
      u.I = 128;
      u.hs = h;
    }
    LAUNCH("gemv_gate_up", launch_gemv_gate_up(u, stream));
    if (af != A_NONE) LAUNCH("quant_rows", launch_quant_rows(h, true, rows, I, nullptr, 1, af, nullptr, nullptr, h, stream));
    GemvDownParams d{};
    d.wfmt = wf;
    d.swfmt = wf;
    d.H = H;
    d.rows = rows;
    d.y = y;
    d.E = E;
    if (routed) {
      d.I = I; d.h = h; d.d = W->down; d.ds = W->down_s; d.seg = seg_offsets;
    } else {
      d.Is = I; d.hs = h; d.sd = W->down; d.sds = W->down_s;
    }
    LAUNCH("gemv_down", launch_gemv_down(d, stream));
    return MOE_OK;
  }

  // GEMM path
  const void* A = x;
  const void* As = x_scale;
  if (!x_scale && af != A_NONE) {
    LAUNCH("quant_rows", launch_quant_rows(x, false, rows, H, nullptr, 1, af, at<void>(ws, L.xq), at<void>(ws, L.xqs), nullptr,
                              stream));
    A = at<void>(ws, L.xq);
    As = at<void>(ws, L.xqs);
  }
  int* tiles = nullptr;
  int* ntiles = nullptr;
  int maxt = 0;
  const int bm = ffn_tile_rows(wf, H, I);
  if (routed) {
    tiles = at<int>(ws, L.tiles);
    ntiles = at<int>(ws, L.ntiles);
    maxt = max_tiles(rows, E, bm);
    LAUNCH("build_tiles", launch_build_tiles(seg_offsets, E, rows, bm, tiles, ntiles, stream));
  }
  return gemm_ffn(cfg, routed, A, As, nullptr, 1, rows, routed ? seg_offsets : nullptr, tiles, ntiles, maxt, bm, W,
                  at<void>(ws, routed ? L.h : L.hsh), at<void>(ws, routed ? L.hs : L.hshs), y, false, stream);
}

moe_status moe_combine(const moe_config* cfg, const float* y_perm, const int32_t* inv_pos, const float* topk_w,
                       const float* y_shared, int32_t T, uint16_t* out, hipStream_t stream) {
  hipStream_t s_ = stream;
  moe_status st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!y_perm || !inv_pos || !topk_w || !out) return MOE_EINVAL;
  if (!aligned16(y_perm) || !aligned16(out) || (y_shared && !aligned16(y_shared))) return MOE_EALIGN;
  LAUNCH("combine", launch_combine(y_perm, false, inv_pos, topk_w, y_shared, false, T, cfg->topk, cfg->hidden, out, stream));
  return MOE_OK;
}

moe_status moe_forward(const moe_config* cfg, const uint16_t* x, int32_t T, const uint16_t* w_router,
                       const float* bias, const moe_ffn_weights* routed, const moe_ffn_weights* shared, uint16_t* out,
                       int32_t* topk_ids_out, float* topk_w_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return forward_impl(cfg, x, T, w_router, bias, routed, shared, out, topk_ids_out, topk_w_out, ws, ws_bytes, stream,
                      true);
}

moe_status moe_forward_norm(const moe_config* cfg, const uint16_t* h, int32_t T, const moe_norm* norm,
                            const uint16_t* w_router, const float* bias, const moe_ffn_weights* routed,
                            const moe_ffn_weights* shared, uint16_t* out, int32_t* topk_ids_out, float* topk_w_out,
                            uint16_t* x_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!norm || !norm->gamma) return MOE_EINVAL;
  NormArgs nm;
  nm.gamma = norm->gamma;
  nm.eps = norm->eps;
  nm.x_out = x_out;
  return forward_impl(cfg, h, T, w_router, bias, routed, shared, out, topk_ids_out, topk_w_out, ws, ws_bytes, stream,
                      true, nm);
}

moe_status moe_route_dispatch(const moe_config* cfg, const uint16_t* h, int32_t T, const moe_norm* norm,
                              const uint16_t* w_router, const float* bias, int32_t* topk_ids, float* topk_w,
                              int32_t* expert_offsets, int32_t* perm_src, int32_t* inv_pos, uint16_t* x_out, void* xq,
                              void* xq_scale, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!h || !w_router || !topk_ids || !topk_w || !expert_offsets || !perm_src || !inv_pos || !ws) return MOE_EINVAL;
  if (norm && !norm->gamma) return MOE_EINVAL;
  if (norm && !(norm->eps >= 0.f)) return MOE_EINVAL;
  if (xq && (cfg->routed_afmt == A_NONE || !xq_scale)) return MOE_EINVAL;
  for (const void* p : {(const void*)h, (const void*)w_router, (const void*)ws})
    if (!aligned16(p)) return MOE_EALIGN;
  if ((norm && !aligned16(norm->gamma)) || (x_out && !aligned16(x_out)) || (xq && !aligned16(xq))) return MOE_EALIGN;
  const Ws L = plan(cfg, T);
  if (ws_bytes < L.total) return MOE_EWORKSPACE;
  NormArgs nm;
  if (norm) {
    nm.gamma = norm->gamma;
    nm.eps = norm->eps;
  }
  return route_dispatch(cfg, h, T, nm, w_router, bias, topk_ids, topk_w, expert_offsets, perm_src, inv_pos, x_out, xq,
                        xq_scale, nullptr, nullptr, 0, ws, L, stream);
}

moe_status moe_backward_workspace_size(const moe_config* cfg, int32_t max_tokens, size_t* bytes) {
  if (!bytes || max_tokens < 0) return MOE_EINVAL;
  moe_status st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!bwd_supported(cfg)) return MOE_EUNSUPPORTED;
  *bytes = bwd_plan(cfg, max_tokens).total;
  return MOE_OK;
}

moe_status moe_backward(const moe_config* cfg, const uint16_t* x, int32_t T, const uint16_t* w_router,
                        const float* bias, const moe_ffn_weights* routed, const moe_ffn_weights* shared,
                        const uint16_t* dy, uint16_t* dx, uint16_t* d_router, float* d_bias,
                        const moe_ffn_grads* d_routed, const moe_ffn_grads* d_shared, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  hipStream_t s_ = stream;
  moe_status st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!bwd_supported(cfg)) return MOE_EUNSUPPORTED;
  if (T < 0) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  const bool has_shared = cfg->shared_inter > 0;
  if (!x || !w_router || !routed || !dy || !dx || !d_router || !d_routed || !ws) return MOE_EINVAL;
  if (!d_routed->gate || !d_routed->up || !d_routed->down) return MOE_EINVAL;
  if (has_shared && (!shared || !d_shared || !d_shared->gate || !d_shared->up || !d_shared->down)) return MOE_EINVAL;
  if ((st = check_weights(routed, W_BF16)) != MOE_OK) return st;
  if (has_shared && (st = check_weights(shared, W_BF16)) != MOE_OK) return st;
  for (const void* p : {(const void*)x, (const void*)w_router, (const void*)dy, (const void*)dx, (const void*)d_router,
                        (const void*)ws, (const void*)d_routed->gate, (const void*)d_routed->up,
                        (const void*)d_routed->down})
    if (!aligned16(p)) return MOE_EALIGN;
  const BwdWs L = bwd_plan(cfg, T);
  if (ws_bytes < L.total) return MOE_EWORKSPACE;
  const int H = cfg->hidden, K = cfg->topk, E = cfg->n_experts, TK = T * K;
  int* ids = at<int>(ws, L.ids);
  float* w = at<float>(ws, L.w);
  int* off = at<int>(ws, L.off);
  int* perm = at<int>(ws, L.perm);
  int* inv = at<int>(ws, L.inv);
  float* logits = at<float>(ws, L.logits);
  // routing again (the forward's: fp32 logits, then the same top-k), with the
  // logits kept for the softmax backward
  {
    GemmParams g{};
    g.A = x;
    g.lda = H;
    g.B0 = w_router;
    g.N = E;
    g.K = H;
    g.M = T;
    g.C = logits;
    g.ldc = E;
    LAUNCH("bwd_router_logits", launch_gemm(W_BF16, EPI_F32, g, stream));
    LAUNCH("bwd_topk", launch_topk(logits, T, bias, route_params(cfg), ids, w, stream));
  }
  LAUNCH("bwd_permute", launch_permute(ids, TK, E, at<int>(ws, L.hist), off, perm, inv, at<int>(ws, L.tiles),
                                       at<int>(ws, L.ntiles), kGemmBM, stream));
  // routed experts: recomputed forward, combine backward, FFN backward
  if ((st = bwd_ffn_forward(cfg, true, x, TK, perm, off, at<int>(ws, L.tiles), at<int>(ws, L.ntiles), routed,
                            at<float>(ws, L.G), at<float>(ws, L.U), at<uint16_t>(ws, L.h), at<float>(ws, L.Y),
                            stream)) != MOE_OK)
    return st;
  float* dw = at<float>(ws, L.dw);
  LAUNCH("bwd_combine", launch_combine_bwd(dy, at<float>(ws, L.Y), inv, w, T, K, H, dw, at<uint16_t>(ws, L.dY), stream));
  if ((st = bwd_ffn_backward(cfg, true, x, TK, perm, off, at<int>(ws, L.tiles), at<int>(ws, L.ntiles), routed,
                             d_routed, at<float>(ws, L.G), at<float>(ws, L.U), at<uint16_t>(ws, L.h),
                             at<uint16_t>(ws, L.dY), at<float>(ws, L.dh), at<uint16_t>(ws, L.dg), at<uint16_t>(ws, L.du),
                             at<float>(ws, L.dXr), stream)) != MOE_OK)
    return st;
  // shared expert: dY = dy on every token
  float* dXs = nullptr;
  if (has_shared) {
    if ((st = bwd_ffn_forward(cfg, false, x, T, nullptr, nullptr, nullptr, nullptr, shared, at<float>(ws, L.Gs),
                              at<float>(ws, L.Us), at<uint16_t>(ws, L.hs), nullptr, stream)) != MOE_OK)
      return st;
    dXs = at<float>(ws, L.dXs);
    if ((st = bwd_ffn_backward(cfg, false, x, T, nullptr, nullptr, nullptr, nullptr, shared, d_shared,
                               at<float>(ws, L.Gs), at<float>(ws, L.Us), at<uint16_t>(ws, L.hs), dy,
                               at<float>(ws, L.dhs), at<uint16_t>(ws, L.dgs), at<uint16_t>(ws, L.dus), dXs, stream)) !=
        MOE_OK)
      return st;
  }
  // router: softmax backward, d_router = dl^T x, dx += dl Wr, d_bias = sum dl
  float* dl = at<float>(ws, L.dl);
  uint16_t* dlb = at<uint16_t>(ws, L.dlb);
  LAUNCH("bwd_router", launch_router_bwd(logits, bias, ids, dw, T, E, K, cfg->route_scale, dl, dlb, stream));
  {
    BwdGemmParams t{};
    t.A0 = dlb;
    t.lda = E;
    t.B0 = x;
    t.ldb = H;
    t.npass = 1;
    t.M = E;
    t.N = H;
    t.rows = T;
    t.C = d_router;
    t.ldc = H;
    LAUNCH("bwd_drouter", launch_bwd_gemm(true, true, t, 1, stream));
    BwdGemmParams n{};
    n.A0 = dlb;
    n.lda = E;
    n.B0 = w_router;
    n.ldb = H;
    n.npass = 1;
    n.N = H;
    n.K = E;
    n.rows = T;
    n.C = at<float>(ws, L.dXw);
    n.ldc = H;
    LAUNCH("bwd_dx_router", launch_bwd_gemm(false, false, n, 1, stream));
  }
  if (d_bias) LAUNCH("bwd_dbias", launch_colsum(dl, T, E, d_bias, stream));
  LAUNCH("bwd_dx_sum", launch_dx_sum(at<float>(ws, L.dXr), inv, K, dXs, at<float>(ws, L.dXw), T, H, dx, stream));
  return MOE_OK;
}

moe_status moe_forward_noalloc(const moe_config* cfg, const uint16_t* x, int32_t T, const uint16_t* w_router,
                               const float* bias, const moe_ffn_weights* routed, const moe_ffn_weights* shared,
                               uint16_t* out, int32_t* topk_ids_out, float* topk_w_out, hipStream_t stream) {
  moe_status st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (plan(cfg, T).total > kScratchBytes) return MOE_EWORKSPACE;
  void* ws = scratch_for(stream);
  if (!ws) return MOE_EHIP;
  return forward_impl(cfg, x, T, w_router, bias, routed, shared, out, topk_ids_out, topk_w_out, ws, kScratchBytes,
                      stream, false);
}

moe_status moe_debug_validate_dispatch(const moe_config* cfg, int32_t T, const int32_t* topk_ids, const void* ws,
                                       size_t ws_bytes, int32_t* flags, hipStream_t stream) {
  hipStream_t s_ = stream;
  moe_status st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (T <= 0 || !topk_ids || !ws || !flags) return MOE_EINVAL;
  const Ws L = plan(cfg, T);
  if (ws_bytes < L.total) return MOE_EWORKSPACE;
  const int bm = ffn_tile_rows(cfg->routed_wfmt, cfg->hidden, cfg->inter);
  LAUNCH("validate_dispatch",
         launch_validate_dispatch(topk_ids, T * cfg->topk, cfg->n_experts, at<int>(const_cast<void*>(ws), L.offsets),
                                  at<int>(const_cast<void*>(ws), L.perm), at<int>(const_cast<void*>(ws), L.inv),
                                  at<int>(const_cast<void*>(ws), L.tiles), at<int>(const_cast<void*>(ws), L.ntiles),
                                  max_tiles(T * cfg->topk, cfg->n_experts, kGemmBM), bm, flags, stream));
  return MOE_OK;
}

moe_status moe_debug_ws_offset(const moe_config* cfg, int32_t max_tokens, int32_t region, size_t* offset) {
  if (!offset || max_tokens < 0) return MOE_EINVAL;
  moe_status st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  const Ws L = plan(cfg, max_tokens);
  switch (region) {
    case 0: *offset = L.offsets; return MOE_OK;
    case 1: *offset = L.perm; return MOE_OK;
    case 2: *offset = L.inv; return MOE_OK;
    case 3: *offset = L.tiles; return MOE_OK;
    case 4: *offset = L.ntiles; return MOE_OK;
    default: return MOE_EINVAL;
  }
}

int32_t moe_debug_ffn_tile_rows(const moe_config* cfg, int32_t which) {
  if (check_cfg(cfg) != MOE_OK || (which != 0 && which != 1)) return -1;
  return which == 0 ? ffn_tile_rows(cfg->routed_wfmt, cfg->hidden, cfg->inter)
                    : ffn_tile_rows(cfg->shared_wfmt, cfg->hidden, cfg->shared_inter);
}

moe_status moe_workspace_check(void* ws, size_t ws_bytes, int32_t clear, hipStream_t stream) {
  if (!ws || ws_bytes < 4) return MOE_EINVAL;
  uint32_t word = 0;
  HIP_TRY(hipMemcpyAsync(&word, ws, 4, hipMemcpyDeviceToHost, stream));
  HIP_TRY(hipStreamSynchronize(stream));
  if (word && clear) {
    static const uint32_t zero = 0;
    HIP_TRY(hipMemcpyAsync(ws, &zero, 4, hipMemcpyHostToDevice, stream));
    HIP_TRY(hipStreamSynchronize(stream));
  }
  return word ? MOE_EWAIT : MOE_OK;
}

moe_status moe_debug_trace(hipEvent_t* events, int32_t n_events) {
  if (events && n_events < 2) return MOE_EINVAL;
  g_trace.ev = events;
  g_trace.max = events ? n_events : 0;
  g_trace.n = 0;
  return MOE_OK;
}

int32_t moe_debug_trace_count(void) { return g_trace.n; }

const char* moe_debug_trace_name(int32_t i) {
  return (i >= 0 && i < g_trace.n && i < 128) ? g_trace.names[i] : "";
}

moe_status moe_debug_e4m3_decode(const uint8_t* codes, float* out, int32_t n, hipStream_t stream) {
  hipStream_t s_ = stream;
  if (n < 0 || (n > 0 && (!codes || !out))) return MOE_EINVAL;
  if (n == 0) return MOE_OK;
  LAUNCH("e4m3_decode", launch_e4m3_decode(codes, out, n, stream));
  return MOE_OK;
}

moe_status moe_debug_e4m3_encode(const float* in, uint8_t* codes, int32_t n, hipStream_t stream) {
  hipStream_t s_ = stream;
  if (n < 0 || (n > 0 && (!codes || !in))) return MOE_EINVAL;
  if (n == 0) return MOE_OK;
  LAUNCH("e4m3_encode", launch_e4m3_encode(in, codes, n, stream));
  return MOE_OK;
}

}  // extern "C"
