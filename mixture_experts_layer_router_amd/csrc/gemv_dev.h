// Device-side GEMV building blocks of the small-batch expert FFN: FP8 / bf16
// weight chunks against fp32 or bf16 activations, per-block scales, the
// gate/up item (SiLU(g) * u) and the down-projection chunk streams.  Shared by
// the multi-launch kernels (gemv.hip) and the single-launch decode (decode.hip).
#pragma once
#include "common.h"
#include "kernels.h"
#include "route_dev.h"

namespace moe {

constexpr int RU = 4;  // intermediate columns per gate/up wave item (4 gate + 4 up rows)
constexpr int CPI = 2; // weight chunks whose loads are issued together in the gate/up loop
constexpr int RD = 8;  // output rows per down workgroup
constexpr int DW = 4;  // waves per down workgroup

template <int WF>
struct Fmt {
  static constexpr int EPL = (WF == W_BF16) ? 8 : 16;  // elements per 16-byte lane load
  static constexpr int CW = 64 * EPL;                  // elements per wave chunk
  static constexpr int ES = (WF == W_BF16) ? 2 : 1;    // bytes per element
};

// partial dot of one 16-byte weight chunk with EPL x values
template <int WF>
MOE_DEV float dot_chunk(u32x4 w, const float* x) {
  float s0 = 0.f, s1 = 0.f;
  if (WF == W_BF16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s0 = fmaf(__uint_as_float(w[q] << 16), x[2 * q], s0);
      s1 = fmaf(__uint_as_float(w[q] & 0xffff0000u), x[2 * q + 1], s1);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x2 a = e4m3x2_to_f32(w[q], false);
      const f32x2 b = e4m3x2_to_f32(w[q], true);
      s0 = fmaf(a.x, x[4 * q + 0], s0);
      s1 = fmaf(a.y, x[4 * q + 1], s1);
      s0 = fmaf(b.x, x[4 * q + 2], s0);
      s1 = fmaf(b.y, x[4 * q + 3], s1);
    }
  }
  return s0 + s1;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// partial dot of one 16-byte weight chunk with EPL bf16 activations held as
// packed pairs: FP8 codes go to bf16 pairs with the gfx950 scaled converter
// (exact: every e4m3 value is a bf16 value) and v_dot2_f32_bf16 accumulates
// two products per instruction in fp32; bf16 weights feed v_dot2 directly.
MOE_DEV bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

template <int WF>
MOE_DEV float dot_chunk_bx(u32x4 w, const uint32_t* xp) {
  // words are taken out of the vector before any bit_cast: bit-casting a
  // vector element directly was lowered to the wrong register
  const uint32_t wq[4] = {w.x, w.y, w.z, w.w};
  float s0 = 0.f, s1 = 0.f;
  if (WF == W_BF16) {
    s0 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wq[0]), as_bf16x2(xp[0]), s0, false);
    s1 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wq[1]), as_bf16x2(xp[1]), s1, false);
    s0 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wq[2]), as_bf16x2(xp[2]), s0, false);
    s1 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wq[3]), as_bf16x2(xp[3]), s1, false);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wq[q], 1.0f, false);
      const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wq[q], 1.0f, true);
      s0 = __builtin_amdgcn_fdot2_f32_bf16(a, as_bf16x2(xp[2 * q]), s0, false);
      s1 = __builtin_amdgcn_fdot2_f32_bf16(b, as_bf16x2(xp[2 * q + 1]), s1, false);
    }
  }
  return s0 + s1;
}

// one 16-byte weight chunk as EPL/2 bf16 pairs, in dot_chunk_bx's order
template <int WF>
MOE_DEV void bf16_pairs(u32x4 w, uint32_t (&p)[Fmt<WF>::EPL / 2]) {
  const uint32_t wq[4] = {w.x, w.y, w.z, w.w};
  if (WF == W_BF16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) p[q] = wq[q];
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      p[2 * q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wq[q], 1.0f, false));
      p[2 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wq[q], 1.0f, true));
    }
  }
}
// dot of NP weight pairs with NP activation pairs: even pairs into one sum,
// odd pairs into the other, as dot_chunk_bx
template <int NP>
MOE_DEV float dot_pairs(const uint32_t (&w)[NP], const uint32_t* xp) {
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int q = 0; q < NP; q += 2) {
    s0 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w[q]), as_bf16x2(xp[q]), s0, false);
    s1 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w[q + 1]), as_bf16x2(xp[q + 1]), s1, false);
  }
  return s0 + s1;
}

// scale of weight element (row n, column k) of an [N][L] matrix
template <int WF>
MOE_DEV float wscale(const void* S, int n, int k, int L) {
  if (WF == W_FP8_B128) return static_cast<const float*>(S)[(n >> 7) * (L >> 7) + (k >> 7)];
  if (WF == W_MXFP8) return e8m0_to_f32(static_cast<const uint8_t*>(S)[size_t(n) * (L >> 5) + (k >> 5)]);
  return 1.0f;
}

template <int WF>
MOE_DEV size_t wstride(int N, int L) { return size_t(N) * L * Fmt<WF>::ES; }
template <int WF>
MOE_DEV size_t sstride(int N, int L) {
  return WF == W_FP8_B128 ? size_t(N / 128) * (L / 128) * 4 : (WF == W_MXFP8 ? size_t(N) * (L / 32) : 0);
}

// EPL activation values at x[off..off+EPL) as fp32 (x is fp32 or bf16)
template <bool F32, int EPL>
MOE_DEV void load_x(const void* x, size_t off, float (&v)[EPL]) {
  if (F32) {
#pragma unroll
    for (int i = 0; i < EPL / 4; ++i) {
      const f32x4 f = *reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + off + 4 * i);
      v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < EPL / 8; ++i) {
      const u32x4 u = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + off + 8 * i);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[8 * i + 2 * q] = __uint_as_float(u[q] << 16);
        v[8 * i + 2 * q + 1] = __uint_as_float(u[q] & 0xffff0000u);
      }
    }
  }
}

// One register stage of the gate/up stream: NR gate rows, NR up rows, x
// (fp32, or packed bf16 pairs when the activations are bf16), scales.
template <int WF, bool XF32, int NR = RU>
struct UpStage {
  u32x4 g[NR], u[NR];
  float x[XF32 ? Fmt<WF>::EPL : 1];
  uint32_t xp[XF32 ? 1 : Fmt<WF>::EPL / 2];
  float sg[NR], su[NR];
};

template <int WF, bool XF32, int NR>
MOE_DEV float up_dot(u32x4 w, const UpStage<WF, XF32, NR>& st) {
  if constexpr (XF32) return dot_chunk<WF>(w, st.x);
  else return dot_chunk_bx<WF>(w, st.xp);
}

// k is a valid column (callers clamp it); every lane always loads
template <int WF, bool XF32, int NR>
MOE_DEV void up_load(UpStage<WF, XF32, NR>& st, const uint8_t* gb, const uint8_t* ub, const void* gs, const void* us,
                     const void* x, int xrow, int H, int i0, int k) {
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    st.g[r] = *reinterpret_cast<const u32x4*>(gb + (size_t(r) * H + k) * Fmt<WF>::ES);
    st.u[r] = *reinterpret_cast<const u32x4*>(ub + (size_t(r) * H + k) * Fmt<WF>::ES);
  }
  if constexpr (XF32) {
    load_x<true, Fmt<WF>::EPL>(x, size_t(xrow) * H + k, st.x);
  } else {
#pragma unroll
    for (int i = 0; i < Fmt<WF>::EPL / 8; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + size_t(xrow) * H + k + 8 * i);
#pragma unroll
      for (int q = 0; q < 4; ++q) st.xp[4 * i + q] = v[q];
    }
  }
  if (WF == W_MXFP8) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      st.sg[r] = wscale<WF>(gs, i0 + r, k, H);
      st.su[r] = wscale<WF>(us, i0 + r, k, H);
    }
  } else {
    st.sg[0] = wscale<WF>(gs, i0, k, H);
    st.su[0] = wscale<WF>(us, i0, k, H);
  }
}

// adds the stage's partial products; lanes past the row end (valid false) add 0
template <int WF, bool XF32, int NR>
MOE_DEV void up_math(const UpStage<WF, XF32, NR>& st, bool valid, float (&ag)[NR], float (&au)[NR]) {
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const float sg = valid ? (WF == W_MXFP8 ? st.sg[r] : st.sg[0]) : 0.0f;
    const float su = valid ? (WF == W_MXFP8 ? st.su[r] : st.su[0]) : 0.0f;
    ag[r] = fmaf(up_dot<WF, XF32, NR>(st.g[r], st), sg, ag[r]);
    au[r] = fmaf(up_dot<WF, XF32, NR>(st.u[r], st), su, au[r]);
  }
}

// h[i0 .. i0+NR) = SiLU(x.Wg^T) * (x.Wu^T) for one x row.  NC chunks per
// iteration: all their loads (NC x 2NR x 16 bytes per lane) are issued before
// any is reduced, and no register stage is carried across iterations, so
// nothing forces a wait on loads still in flight.
// COH: store h with agent-scope atomic stores, so workgroups on other XCDs can
// read it inside the same launch once the producer has published completion.
template <int WF, bool XF32, int NR = RU, int NC = CPI, bool COH = false>
MOE_DEV void gate_up_item(const void* x, int H, int xrow, const void* g, const void* u, const void* gs,
                          const void* us, int i0, float* hrow) {
  constexpr int CW = Fmt<WF>::CW, EPL = Fmt<WF>::EPL;
  const int lane = lane_id();
  const uint8_t* gb = static_cast<const uint8_t*>(g) + size_t(i0) * H * Fmt<WF>::ES;
  const uint8_t* ub = static_cast<const uint8_t*>(u) + size_t(i0) * H * Fmt<WF>::ES;
  float ag[NR] = {}, au[NR] = {};
  const int kl = lane * EPL;
  for (int k0 = 0; k0 < H; k0 += NC * CW) {
    UpStage<WF, XF32, NR> st[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
      if (c == 0 || k0 + c * CW < H)  // uniform
        up_load<WF, XF32, NR>(st[c], gb, ub, gs, us, x, xrow, H, i0, min(k0 + c * CW + kl, H - EPL));
#pragma unroll
    for (int c = 0; c < NC; ++c)
      if (c == 0 || k0 + c * CW < H) up_math<WF, XF32, NR>(st[c], k0 + c * CW + kl < H, ag, au);
  }
  float mine = 0.f;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const float gv = wave_sum(ag[r]);
    const float uv = wave_sum(au[r]);
    if (lane == r) mine = silu(gv) * uv;
  }
  if (lane < NR) {
    if (COH)
      __hip_atomic_store(hrow + i0 + lane, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      hrow[i0 + lane] = mine;
  }
}

MOE_DEV int seg_of(const int* seg, int E, int r) {
  int lo = 0, hi = E;  // e with seg[e] <= r < seg[e+1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (seg[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

// ------------------------------------------------------------------ down

// Where one lane's 16-byte chunk of the concatenated K lives.
struct DownSrc {
  const uint8_t* w;  // weight row n0 at this chunk's column
  const float* h;    // activation at this chunk's column
  const void* s;     // scale array of the matrix (null for bf16)
  int L;             // row length of the matrix
  int off;           // column within the matrix
  float f;           // routing weight folded into the scale
  bool ok;
};

template <int WF>
struct DownStage {
  u32x4 w[RD];
  float h[Fmt<WF>::EPL];
  float sc[RD];
};

template <int WF>
MOE_DEV void down_load(DownStage<WF>& st, const DownSrc& d, int n0) {
#pragma unroll
  for (int r = 0; r < RD; ++r) st.w[r] = *reinterpret_cast<const u32x4*>(d.w + size_t(r) * d.L * Fmt<WF>::ES);
  load_x<true, Fmt<WF>::EPL>(d.h, 0, st.h);
  if (WF == W_MXFP8) {
#pragma unroll
    for (int r = 0; r < RD; ++r) st.sc[r] = d.f * wscale<WF>(d.s, n0 + r, d.off, d.L);
  } else {
    st.sc[0] = d.f * wscale<WF>(d.s, n0, d.off, d.L);
  }
}

// lanes whose chunk column lies past the end (ok false) add 0
template <int WF>
MOE_DEV void down_math(const DownStage<WF>& st, bool ok, float (&acc)[RD]) {
#pragma unroll
  for (int r = 0; r < RD; ++r) {
    const float sc = ok ? (WF == W_MXFP8 ? st.sc[r] : st.sc[0]) : 0.0f;
    acc[r] = fmaf(dot_chunk<WF>(st.w[r], st.h), sc, acc[r]);
  }
}

// chunk c (global index over the routed part) of the concatenation of nseg
// routed [H][I] matrices for this lane
// sid/swt: the row's expert ids and routing weights staged in LDS
template <int WF>
MOE_DEV DownSrc routed_src(const GemvDownParams& p, int row, int n0, int c, int nseg, float inv_i, const int* sid,
                           const float* swt) {
  DownSrc d{};
  const int kraw = c * Fmt<WF>::CW + lane_id() * Fmt<WF>::EPL;
  d.ok = kraw < nseg * p.I;
  const int kc = min(kraw, nseg * p.I - Fmt<WF>::EPL);  // past the end: a valid column, masked later
  int j = int(float(kc) * inv_i);                       // segment index without an integer division
  j -= (j * p.I > kc);
  j += ((j + 1) * p.I <= kc);
  d.off = kc - j * p.I;
  d.L = p.I;
  const int e = sid[j];
  const int hrow = nseg == 1 ? row : row * p.K + j;
  d.f = swt[j];
  d.w = static_cast<const uint8_t*>(p.d) + e * wstride<WF>(p.H, p.I) + (size_t(n0) * p.I + d.off) * Fmt<WF>::ES;
  d.s = p.ds ? static_cast<const uint8_t*>(p.ds) + e * sstride<WF>(p.H, p.I) : nullptr;
  d.h = p.h + size_t(hrow) * p.I + d.off;
  return d;
}

template <int SWF>
MOE_DEV DownSrc shared_src(const GemvDownParams& p, int row, int n0, int c) {
  DownSrc d{};
  const int kraw = c * Fmt<SWF>::CW + lane_id() * Fmt<SWF>::EPL;
  d.ok = kraw < p.Is;
  const int kc = min(kraw, p.Is - Fmt<SWF>::EPL);
  d.off = kc;
  d.L = p.Is;
  d.f = 1.0f;
  d.w = static_cast<const uint8_t*>(p.sd) + (size_t(n0) * p.Is + kc) * Fmt<SWF>::ES;
  d.s = p.sds;
  d.h = p.hs + size_t(row) * p.Is + kc;
  return d;
}

// Stream this wave's chunks (c = first, first + step, ...) of one format, two
// per iteration (both loads issued before either reduction); loop bounds are
// uniform across the wave and loads are never predicated.
template <int WF, class Src>
MOE_DEV void down_stream(int first, int nchunks, int step, int n0, Src src, float (&acc)[RD]) {
  for (int c = first; c < nchunks; c += 2 * step) {
    DownStage<WF> sa, sb;
    const bool two = c + step < nchunks;
    const DownSrc da = src(c);
    const DownSrc db = two ? src(c + step) : da;
    down_load<WF>(sa, da, n0);
    if (two) down_load<WF>(sb, db, n0);
    down_math<WF>(sa, da.ok, acc);
    if (two) down_math<WF>(sb, db.ok, acc);
  }
}

}  // namespace moe
