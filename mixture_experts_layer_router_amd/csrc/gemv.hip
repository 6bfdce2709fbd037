// Small-batch expert FFN as bandwidth-bound GEMVs ("From 35 to 873
// tokens/s", Skill 5: decode is a GEMV; the BS=1 GEMM is bandwidth bound).
//
// gate/up: one wave per (slot, block of 8 intermediate rows) reads 8 gate and
// 8 up weight rows once with 16-byte lane loads (1 KB per wave per row chunk,
// fully coalesced), converts FP8 codes with the hardware e4m3 converter,
// accumulates in fp32 against the token's row, applies the per-block scale
// once per 16-element lane chunk, and writes h = SiLU(g) * u (stages P1/Q1).
//
// down: one wave per (token, block of 8 output rows) walks the concatenation
// of the token's K routed down matrices and the shared one (stages P2/Q2),
// folding each routing weight into the block scale, and writes the bf16
// output directly: the combine of stage R happens in registers, in a fixed
// order, with one rounding.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int RB = 8;  // rows per wave item

// elements per 16-byte lane load
template <int WF>
struct Epl {
  static constexpr int v = (WF == W_BF16) ? 8 : 16;
};

// partial dot of one 16-byte weight chunk with EPL x values
template <int WF>
MOE_DEV float dot_chunk(uint4 w, const float* x) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  float s0 = 0.f, s1 = 0.f;
  if (WF == W_BF16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s0 = fmaf(__uint_as_float(u[q] << 16), x[2 * q], s0);
      s1 = fmaf(__uint_as_float(u[q] & 0xffff0000u), x[2 * q + 1], s1);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x2 a = e4m3x2_to_f32(u[q], false);
      f32x2 b = e4m3x2_to_f32(u[q], true);
      s0 = fmaf(a.x, x[4 * q + 0], s0);
      s1 = fmaf(a.y, x[4 * q + 1], s1);
      s0 = fmaf(b.x, x[4 * q + 2], s0);
      s1 = fmaf(b.y, x[4 * q + 3], s1);
    }
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
MOE_DEV constexpr int esize() { return WF == W_BF16 ? 2 : 1; }

template <bool F32>
MOE_DEV void load_x(const void* x, size_t off, float* v, int n) {
  if (F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + off);
    for (int i = 0; i < n / 4; ++i) {
      float4 f = p[i];
      v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + off);
    for (int i = 0; i < n / 8; ++i) {
      uint4 u = p[i];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[8 * i + 2 * q] = __uint_as_float(w[q] << 16);
        v[8 * i + 2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
      }
    }
  }
}

// h[i0 .. i0+RB) = SiLU(x.Wg^T) * (x.Wu^T) for one x row.
template <int WF, bool XF32>
MOE_DEV void gate_up_item(const void* x, int H, int xrow, const void* g, const void* u, const void* gs,
                          const void* us, int I, int i0, float* hrow) {
  constexpr int EPL = Epl<WF>::v;
  constexpr int CW = 64 * EPL;
  const int lane = lane_id();
  float ag[RB] = {}, au[RB] = {};
  const uint8_t* gb = static_cast<const uint8_t*>(g) + size_t(i0) * H * esize<WF>();
  const uint8_t* ub = static_cast<const uint8_t*>(u) + size_t(i0) * H * esize<WF>();
  for (int k = lane * EPL; k < H; k += CW) {
    float xv[EPL];
    load_x<XF32>(x, size_t(xrow) * H + k, xv, EPL);
    uint4 wg[RB], wu[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      wg[r] = *reinterpret_cast<const uint4*>(gb + (size_t(r) * H + k) * esize<WF>());
      wu[r] = *reinterpret_cast<const uint4*>(ub + (size_t(r) * H + k) * esize<WF>());
    }
    if (WF == W_MXFP8) {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        ag[r] = fmaf(dot_chunk<WF>(wg[r], xv), wscale<WF>(gs, i0 + r, k, H), ag[r]);
        au[r] = fmaf(dot_chunk<WF>(wu[r], xv), wscale<WF>(us, i0 + r, k, H), au[r]);
      }
    } else {
      const float sg = wscale<WF>(gs, i0, k, H), su = wscale<WF>(us, i0, k, H);
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        ag[r] = fmaf(dot_chunk<WF>(wg[r], xv), sg, ag[r]);
        au[r] = fmaf(dot_chunk<WF>(wu[r], xv), su, au[r]);
      }
    }
  }
  float mine = 0.f;
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    float gv = wave_sum(ag[r]);
    float uv = wave_sum(au[r]);
    if (lane == r) mine = silu(gv) * uv;
  }
  if (lane < RB) hrow[i0 + lane] = mine;
}

MOE_DEV int seg_of(const int* seg, int E, int r) {
  int lo = 0, hi = E;  // find e with seg[e] <= r < seg[e+1]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (seg[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

template <int WF, int SWF, bool XF32, bool XSF32>
__global__ __launch_bounds__(256) void gemv_gate_up_kernel(GemvUpParams p) {
  const long wid = long(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int nslots = p.ids ? p.T * p.K : (p.seg ? p.T : 0);
  const long nr = long(nslots) * (p.I / RB);
  const long ns = p.hs ? long(p.T) * (p.Is / RB) : 0;
  if (wid < nr) {
    const int slot = int(wid / (p.I / RB)), i0 = int(wid % (p.I / RB)) * RB;
    int e, xrow;
    if (p.ids) {
      e = p.ids[slot];
      xrow = slot / p.K;
    } else {
      e = seg_of(p.seg, p.E, slot);
      xrow = slot;
    }
    const size_t wstride = size_t(p.I) * p.H * esize<WF>();
    const size_t sstride = WF == W_FP8_B128 ? size_t(p.I / 128) * (p.H / 128) * 4
                                            : (WF == W_MXFP8 ? size_t(p.I) * (p.H / 32) : 0);
    gate_up_item<WF, XF32>(p.x, p.H, xrow, static_cast<const uint8_t*>(p.g) + e * wstride,
                           static_cast<const uint8_t*>(p.u) + e * wstride,
                           p.gs ? static_cast<const uint8_t*>(p.gs) + e * sstride : nullptr,
                           p.us ? static_cast<const uint8_t*>(p.us) + e * sstride : nullptr, p.I, i0,
                           p.h + size_t(slot) * p.I);
  } else if (wid < nr + ns) {
    const long w2 = wid - nr;
    const int t = int(w2 / (p.Is / RB)), i0 = int(w2 % (p.Is / RB)) * RB;
    gate_up_item<SWF, XSF32>(p.xs, p.H, t, p.sg, p.su, p.sgs, p.sus, p.Is, i0, p.hs + size_t(t) * p.Is);
  }
}

// acc[r] += factor * sum_k W[n0+r][k] * h[k] over one [H][L] matrix
template <int WF>
MOE_DEV void down_segment(const void* W, const void* S, int L, const float* h, float factor, int n0,
                          float (&acc)[RB]) {
  constexpr int EPL = Epl<WF>::v;
  constexpr int CW = 64 * EPL;
  const int lane = lane_id();
  const uint8_t* wb = static_cast<const uint8_t*>(W) + size_t(n0) * L * esize<WF>();
  for (int k = lane * EPL; k < L; k += CW) {
    float hv[EPL];
    load_x<true>(h, k, hv, EPL);
    uint4 w[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) w[r] = *reinterpret_cast<const uint4*>(wb + (size_t(r) * L + k) * esize<WF>());
    if (WF == W_MXFP8) {
#pragma unroll
      for (int r = 0; r < RB; ++r) acc[r] = fmaf(dot_chunk<WF>(w[r], hv), factor * wscale<WF>(S, n0 + r, k, L), acc[r]);
    } else {
      const float f = factor * wscale<WF>(S, n0, k, L);
#pragma unroll
      for (int r = 0; r < RB; ++r) acc[r] = fmaf(dot_chunk<WF>(w[r], hv), f, acc[r]);
    }
  }
}

template <int WF>
MOE_DEV size_t down_wstride(int H, int L) { return size_t(H) * L * esize<WF>(); }
template <int WF>
MOE_DEV size_t down_sstride(int H, int L) {
  return WF == W_FP8_B128 ? size_t(H / 128) * (L / 128) * 4 : (WF == W_MXFP8 ? size_t(H) * (L / 32) : 0);
}

template <int WF, int SWF>
__global__ __launch_bounds__(256) void gemv_down_kernel(GemvDownParams p) {
  const long wid = long(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int nb = p.H / RB;
  const int nrows = p.out ? p.T : p.rows;
  if (wid >= long(nrows) * nb) return;
  const int row = int(wid / nb), n0 = int(wid % nb) * RB;
  const int lane = lane_id();
  float acc[RB] = {};
  if (p.out) {  // combine mode: token `row`
    for (int j = 0; j < p.K; ++j) {
      const int e = p.ids[row * p.K + j];
      down_segment<WF>(static_cast<const uint8_t*>(p.d) + e * down_wstride<WF>(p.H, p.I),
                       p.ds ? static_cast<const uint8_t*>(p.ds) + e * down_sstride<WF>(p.H, p.I) : nullptr, p.I,
                       p.h + size_t(row * p.K + j) * p.I, p.w[row * p.K + j], n0, acc);
    }
    if (p.hs) down_segment<SWF>(p.sd, p.sds, p.Is, p.hs + size_t(row) * p.Is, 1.0f, n0, acc);
    uint32_t mine = 0;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      float v = wave_sum(acc[r]);
      if (lane == r) mine = f32_to_bf16(v);
    }
    if (lane < RB) p.out[size_t(row) * p.H + n0 + lane] = uint16_t(mine);
  } else {  // per-row mode: y[row] = h[row] . Wd_e^T
    if (p.seg) {
      const int e = seg_of(p.seg, p.E, row);
      down_segment<WF>(static_cast<const uint8_t*>(p.d) + e * down_wstride<WF>(p.H, p.I),
                       p.ds ? static_cast<const uint8_t*>(p.ds) + e * down_sstride<WF>(p.H, p.I) : nullptr, p.I,
                       p.h + size_t(row) * p.I, 1.0f, n0, acc);
    } else {
      down_segment<SWF>(p.sd, p.sds, p.Is, p.hs + size_t(row) * p.Is, 1.0f, n0, acc);
    }
    float mine = 0.f;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      float v = wave_sum(acc[r]);
      if (lane == r) mine = v;
    }
    if (lane < RB) p.y[size_t(row) * p.H + n0 + lane] = mine;
  }
}

template <int WF, int SWF>
hipError_t up_dispatch_x(const GemvUpParams& p, dim3 grid, hipStream_t s) {
  if (p.x_f32 && p.xs_f32)
    hipLaunchKernelGGL((gemv_gate_up_kernel<WF, SWF, true, true>), grid, dim3(256), 0, s, p);
  else if (p.x_f32)
    hipLaunchKernelGGL((gemv_gate_up_kernel<WF, SWF, true, false>), grid, dim3(256), 0, s, p);
  else if (p.xs_f32)
    hipLaunchKernelGGL((gemv_gate_up_kernel<WF, SWF, false, true>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((gemv_gate_up_kernel<WF, SWF, false, false>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int WF>
hipError_t up_dispatch_s(const GemvUpParams& p, dim3 grid, hipStream_t s) {
  switch (p.swfmt) {
    case W_BF16: return up_dispatch_x<WF, W_BF16>(p, grid, s);
    case W_FP8_B128: return up_dispatch_x<WF, W_FP8_B128>(p, grid, s);
    default: return up_dispatch_x<WF, W_MXFP8>(p, grid, s);
  }
}

template <int WF>
hipError_t down_dispatch_s(const GemvDownParams& p, dim3 grid, hipStream_t s) {
  switch (p.swfmt) {
    case W_BF16: hipLaunchKernelGGL((gemv_down_kernel<WF, W_BF16>), grid, dim3(256), 0, s, p); break;
    case W_FP8_B128: hipLaunchKernelGGL((gemv_down_kernel<WF, W_FP8_B128>), grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((gemv_down_kernel<WF, W_MXFP8>), grid, dim3(256), 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_gate_up(const GemvUpParams& p, hipStream_t s) {
  const int nslots = p.ids ? p.T * p.K : (p.seg ? p.T : 0);
  const long items = long(nslots) * (p.I / RB) + (p.hs ? long(p.T) * (p.Is / RB) : 0);
  if (items == 0) return hipSuccess;
  const dim3 grid(unsigned((items + 3) / 4));
  switch (p.wfmt) {
    case W_BF16: return up_dispatch_s<W_BF16>(p, grid, s);
    case W_FP8_B128: return up_dispatch_s<W_FP8_B128>(p, grid, s);
    default: return up_dispatch_s<W_MXFP8>(p, grid, s);
  }
}

hipError_t launch_gemv_down(const GemvDownParams& p, hipStream_t s) {
  const int nrows = p.out ? p.T : p.rows;
  const long items = long(nrows) * (p.H / RB);
  if (items == 0) return hipSuccess;
  const dim3 grid(unsigned((items + 3) / 4));
  switch (p.wfmt) {
    case W_BF16: return down_dispatch_s<W_BF16>(p, grid, s);
    case W_FP8_B128: return down_dispatch_s<W_FP8_B128>(p, grid, s);
    default: return down_dispatch_s<W_MXFP8>(p, grid, s);
  }
}

}  // namespace moe
