// Small-batch expert FFN as bandwidth-bound GEMVs ("From 35 to 873
// tokens/s", Skill 5: decode is a GEMV; the BS=1 GEMM is bandwidth bound).
//
// gate/up (stages P1/Q1): one wave per (slot, block of 4 intermediate
// columns) streams the 4 gate and 4 up weight rows with 16-byte lane loads
// (1 KB contiguous per wave per row and chunk); each chunk's 8 loads are
// issued together and many resident waves keep HBM busy.
// FP8 codes go through the hardware e4m3 converter, the products accumulate
// in fp32 against the token's row, the block scale is applied once per
// 16-element lane chunk, and the wave writes h = SiLU(g) * u.
//
// down (stages P2/Q2 and the sum of R): one workgroup per (token, block of 8
// output rows).  Its K dimension is the concatenation of the token's K routed
// down matrices and the shared one; the 4 waves take chunks of it round robin,
// fold each routing weight into the block scale, and their partial sums are
// added through LDS in wave order.  The bf16 output is written directly: the
// combine happens in registers, in a fixed order, with one rounding.
#include "gemv_dev.h"

namespace moe {

namespace {

template <int WF, int SWF, bool XF32, bool XSF32, int NR = RU, int NC = CPI>
MOE_DEV void gemv_gate_up_kernel_body(const GemvUpParams& p) {
  const long wid = long(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int nslots = p.ids ? p.T * p.K : (p.seg ? p.T : 0);
  const long nr = long(nslots) * (p.I / NR);
  const long ns = p.hs ? long(p.T) * (p.Is / NR) : 0;
  if (wid < nr) {
    const int slot = int(wid / (p.I / NR)), i0 = int(wid % (p.I / NR)) * NR;
    int e, xrow;
    if (p.ids) {
      e = p.ids[slot];
      xrow = slot / p.K;
    } else {
      e = seg_of(p.seg, p.E, slot);
      xrow = slot;
    }
    const size_t ws = wstride<WF>(p.I, p.H), ss = sstride<WF>(p.I, p.H);
    gate_up_item<WF, XF32, NR, NC>(p.x, p.H, xrow, static_cast<const uint8_t*>(p.g) + e * ws,
                           static_cast<const uint8_t*>(p.u) + e * ws,
                           p.gs ? static_cast<const uint8_t*>(p.gs) + e * ss : nullptr,
                           p.us ? static_cast<const uint8_t*>(p.us) + e * ss : nullptr, i0,
                           p.h + size_t(slot) * p.I);
  } else if (wid < nr + ns) {
    const long w2 = wid - nr;
    const int t = int(w2 / (p.Is / NR)), i0 = int(w2 % (p.Is / NR)) * NR;
    gate_up_item<SWF, XSF32, NR, NC>(p.xs, p.H, t, p.sg, p.su, p.sgs, p.sus, i0, p.hs + size_t(t) * p.Is);
  }
}

template <int WF, int SWF, bool XF32, bool XSF32>
__global__ __launch_bounds__(256) void gemv_gate_up_kernel(GemvUpParams p) {
  gemv_gate_up_kernel_body<WF, SWF, XF32, XSF32>(p);
}

template <int WF, int SWF>
__global__ __launch_bounds__(256) void gemv_down_kernel(GemvDownParams p) {
  __shared__ float part[DW][RD];
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int nb = p.H / RD;
  const int row = blockIdx.x / nb, n0 = (blockIdx.x % nb) * RD;
  float acc[RD] = {};
  const bool combine = p.out != nullptr;
  // routed part: K segments (combine) or the row's own expert (per-row mode)
  const bool routed = combine ? true : (p.seg != nullptr);
  __shared__ int sid[16];
  __shared__ float swt[16];
  const int nseg = combine ? p.K : 1;
  if (routed && threadIdx.x < nseg) {
    sid[threadIdx.x] = combine ? p.ids[row * p.K + threadIdx.x] : seg_of(p.seg, p.E, row);
    swt[threadIdx.x] = combine ? p.w[row * p.K + threadIdx.x] : 1.0f;
  }
  if (p.hs && (combine || p.seg == nullptr)) {  // the shared part needs no routing: start it first
    const int nch = (p.Is + Fmt<SWF>::CW - 1) / Fmt<SWF>::CW;
    down_stream<SWF>(wave, nch, DW, n0, [&](int c) { return shared_src<SWF>(p, row, n0, c); }, acc);
  }
  __syncthreads();
  if (routed) {
    const int nch = (nseg * p.I + Fmt<WF>::CW - 1) / Fmt<WF>::CW;
    const float inv_i = 1.0f / float(p.I);
    down_stream<WF>(wave, nch, DW, n0, [&](int c) { return routed_src<WF>(p, row, n0, c, nseg, inv_i, sid, swt); },
                    acc);
  }
#pragma unroll
  for (int r = 0; r < RD; ++r) {
    const float v = wave_sum(acc[r]);
    if (lane == r) part[wave][r] = v;
  }
  __syncthreads();
  if (threadIdx.x < RD) {
    const int r = threadIdx.x;
    float v = part[0][r];
#pragma unroll
    for (int w = 1; w < DW; ++w) v += part[w][r];
    if (combine) {
      if (p.ys_add) v += p.ys_add[size_t(row) * p.H + n0 + r];
      p.out[size_t(row) * p.H + n0 + r] = f32_to_bf16(v);
    } else {
      p.y[size_t(row) * p.H + n0 + r] = v;
    }
  }
}

// ------------------------------------------------------------------ small-T stages

// blocks [0, E): router logits of expert row blockIdx.x; the rest: shared
// gate/up items (4 per block), which do not depend on the routing.
template <int SWF, bool XSF32>
__global__ __launch_bounds__(256) void decode_stage1_kernel(DecodeParams p) {
  __shared__ float part[4][kRouteGemvMaxT];
  if (int(blockIdx.x) < p.rp.E) {
    router_row<kRouteGemvMaxT>(p.x, p.T, p.wr, p.rp, blockIdx.x, p.logits, part);
    return;
  }
  const long wid = long(blockIdx.x - p.rp.E) * 4 + (threadIdx.x >> 6);
  if (wid >= long(p.T) * (p.Is / RU)) return;
  const int t = int(wid / (p.Is / RU)), i0 = int(wid % (p.Is / RU)) * RU;
  gate_up_item<SWF, XSF32>(p.xs, p.H, t, p.sg, p.su, p.sgs, p.sus, i0, p.hs + size_t(t) * p.Is);
}

// block 0: top-k of every token (one wave each); the rest: shared down of
// (token, 8 output rows) into ysh, split over the block's 4 waves.
template <int SWF>
__global__ __launch_bounds__(256) void decode_stage2_kernel(DecodeParams p) {
  const int wave = threadIdx.x >> 6, lane = lane_id();
  if (blockIdx.x == 0) {
    const TopkLayout L(p.rp, lane);
    for (int t = wave; t < p.T; t += 4) {
      float lg[kMpl];
      topk_load(p.rp, L, p.logits + size_t(t) * p.rp.E, p.bias, lg);
      topk_select(p.rp, L, lg, p.ids + t * p.rp.K, p.w + t * p.rp.K);
    }
    return;
  }
  __shared__ float part[DW][RD];
  const int nb = p.H / RD;
  const int b = blockIdx.x - 1;
  const int row = b / nb, n0 = (b % nb) * RD;
  GemvDownParams d{};
  d.H = p.H;
  d.Is = p.Is;
  d.hs = p.hs;
  d.sd = p.sd;
  d.sds = p.sds;
  float acc[RD] = {};
  const int nch = (p.Is + Fmt<SWF>::CW - 1) / Fmt<SWF>::CW;
  down_stream<SWF>(wave, nch, DW, n0, [&](int c) { return shared_src<SWF>(d, row, n0, c); }, acc);
#pragma unroll
  for (int r = 0; r < RD; ++r) {
    const float v = wave_sum(acc[r]);
    if (lane == r) part[wave][r] = v;
  }
  __syncthreads();
  if (threadIdx.x < RD) {
    const int r = threadIdx.x;
    float v = part[0][r];
#pragma unroll
    for (int w = 1; w < DW; ++w) v += part[w][r];
    p.ysh[size_t(row) * p.H + n0 + r] = v;
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

hipError_t launch_decode_stage1(const DecodeParams& p, hipStream_t s) {
  const long items = p.Is ? long(p.T) * (p.Is / RU) : 0;
  const dim3 grid(unsigned(p.rp.E + (items + 3) / 4));
  const bool f = p.xs_f32;
  switch (p.swfmt) {
    case W_BF16:
      if (f) hipLaunchKernelGGL((decode_stage1_kernel<W_BF16, true>), grid, dim3(256), 0, s, p);
      else hipLaunchKernelGGL((decode_stage1_kernel<W_BF16, false>), grid, dim3(256), 0, s, p);
      break;
    case W_FP8_B128:
      if (f) hipLaunchKernelGGL((decode_stage1_kernel<W_FP8_B128, true>), grid, dim3(256), 0, s, p);
      else hipLaunchKernelGGL((decode_stage1_kernel<W_FP8_B128, false>), grid, dim3(256), 0, s, p);
      break;
    default:
      if (f) hipLaunchKernelGGL((decode_stage1_kernel<W_MXFP8, true>), grid, dim3(256), 0, s, p);
      else hipLaunchKernelGGL((decode_stage1_kernel<W_MXFP8, false>), grid, dim3(256), 0, s, p);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_decode_stage2(const DecodeParams& p, hipStream_t s) {
  const dim3 grid(unsigned(1 + (p.Is ? p.T * (p.H / RD) : 0)));
  switch (p.swfmt) {
    case W_BF16: hipLaunchKernelGGL((decode_stage2_kernel<W_BF16>), grid, dim3(256), 0, s, p); break;
    case W_FP8_B128: hipLaunchKernelGGL((decode_stage2_kernel<W_FP8_B128>), grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((decode_stage2_kernel<W_MXFP8>), grid, dim3(256), 0, s, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemv_gate_up(const GemvUpParams& p, hipStream_t s) {
  const int nslots = p.ids ? p.T * p.K : (p.seg ? p.T : 0);
  const long items = long(nslots) * (p.I / RU) + (p.hs ? long(p.T) * (p.Is / RU) : 0);
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
  const long blocks = long(nrows) * (p.H / RD);
  if (blocks == 0) return hipSuccess;
  switch (p.wfmt) {
    case W_BF16: return down_dispatch_s<W_BF16>(p, dim3(unsigned(blocks)), s);
    case W_FP8_B128: return down_dispatch_s<W_FP8_B128>(p, dim3(unsigned(blocks)), s);
    default: return down_dispatch_s<W_MXFP8>(p, dim3(unsigned(blocks)), s);
  }
}

}  // namespace moe
