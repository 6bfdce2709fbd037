// Router (stage N) and group-limited greedy top-k (stage O) of the
// DSV2-236B-MegaKernel README flowchart: logits = x.Wr^T (+ bias), softmax
// over all experts, the topk_groups groups with the largest max member score,
// then the topk experts of those groups, w = route_scale * score.
//
// The selection runs on fp32 logits (softmax is monotone, so the chosen ids
// are those of the scores), one wave per token: each group's experts sit on an
// aligned set of lanes so all group maxima come from one DPP reduction; groups
// are kept by rank; then K rounds pick the largest remaining logit (ties to the
// lower id), so slots come out in descending score order.  The router GEMV and
// the top-k are separate launches: the kernel boundary orders the logits
// without any device-wide fence (agent-scope fences write back and invalidate
// each XCD's L2, which costs microseconds per workgroup).
#include "route_dev.h"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void route_logits_kernel(const uint16_t* __restrict__ x, int T,
                                                           const uint16_t* __restrict__ wr, RouteParams p,
                                                           float* __restrict__ logits) {
  __shared__ float part[4][kRouteGemvMaxT];
  router_row<kRouteGemvMaxT>(x, T, wr, p, blockIdx.x, logits, part);
}

// topk_load for logits summed over nslice split-K slices: every slice value
// of the lane's experts is loaded before any is added (one memory latency, not
// one per slice), then the slices are added in slice order as topk_load does.
MOE_DEV void topk_load_sliced(const RouteParams& p, const TopkLayout& L, const float* logits_row, const float* bias,
                              float (&lg)[kMpl], int nslice, long slice_stride) {
  float s[kMpl][kRouterMaxSplit];
#pragma unroll
  for (int j = 0; j < kMpl; ++j) {
    const int e = L.expert(p, j);
#pragma unroll
    for (int z = 0; z < kRouterMaxSplit; ++z) s[j][z] = (e >= 0 && z < nslice) ? logits_row[z * slice_stride + e] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < kMpl; ++j) {
    const int e = L.expert(p, j);
    float v = kNegInfF;
    if (e >= 0) {
      v = s[j][0];
#pragma unroll
      for (int z = 1; z < kRouterMaxSplit; ++z)
        if (z < nslice) v += s[j][z];
      if (bias) v += bias[e];
    }
    lg[j] = v;
  }
}

// One wave per token over fp32 logits [T][E] (bias added here).
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T,
                                                   const float* __restrict__ bias, RouteParams p, int* ids,
                                                   float* w, int nslice, long slice_stride) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave
  const TopkLayout L(p, lane_id());
  float lg[kMpl];
  if (nslice > 1)
    topk_load_sliced(p, L, logits + size_t(t) * p.E, bias, lg, nslice, slice_stride);
  else
    topk_load(p, L, logits + size_t(t) * p.E, bias, lg);
  topk_select(p, L, lg, ids + size_t(t) * p.K, w + size_t(t) * p.K);
}

}  // namespace

hipError_t launch_route_logits(const uint16_t* x, int T, const uint16_t* wr, const RouteParams& p, float* logits,
                               hipStream_t s) {
  hipLaunchKernelGGL(route_logits_kernel, dim3(p.E), dim3(256), 0, s, x, T, wr, p, logits);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, const float* bias, const RouteParams& p, int* ids, float* w,
                       hipStream_t s, int nslice, long slice_stride) {
  hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, bias, p, ids, w,
                     nslice < 1 ? 1 : nslice, slice_stride);
  return hipGetLastError();
}

}  // namespace moe
