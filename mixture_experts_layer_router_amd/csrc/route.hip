// Router (stage N) and group-limited greedy top-k (stage O) of the
// DSV2-236B-MegaKernel README flowchart: logits = x.Wr^T (+ bias), softmax
// over all experts, the topk_groups groups with the largest max member score,
// then the topk experts of those groups, w = route_scale * score.
//
// The selection runs on fp32 logits (softmax is monotone, so the chosen ids
// are those of the scores); slots are emitted in descending score order with
// ties going to the lower expert id.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr float kNegInf = -INFINITY;

// (value, index) maximum over the wave; ties go to the lower index.
MOE_DEV void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o, 64);
    int oi = __shfl_xor(i, o, 64);
    if (ov > v || (ov == v && oi < i)) {
      v = ov;
      i = oi;
    }
  }
}

// One wave routes one token.  l[i] holds the logit (bias included) of expert
// lane + 64*i, -inf past E.  Lane 0 writes ids[0..K) and w[0..K).
MOE_DEV void topk_token(float (&l)[4], const RouteParams& p, int* ids, float* w) {
  const int lane = lane_id();
  const int gsz = p.E / p.G;
  float m = fmaxf(fmaxf(l[0], l[1]), fmaxf(l[2], l[3]));
  m = wave_max(m);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (lane + 64 * i < p.E) s += expf(l[i] - m);
  s = wave_sum(s);

  // group maxima: lane g ends up holding the max logit of group g
  float gmax = kNegInf;
  for (int g = 0; g < p.G; ++g) {
    float v = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = lane + 64 * i;
      if (e < p.E && e / gsz == g) v = fmaxf(v, l[i]);
    }
    v = wave_max(v);
    if (lane == g) gmax = v;
  }
  // keep the topk_groups best groups (ties to the lower group)
  int kept = 0;
  float gv = lane < p.G ? gmax : kNegInf;
  for (int r = 0; r < p.TG; ++r) {
    float v = gv;
    int i = lane < p.G ? lane : 0x7fffffff;
    wave_argmax(v, i);
    if (lane == i) {
      kept = 1;
      gv = kNegInf;
    }
  }
  float c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int e = lane + 64 * i;
    int ge = e < p.E ? e / gsz : 0;
    int k = __shfl(kept, ge, 64);
    c[i] = (e < p.E && k) ? l[i] : kNegInf;
  }
  for (int j = 0; j < p.K; ++j) {
    float v = c[0];
    int idx = lane;
#pragma unroll
    for (int i = 1; i < 4; ++i)
      if (c[i] > v) {
        v = c[i];
        idx = lane + 64 * i;
      }
    wave_argmax(v, idx);
    if (lane == (idx & 63)) c[idx >> 6] = kNegInf;
    if (lane == 0) {
      ids[j] = idx;
      w[j] = p.scale * (expf(v - m) / s);
    }
  }
}

MOE_DEV void load_logits(const float* row, const float* bias, int E, float (&l)[4]) {
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int e = lane + 64 * i;
    float v = kNegInf;
    if (e < E) {
      v = __hip_atomic_load(row + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (bias) v += bias[e];
    }
    l[i] = v;
  }
}

__global__ __launch_bounds__(256) void route_gemv_topk_kernel(const uint16_t* __restrict__ x, int T,
                                                              const uint16_t* __restrict__ wr,
                                                              const float* __restrict__ bias, RouteParams p,
                                                              float* logits, unsigned* counter, int* ids,
                                                              float* w) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nw = gridDim.x * 4;
  for (int e = blockIdx.x * 4 + wave; e < p.E; e += nw) {
    const uint16_t* row = wr + size_t(e) * p.H;
    float acc[kRouteGemvMaxT] = {};
#pragma unroll 2
    for (int k = lane * 8; k < p.H; k += 512) {
      uint4 wv = *reinterpret_cast<const uint4*>(row + k);
      float wf[8];
      const uint32_t wu[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        wf[2 * q] = __uint_as_float(wu[q] << 16);
        wf[2 * q + 1] = __uint_as_float(wu[q] & 0xffff0000u);
      }
#pragma unroll
      for (int t = 0; t < kRouteGemvMaxT; ++t) {
        if (t < T) {
          uint4 xv = *reinterpret_cast<const uint4*>(x + size_t(t) * p.H + k);
          const uint32_t xu[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[t] = fmaf(__uint_as_float(xu[q] << 16), wf[2 * q], acc[t]);
            acc[t] = fmaf(__uint_as_float(xu[q] & 0xffff0000u), wf[2 * q + 1], acc[t]);
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kRouteGemvMaxT; ++t) {
      if (t < T) {
        float v = wave_sum(acc[t]);
        if (lane == 0) __hip_atomic_store(logits + t * p.E + e, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  // the last workgroup to finish routes every token
  __shared__ unsigned is_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    is_last = (old == gridDim.x - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  for (int t = wave; t < T; t += 4) {
    float l[4];
    load_logits(logits + t * p.E, bias, p.E, l);
    topk_token(l, p, ids + t * p.K, w + t * p.K);
  }
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T,
                                                   const float* __restrict__ bias, RouteParams p, int* ids,
                                                   float* w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float l[4];
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int e = lane + 64 * i;
    float v = kNegInf;
    if (e < p.E) {
      v = logits[size_t(t) * p.E + e];
      if (bias) v += bias[e];
    }
    l[i] = v;
  }
  topk_token(l, p, ids + size_t(t) * p.K, w + size_t(t) * p.K);
}

}  // namespace

hipError_t launch_route_gemv_topk(const uint16_t* x, int T, const uint16_t* wr, const float* bias,
                                  const RouteParams& p, float* logits_ws, unsigned* counter_ws, int* ids,
                                  float* w, hipStream_t s) {
  int blocks = (p.E + 3) / 4;
  hipLaunchKernelGGL(route_gemv_topk_kernel, dim3(blocks), dim3(256), 0, s, x, T, wr, bias, p, logits_ws,
                     counter_ws, ids, w);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, const float* bias, const RouteParams& p, int* ids, float* w,
                       hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, bias, p, ids, w);
  return hipGetLastError();
}

}  // namespace moe
