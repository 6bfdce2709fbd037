// Device-side routing pieces shared by the router kernels: the small-T router
// GEMV row and the per-token group-limited greedy top-k (stage O of the
// DSV2-236B-MegaKernel README flowchart).
#pragma once
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr float kNegInfF = -INFINITY;

MOE_DEV int wave_min_i(int v) {
  auto step = [](int a, int b) { return a < b ? a : b; };
  v = step(v, __builtin_amdgcn_update_dpp(v, v, 0xb1, 0xf, 0xf, false));
  v = step(v, __builtin_amdgcn_update_dpp(v, v, 0x4e, 0xf, 0xf, false));
  v = step(v, __builtin_amdgcn_update_dpp(v, v, 0x141, 0xf, 0xf, false));
  v = step(v, __builtin_amdgcn_update_dpp(v, v, 0x140, 0xf, 0xf, false));
  v = step(v, __builtin_amdgcn_update_dpp(v, v, 0x142, 0xa, 0xf, false));
  v = step(v, __builtin_amdgcn_update_dpp(v, v, 0x143, 0xc, 0xf, false));
  return __builtin_amdgcn_readlane(v, 63);
}

// max over aligned groups of `lpg` lanes (lpg a power of two <= 64); every lane
// of a group gets the group's value
MOE_DEV float lanes_max(float v, int lpg) {
  if (lpg >= 2) v = fmaxf(v, dpp_f<0xb1>(v, v));
  if (lpg >= 4) v = fmaxf(v, dpp_f<0x4e>(v, v));
  if (lpg >= 8) v = fmaxf(v, dpp_f<0x141>(v, v));
  if (lpg >= 16) v = fmaxf(v, dpp_f<0x140>(v, v));
  if (lpg >= 32) v = fmaxf(v, __shfl_xor(v, 16, 64));
  if (lpg >= 64) v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

// Lane layout of one token's logits: groups of gsz contiguous experts, each
// group spread over lpg = 64 / next_pow2(G) lanes; lane l holds members
// (l % lpg) + lpg*j of group l / lpg, j < kMpl.  E <= 256 gives at most 8.
constexpr int kMpl = 8;
struct TopkLayout {
  int gsz, lpg, g, m0;
  MOE_DEV TopkLayout(const RouteParams& p, int lane) {
    gsz = p.E / p.G;
    int gp = 1;
    while (gp < p.G) gp <<= 1;
    lpg = 64 / gp;
    g = lane / lpg;
    m0 = lane % lpg;
  }
  // expert id of slot j, or -1
  MOE_DEV int expert(const RouteParams& p, int j) const {
    const int m = m0 + lpg * j;
    return (g < p.G && m < gsz) ? g * gsz + m : -1;
  }
};

// One wave routes one token.  lg[j]: logit (bias included) of layout slot j
// (empty slots are ignored whatever they hold).  Writes ids[0..K) and w[0..K)
// (lane 0).
//   softmax over all experts; group score = max member; top-TG groups by
//   rank (ties to the lower group); then K rounds of (largest logit among the
//   kept groups' experts, ties to the lower id).  w = scale * softmax score.
// Every id written is a member of a kept group, so it lies in [0, E), for any
// logits: -inf logits are candidates that tie (lowest ids first) below every
// finite one, and a token whose softmax is undefined (a NaN or +inf logit)
// has all its candidates tie, so it takes the lowest ids of the lowest
// groups; its weights are NaN.
// COH: agent-scope atomic stores of ids / w (read by other workgroups in the same launch).
template <bool COH = false>
MOE_DEV void topk_select(const RouteParams& p, const TopkLayout& L, float (&lg)[kMpl], int* ids, float* w) {
  const int lane = lane_id();
  unsigned live = 0;  // bit j: slot j holds an expert
  bool bad = false;   // a NaN or +inf logit
#pragma unroll
  for (int j = 0; j < kMpl; ++j)
    if (L.expert(p, j) >= 0) {
      live |= 1u << j;
      bad |= !(lg[j] == lg[j]) || lg[j] == INFINITY;
    } else {
      lg[j] = kNegInfF;
    }
  float mx = kNegInfF;
#pragma unroll
  for (int j = 0; j < kMpl; ++j) mx = fmaxf(mx, lg[j]);
  const float m = wave_max(mx);
  float se = 0.f;
#pragma unroll
  for (int j = 0; j < kMpl; ++j)
    if (lg[j] != kNegInfF) se += expf(lg[j] - m);  // NaN and +inf make s NaN
  const float s = wave_sum(se);
  // selection keys, in place of the logits: the logits, or all equal when
  // the softmax is undefined (m and s above keep what the weights need)
  const bool degenerate = __any(bad);
#pragma unroll
  for (int j = 0; j < kMpl; ++j) lg[j] = degenerate ? kNegInfF : lg[j];
  float (&key)[kMpl] = lg;
  float kmx = kNegInfF;
#pragma unroll
  for (int j = 0; j < kMpl; ++j) kmx = fmaxf(kmx, key[j]);
  const float gmax = lanes_max(kmx, L.lpg);  // this lane's group maximum
  // rank of this lane's group among the G group maxima
  int grank = 0;
  for (int q = 0; q < p.G; ++q) {
    const float o = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gmax), q * L.lpg));
    grank += (o > gmax) || (o == gmax && q < L.g);
  }
  if (!(L.g < p.G && grank < p.TG)) live = 0;
  for (int r = 0; r < p.K; ++r) {
    float best = kNegInfF;
    int bj = -1;
#pragma unroll
    for (int j = 0; j < kMpl; ++j)
      if (((live >> j) & 1u) && (bj < 0 || key[j] > best)) {  // strict: the lower slot (lower id) wins ties
        best = key[j];
        bj = j;
      }
    const float v = wave_max(best);
    const int mine = (bj >= 0 && best == v) ? L.expert(p, bj) : 0x7fffffff;
    const int e = wave_min_i(mine);  // a candidate always exists: K <= TG * E / G
    if (mine == e) live &= ~(1u << bj);
    if (lane == 0) {
      const float wr = p.scale * (expf(v - m) / s);  // s is NaN for a degenerate token
      if (COH) {
        __hip_atomic_store(ids + r, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(w + r, wr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        ids[r] = e;
        w[r] = wr;
      }
    }
  }
}

// Router logits of one expert row e for T <= kRouteGemvMaxT tokens, computed
// by one workgroup of 256 threads: all of the row's and the tokens' 16-byte
// loads are issued before any arithmetic (rows past T reload row T-1 and are
// masked, so no load sits behind a branch); partial sums meet in `part` (LDS)
// in wave order.  coherent: agent-scope atomic stores of the logits (read by
// another workgroup in the same launch).
// xl: when not null, x as bf16 pairs in LDS (token t's row at xl + t * H / 2),
// read there instead of from x.  tagged: when not null, the logits go there
// instead, as 64-bit words (tag << 32 | float bits) stored with agent-scope
// atomic stores, so a reader can tell this launch's value from an old one.
// MAXT: the most tokens the caller passes (T <= MAXT <= kRouteGemvMaxT).
template <int MAXT = kRouteGemvMaxT>
MOE_DEV void router_row(const uint16_t* __restrict__ x, int T, const uint16_t* __restrict__ wr, const RouteParams& p,
                        int e, float* __restrict__ logits, float (*part)[MAXT], bool coherent = false,
                        const uint32_t* xl = nullptr, uint64_t* tagged = nullptr, unsigned tag = 0) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint16_t* row = wr + size_t(e) * p.H;
  float acc[MAXT] = {};
  // 256 threads x 8 bf16 = 2048 columns per pass; 4 passes issued together
  if (xl) {
    for (int k0 = 0; k0 < p.H; k0 += 4 * 2048) {
      u32x4 wv[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) wv[c] = *reinterpret_cast<const u32x4*>(row + min(k0 + c * 2048 + tid * 8, p.H - 8));
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int k = min(k0 + c * 2048 + tid * 8, p.H - 8);
        const float on = k0 + c * 2048 + tid * 8 < p.H ? 1.0f : 0.0f;
#pragma unroll
        for (int t = 0; t < MAXT; ++t) {
          if (t >= T) break;  // uniform
          const u32x4 xv = *reinterpret_cast<const u32x4*>(xl + (size_t(t) * p.H + k) / 2);
          float a = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            a = fmaf(__uint_as_float(xv[q] << 16), __uint_as_float(wv[c][q] << 16), a);
            a = fmaf(__uint_as_float(xv[q] & 0xffff0000u), __uint_as_float(wv[c][q] & 0xffff0000u), a);
          }
          acc[t] = fmaf(a, on, acc[t]);
        }
      }
    }
  } else
  for (int k0 = 0; k0 < p.H; k0 += 4 * 2048) {
    u32x4 wv[4], xv[4][MAXT];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int k = min(k0 + c * 2048 + tid * 8, p.H - 8);
      wv[c] = *reinterpret_cast<const u32x4*>(row + k);
#pragma unroll
      for (int t = 0; t < MAXT; ++t)
        if (t < T || t < 4)  // rows 4 .. T-1 only when present (rows past T up to 4 reload row T-1, masked)
          xv[c][t] = *reinterpret_cast<const u32x4*>(x + size_t(min(t, T - 1)) * p.H + k);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float on = k0 + c * 2048 + tid * 8 < p.H ? 1.0f : 0.0f;
#pragma unroll
      for (int t = 0; t < MAXT; ++t) {
        if (t >= 4 && t >= T) break;  // uniform
        float a = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          a = fmaf(__uint_as_float(xv[c][t][q] << 16), __uint_as_float(wv[c][q] << 16), a);
          a = fmaf(__uint_as_float(xv[c][t][q] & 0xffff0000u), __uint_as_float(wv[c][q] & 0xffff0000u), a);
        }
        acc[t] = fmaf(a, on, acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    const float v = wave_sum(acc[t]);
    if (lane == 0) part[wave][t] = v;
  }
  __syncthreads();
  if (tid < T) {
    const float v = ((part[0][tid] + part[1][tid]) + part[2][tid]) + part[3][tid];
    if (tagged)
      __hip_atomic_store(tagged + tid * p.E + e, (uint64_t(tag) << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    else if (coherent)
      __hip_atomic_store(logits + tid * p.E + e, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      logits[tid * p.E + e] = v;
  }
}

// ------------------------------------------------------------------ stage M
// RMSNorm of one bf16 row (DSV2-236B-MegaKernel flowchart, stage M):
// r = fl32(1 / sqrt(mean(h^2) + eps)) with the mean in float64 (the squares
// of bf16 values are exact, so only the additions round), and
// x = bf16(fl32(fl32(h * gamma) * r)), each step rounded to nearest even.

MOE_DEV double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// r of one row, computed by one whole wave (every lane gets it); H % 8 == 0
MOE_DEV float row_rms_inv(const uint16_t* row, int H, float eps) {
  double acc = 0.0;
  for (int c = lane_id() * 8; c < H; c += 512) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(row + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const double lo = __uint_as_float(v[q] << 16), hi = __uint_as_float(v[q] & 0xffff0000u);
      acc = fma(lo, lo, acc);
      acc = fma(hi, hi, acc);
    }
  }
  acc = wave_sum_d(acc);
  return float(1.0 / sqrt(acc / double(H) + double(eps)));
}

// x for 8 columns (4 bf16 pairs) of h with their gamma
MOE_DEV u32x4 norm_pairs(u32x4 hv, u32x4 gv, float r) {
  u32x4 xb;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float lo = (__uint_as_float(hv[q] << 16) * __uint_as_float(gv[q] << 16)) * r;
    const float hi = (__uint_as_float(hv[q] & 0xffff0000u) * __uint_as_float(gv[q] & 0xffff0000u)) * r;
    xb[q] = uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
  }
  return xb;
}
MOE_DEV u32x4 norm_chunk(const uint16_t* row, const uint16_t* gamma, int c, float r) {
  return norm_pairs(*reinterpret_cast<const u32x4*>(row + c), *reinterpret_cast<const u32x4*>(gamma + c), r);
}

// Load one token's logits (+ bias) into the layout.  The logits may be the sum
// of nslice partial slices (stride slice_stride elements), added in order.
MOE_DEV void topk_load(const RouteParams& p, const TopkLayout& L, const float* logits_row, const float* bias,
                       float (&lg)[kMpl], int nslice = 1, long slice_stride = 0) {
#pragma unroll
  for (int j = 0; j < kMpl; ++j) {
    const int e = L.expert(p, j);
    float v = kNegInfF;
    if (e >= 0) {
      v = logits_row[e];
      for (int z = 1; z < nslice; ++z) v += logits_row[z * slice_stride + e];
      if (bias) v += bias[e];
    }
    lg[j] = v;
  }
}

}  // namespace moe
