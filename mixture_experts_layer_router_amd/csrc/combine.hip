// Weighted combine plus shared-expert add (stage R's sum in the
// DSV2-236B-MegaKernel README flowchart; "From 35 to 873 tokens/s",
// Rounds 12-15: expert-weighted reduction and shared-expert add in one
// kernel).  Deterministic: each output element sums its K routed rows in slot
// order, then adds the shared row, in fp32, and rounds to bf16 once.  No float
// atomics, so the result does not depend on arrival order.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

template <bool YBF>
MOE_DEV void load4(const void* p, size_t off, float (&v)[4]) {
  if (YBF) {
    uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + off);
    v[0] = __uint_as_float(u.x << 16);
    v[1] = __uint_as_float(u.x & 0xffff0000u);
    v[2] = __uint_as_float(u.y << 16);
    v[3] = __uint_as_float(u.y & 0xffff0000u);
  } else {
    float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + off);
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  }
}

// grid: (ceil(H / 1024), T); each thread owns 4 consecutive columns.
template <bool YBF, bool SBF>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y_perm, const int* __restrict__ inv_pos,
                                                      const float* __restrict__ w, const void* __restrict__ ys, int T,
                                                      int K, int H, uint16_t* __restrict__ out) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= H) return;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < K; ++j) {
    const int pos = inv_pos[t * K + j];
    if (pos < 0) continue;
    const float wj = w[t * K + j];
    float v[4];
    load4<YBF>(y_perm, size_t(pos) * H + c, v);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(wj, v[i], acc[i]);
  }
  if (ys) {
    float v[4];
    load4<SBF>(ys, size_t(t) * H + c, v);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += v[i];
  }
  uint2 o;
  o.x = uint32_t(f32_to_bf16(acc[0])) | (uint32_t(f32_to_bf16(acc[1])) << 16);
  o.y = uint32_t(f32_to_bf16(acc[2])) | (uint32_t(f32_to_bf16(acc[3])) << 16);
  *reinterpret_cast<uint2*>(out + size_t(t) * H + c) = o;
}

// The batched layer's combine (bf16 Y_perm and shared rows, K <= kCombWideK,
// H a multiple of 8): one workgroup per token, each thread 8 consecutive
// columns with 16-byte loads, every slot's row load issued before any
// arithmetic; the same sum order as combine_kernel (slots in order from 0,
// then the shared row, one rounding).
constexpr int kCombWideK = 8;
__global__ __launch_bounds__(1024) void combine_wide_kernel(const uint16_t* __restrict__ y_perm,
                                                            const int* __restrict__ inv_pos, const float* __restrict__ w,
                                                            const uint16_t* __restrict__ ys, int K, int H,
                                                            uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  const int c = threadIdx.x * 8;
  if (c >= H) return;
  uint4 v[kCombWideK];
  int pos[kCombWideK];
#pragma unroll
  for (int j = 0; j < kCombWideK; ++j) {
    pos[j] = j < K ? inv_pos[t * K + j] : -1;
    if (pos[j] >= 0) v[j] = *reinterpret_cast<const uint4*>(y_perm + size_t(pos[j]) * H + c);
  }
  uint4 s{0u, 0u, 0u, 0u};
  if (ys) s = *reinterpret_cast<const uint4*>(ys + size_t(t) * H + c);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kCombWideK; ++j) {
    if (pos[j] < 0) continue;
    const float wj = w[t * K + j];
    const uint32_t q[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = fmaf(wj, __uint_as_float(q[i] << 16), acc[2 * i]);
      acc[2 * i + 1] = fmaf(wj, __uint_as_float(q[i] & 0xffff0000u), acc[2 * i + 1]);
    }
  }
  const uint32_t sq[4] = {s.x, s.y, s.z, s.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = ys ? acc[2 * i] + __uint_as_float(sq[i] << 16) : acc[2 * i];
    const float hi = ys ? acc[2 * i + 1] + __uint_as_float(sq[i] & 0xffff0000u) : acc[2 * i + 1];
    o[i] = uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
  }
  *reinterpret_cast<uint4*>(out + size_t(t) * H + c) = uint4{o[0], o[1], o[2], o[3]};
}

}  // namespace

hipError_t launch_combine(const void* y_perm, bool y_bf16, const int* inv_pos, const float* w, const void* y_shared,
                          bool ys_bf16, int T, int K, int H, uint16_t* out, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (y_bf16 && (ys_bf16 || !y_shared) && K <= kCombWideK && H % 8 == 0 && H / 8 <= 1024) {
    hipLaunchKernelGGL(combine_wide_kernel, dim3(T), dim3((H / 8 + 63) / 64 * 64), 0, s,
                       static_cast<const uint16_t*>(y_perm), inv_pos, w, static_cast<const uint16_t*>(y_shared), K,
                       H, out);
    return hipGetLastError();
  }
  const dim3 grid((H + 1023) / 1024, T);
  if (y_bf16 && ys_bf16)
    hipLaunchKernelGGL((combine_kernel<true, true>), grid, dim3(256), 0, s, y_perm, inv_pos, w, y_shared, T, K, H, out);
  else if (y_bf16)
    hipLaunchKernelGGL((combine_kernel<true, false>), grid, dim3(256), 0, s, y_perm, inv_pos, w, y_shared, T, K, H, out);
  else if (ys_bf16)
    hipLaunchKernelGGL((combine_kernel<false, true>), grid, dim3(256), 0, s, y_perm, inv_pos, w, y_shared, T, K, H, out);
  else
    hipLaunchKernelGGL((combine_kernel<false, false>), grid, dim3(256), 0, s, y_perm, inv_pos, w, y_shared, T, K, H, out);
  return hipGetLastError();
}

}  // namespace moe
