// Activation quantisation of the rows entering the expert FFNs ("From 35 to
// 873 tokens/s", Rounds 12-15: MXFP8 quantisation of the expert inputs), with
// an optional row gather so dispatch and quantisation are one pass.
//
//   1x128: s = fl32(amax/448) (1 if amax = 0), q = RNE_e4m3(fl32(v/s)), fp32 scale
//   1x32 : X = 2^(floor(log2 amax) - 8), q = RNE_e4m3(v/X), e8m0 scale
//
// One wave covers 512 columns of a row (8 per lane): a 1x128 block is 16
// lanes, a 1x32 block 4 lanes, so each block's amax is a short xor-shuffle.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

template <bool IN_F32>
MOE_DEV void load8(const void* in, size_t off, float (&v)[8]) {
  if (IN_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(in) + off);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(in) + off);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(w[q] << 16);
      v[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
    }
  }
}

MOE_DEV float dec1(uint32_t code) {
  f32x2 d = e4m3x2_to_f32(code, false);
  return d.x;
}

template <bool IN_F32, int AF>
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* __restrict__ in, int rows, int H,
                                                         const int* __restrict__ row_map, int row_div,
                                                         void* __restrict__ q, void* __restrict__ qs,
                                                         float* __restrict__ deq) {
  const int nch = (H + 511) / 512;
  const long wid = long(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (wid >= long(rows) * nch) return;
  const int r = int(wid / nch), ch = int(wid % nch);
  const int lane = lane_id();
  const int c = ch * 512 + lane * 8;
  const bool active = c < H;
  const int src = row_map ? row_map[r] / row_div : r;
  float v[8] = {};
  if (active) load8<IN_F32>(in, size_t(src) * H + c, v);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));

  if (AF == A_NONE) {
    if (!active) return;
    if (deq) {
      float4* o = reinterpret_cast<float4*>(deq + size_t(r) * H + c);
      o[0] = make_float4(v[0], v[1], v[2], v[3]);
      o[1] = make_float4(v[4], v[5], v[6], v[7]);
    } else {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = uint32_t(f32_to_bf16(v[2 * i])) | (uint32_t(f32_to_bf16(v[2 * i + 1])) << 16);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(q) + size_t(r) * H + c) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    return;
  }

  float a[8];  // the values divided by the block scale, then encoded with e4m3x4_sat
  float scale;
  if (AF == A_FP8_1X128) {
    amax = group_max<16>(amax);
    scale = amax > 0.f ? __fdiv_rn(amax, kE4M3Max) : 1.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = __fdiv_rn(v[i], scale);
  } else {
    amax = group_max<4>(amax);
    const int xe = mx_exponent(amax);
    scale = __builtin_amdgcn_ldexpf(1.0f, xe);
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = __builtin_amdgcn_ldexpf(v[i], -xe);
    if (active && (lane & 3) == 0 && !deq)
      static_cast<uint8_t*>(qs)[size_t(r) * (H / 32) + c / 32] = uint8_t(xe + 127);
  }
  if (!active) return;
  const uint32_t lo = e4m3x4_sat(a[0], a[1], a[2], a[3]), hi = e4m3x4_sat(a[4], a[5], a[6], a[7]);
  if (deq) {
    float d[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) d[i] = dec1(((i < 4 ? lo : hi) >> (8 * (i & 3))) & 0xffu) * scale;
    float4* o = reinterpret_cast<float4*>(deq + size_t(r) * H + c);
    o[0] = make_float4(d[0], d[1], d[2], d[3]);
    o[1] = make_float4(d[4], d[5], d[6], d[7]);
    return;
  }
  *reinterpret_cast<uint2*>(static_cast<uint8_t*>(q) + size_t(r) * H + c) = make_uint2(lo, hi);
  if (AF == A_FP8_1X128 && (lane & 15) == 0) static_cast<float*>(qs)[size_t(r) * (H / 128) + c / 128] = scale;
}

__global__ __launch_bounds__(256) void dequant_rows_kernel(const uint8_t* __restrict__ q, const void* __restrict__ qs,
                                                          int afmt, long n, int H, float* __restrict__ out) {
  const long i = (long(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  const uint32_t w = *reinterpret_cast<const uint32_t*>(q + i);
  const long r = i / H;
  const int c = int(i % H);
  const float sc = afmt == A_FP8_1X128 ? static_cast<const float*>(qs)[r * (H / 128) + c / 128]
                                       : e8m0_to_f32(static_cast<const uint8_t*>(qs)[r * (H / 32) + c / 32]);
  const f32x2 a = e4m3x2_to_f32(w, false), b = e4m3x2_to_f32(w, true);
  *reinterpret_cast<float4*>(out + i) = make_float4(a.x * sc, a.y * sc, b.x * sc, b.y * sc);
}

__global__ void e4m3_decode_kernel(const uint8_t* codes, float* out, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = dec1(codes[i]);
}
__global__ void e4m3_encode_kernel(const float* in, uint8_t* codes, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) codes[i] = uint8_t(e4m3x4_sat(in[i], 0.f, 0.f, 0.f) & 0xffu);  // the quantisers' encoder
}

template <bool IN_F32>
hipError_t launch_q(const void* in, int rows, int H, const int* row_map, int row_div, int afmt, void* q, void* qs,
                    float* deq, hipStream_t s) {
  const long waves = long(rows) * ((H + 511) / 512);
  const dim3 grid(unsigned((waves + 3) / 4));
  switch (afmt) {
    case A_NONE:
      hipLaunchKernelGGL((quant_rows_kernel<IN_F32, A_NONE>), grid, dim3(256), 0, s, in, rows, H, row_map, row_div, q,
                         qs, deq);
      break;
    case A_FP8_1X128:
      hipLaunchKernelGGL((quant_rows_kernel<IN_F32, A_FP8_1X128>), grid, dim3(256), 0, s, in, rows, H, row_map,
                         row_div, q, qs, deq);
      break;
    default:
      hipLaunchKernelGGL((quant_rows_kernel<IN_F32, A_MXFP8_1X32>), grid, dim3(256), 0, s, in, rows, H, row_map,
                         row_div, q, qs, deq);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_rows(const void* in, bool in_f32, int rows, int H, const int* row_map, int row_div, int afmt,
                             void* q, void* qs, float* deq_out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  return in_f32 ? launch_q<true>(in, rows, H, row_map, row_div, afmt, q, qs, deq_out, s)
                : launch_q<false>(in, rows, H, row_map, row_div, afmt, q, qs, deq_out, s);
}

hipError_t launch_dequant_rows(const uint8_t* q, const void* qs, int afmt, int rows, int H, float* out, hipStream_t s) {
  const long n = long(rows) * H;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_rows_kernel, dim3(unsigned((n / 4 + 255) / 256)), dim3(256), 0, s, q, qs, afmt, n, H, out);
  return hipGetLastError();
}

hipError_t launch_e4m3_decode(const uint8_t* codes, float* out, int n, hipStream_t s) {
  hipLaunchKernelGGL(e4m3_decode_kernel, dim3((n + 255) / 256), dim3(256), 0, s, codes, out, n);
  return hipGetLastError();
}
hipError_t launch_e4m3_encode(const float* in, uint8_t* codes, int n, hipStream_t s) {
  hipLaunchKernelGGL(e4m3_encode_kernel, dim3((n + 255) / 256), dim3(256), 0, s, in, codes, n);
  return hipGetLastError();
}

}  // namespace moe
