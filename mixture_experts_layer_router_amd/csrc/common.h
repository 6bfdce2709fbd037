// Device helpers shared by the gfx950 kernels: bf16 / e4m3fn / e8m0
// conversions and wave64 reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_DEV __device__ __forceinline__

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

namespace moe {

constexpr float kE4M3Max = 448.0f;

// ---------------------------------------------------------------- bf16
MOE_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// round to nearest even; NaN stays NaN
MOE_DEV uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// ---------------------------------------------------------------- e4m3fn
// Decode two codes (bytes `hi`*2, `hi`*2+1 of w) with the hardware converter.
// gfx950 converts OCP e4m3fn exactly (every code is an fp32 value).
MOE_DEV f32x2 e4m3x2_to_f32(uint32_t w, bool hi) {
  return hi ? __builtin_amdgcn_cvt_pk_f32_fp8(int(w), true) : __builtin_amdgcn_cvt_pk_f32_fp8(int(w), false);
}

// fp32 -> e4m3fn code: round to nearest, ties to even, saturating at +-448.
// Subnormal range (|v| < 2^-6) is quantised in steps of 2^-9.
MOE_DEV uint32_t f32_to_e4m3(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 24) & 0x80u;
  float a = fminf(fabsf(v), kE4M3Max);
  uint32_t au = __float_as_uint(a);
  int e = int(au >> 23) - 127;
  uint32_t code;
  if (e < -6) {
    code = uint32_t(__builtin_rintf(a * 512.0f));  // 0..8 (8 = smallest normal)
  } else {
    uint32_t mant = au & 0x7fffffu;
    uint32_t keep = mant >> 20, rest = mant & 0xfffffu;
    if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) keep++;
    code = (uint32_t(e + 7) << 3) + keep;  // a carry of keep moves into the exponent
    code = code > 0x7eu ? 0x7eu : code;
  }
  return code | sign;
}

// ---------------------------------------------------------------- e8m0
MOE_DEV float e8m0_to_f32(uint32_t c) { return __builtin_amdgcn_ldexpf(1.0f, int(c) - 127); }

// e8m0 exponent of an MX block from its amax: floor(log2 amax) - 8, clamped to
// [-127, 127]; 0 when amax == 0.  fp32 subnormals give an exponent field of 0,
// which already clamps to -127.
MOE_DEV int mx_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  int e = int(__float_as_uint(amax) >> 23) - 127 - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// ---------------------------------------------------------------- SiLU
MOE_DEV float silu(float g) { return g / (1.0f + __expf(-g)); }

// ---------------------------------------------------------------- wave64 reductions
MOE_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
MOE_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
// max over aligned groups of `w` lanes (w a power of two <= 64)
template <int W>
MOE_DEV float group_max(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

MOE_DEV int lane_id() { return __lane_id(); }

}  // namespace moe
