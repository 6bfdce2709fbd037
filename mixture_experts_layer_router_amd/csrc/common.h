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
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
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

// Four fp32 -> four e4m3fn codes (byte k from the k-th argument) with the
// hardware converter: round to nearest even; the inputs are clamped to
// +-448 first, which gives the saturation of f32_to_e4m3 (the converter
// alone turns overflow into NaN).  Equal to f32_to_e4m3 for every non-NaN
// input (checked on all fp32 magnitudes below 1024 on gfx950).
MOE_DEV uint32_t e4m3x4_sat(float a, float b, float c, float d) {
  auto cl = [](float v) { return __builtin_amdgcn_fmed3f(v, -kE4M3Max, kE4M3Max); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), w, true);
  return uint32_t(w);
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
// DPP lane moves (GFX9 DPP controls): quad_perm [1,0,3,2] = 0xb1 (xor 1),
// quad_perm [2,3,0,1] = 0x4e (xor 2), row_half_mirror = 0x141 (lane i <- 7-i
// within 8), row_mirror = 0x140 (lane i <- 15-i within 16), row_bcast:15 =
// 0x142 (row r+1 <- lane 15 of row r), row_bcast:31 = 0x143 (rows 2,3 <- lane 31).
// Lanes of rows outside row_mask keep `old`.
template <int CTRL, int ROW_MASK = 0xf>
MOE_DEV float dpp_f(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, v),
                                                               CTRL, ROW_MASK, 0xf, false));
}

// reduction within each row of 16 lanes; every lane of the row gets the result
MOE_DEV float row16_sum(float v) {
  v += dpp_f<0xb1>(0.f, v);
  v += dpp_f<0x4e>(0.f, v);
  v += dpp_f<0x141>(0.f, v);
  v += dpp_f<0x140>(0.f, v);
  return v;
}
MOE_DEV float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xb1>(v, v));
  v = fmaxf(v, dpp_f<0x4e>(v, v));
  v = fmaxf(v, dpp_f<0x141>(v, v));
  v = fmaxf(v, dpp_f<0x140>(v, v));
  return v;
}
// sum / max over the whole wave, returned uniform (read from lane 63)
MOE_DEV float wave_sum(float v) {
  v = row16_sum(v);
  v += dpp_f<0x142, 0xa>(0.f, v);
  v += dpp_f<0x143, 0xc>(0.f, v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
MOE_DEV float wave_max(float v) {
  v = row16_max(v);
  v = fmaxf(v, dpp_f<0x142, 0xa>(v, v));
  v = fmaxf(v, dpp_f<0x143, 0xc>(v, v));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
// max over aligned groups of W lanes (W = 4 or 16); every lane of the group gets it
template <int W>
MOE_DEV float group_max(float v) {
  static_assert(W == 4 || W == 16, "group of 4 or 16 lanes");
  v = fmaxf(v, dpp_f<0xb1>(v, v));
  v = fmaxf(v, dpp_f<0x4e>(v, v));
  if (W == 16) {
    v = fmaxf(v, dpp_f<0x141>(v, v));
    v = fmaxf(v, dpp_f<0x140>(v, v));
  }
  return v;
}

MOE_DEV int lane_id() { return __lane_id(); }

}  // namespace moe
