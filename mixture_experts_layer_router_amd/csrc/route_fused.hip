// Batched routing in one launch: stage M (the post-attention RMSNorm, when a
// norm weight is given), stage N (router) and stage O (group-limited top-k)
// of the DSV2-236B-MegaKernel README flowchart, plus the expert input in the
// layout the experts read ("From 35 to 873 tokens/s", Rounds 12-15: the
// router emits the layout the experts need, and the expert inputs are
// quantised there) and the per-block expert counts the stable scatter of the
// dispatch needs (Mixture-of-Kittens, Figure 1: dispatch scheduling on the
// GPU).  Only the scatter itself is a second launch (permute.hip).
//
// One workgroup of 8 waves per 16 tokens:
//   pass 1 (norm only): each wave sums h^2 over 2 rows in float64 (the squares
//     of bf16 values are exact, so only the additions round), and
//     r = fl32(1 / sqrt(mean + eps)) per row;
//   pass 2: the 8 waves take the 128-column blocks of the rows round robin.
//     For MFMA step s of a block, lane l holds row l % 16, columns
//     32 s + 8 (l / 16) + [0, 8), the 8 K values v_mfma_f32_16x16x32_bf16
//     expects, so the 4 lanes of a row load 64 contiguous bytes; the B
//     operand (16 router rows per expert block) is read straight from global
//     memory the same way.  x = bf16(fl32(fl32(h * gamma) * r)) (or x = h
//     without a norm) is formed per lane, may be written out as bf16 for the
//     FFNs that read it unquantised, and goes through a per-wave LDS tile
//     (16 rows x 128 columns) so that each lane then holds 32 consecutive
//     columns of one row: a 1x32 quantisation block is one lane's values, a
//     1x128 block the 4 adjacent lanes' (the same arithmetic as quant.hip);
//   the 8 waves' partial logits meet in LDS and are added in wave order by
//   all threads, each wave routes 2 tokens (topk_select), and LDS counters
//   give the workgroup's slots per expert (hist row = this block).
// Router rows are re-read by every workgroup (from L2): one workgroup per
// 16 tokens keeps the rows each workgroup streams (router + its tokens' h)
// small next to the per-CU load rate and fills the chip from 4,096 tokens.
// Below that, each block of 16 tokens is split over `slices` workgroups along
// H (contiguous ranges of 128-column blocks, each quantising its own
// columns); they hand their partial logits over through memory, and the
// workgroup that completes the block's counter adds them in slice order and
// routes the block, so the result does not depend on which finishes last.
#include "route_dev.h"

namespace moe {

namespace {

constexpr int kTB = 16;  // tokens per workgroup
constexpr int kWv = 8;   // waves per workgroup

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));

template <int EB, bool NORM, int AF>
__global__ __launch_bounds__(kWv * 64) void route_fused_kernel(RouteFusedParams p) {
  // per wave: its x tile (16 rows x 128 bf16) during the K loop, then its
  // partial logits [16][EB * 16] (a wave is done with its tile when it writes them)
  constexpr int kWR = kTB * EB * 16 > kTB * 64 ? kTB * EB * 16 : kTB * 64;
  __shared__ __attribute__((aligned(16))) float wbuf[kWv * kWR];
  auto red = [&](int w, int tl, int e) -> float& { return wbuf[w * kWR + tl * (EB * 16) + e]; };
  uint32_t* const sxt = reinterpret_cast<uint32_t*>(wbuf + (threadIdx.x >> 6) * kWR);  // this wave's [16][64]
  __shared__ float sr[kTB];
  __shared__ int sids[kTB * 16];
  __shared__ float sw[kTB * 16];
  __shared__ float sbias[EB * 16];
  __shared__ int scnt[EB * 16];
  __shared__ int s_last;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int S = p.slices, blk = blockIdx.x / S, z = blockIdx.x % S;  // token block, H slice
  const int t0 = blk * kTB;
  const int T = p.T, H = p.H, E = p.rp.E, K = p.rp.K;
  for (int e = tid; e < EB * 16; e += kWv * 64) {
    sbias[e] = (p.bias && e < E) ? p.bias[e] : 0.f;
    scnt[e] = 0;
  }

  // ---- pass 1: r per row (stage M)
  if constexpr (NORM) {
#pragma unroll 1
    for (int i = 0; i < kTB / kWv; ++i) {
      const int tl = wave * (kTB / kWv) + i, t = t0 + tl;
      const float r = t < T ? row_rms_inv(p.h + size_t(t) * H, H, p.eps) : 0.f;  // t uniform across the wave
      if (lane == 0) sr[tl] = r;
    }
    __syncthreads();
  }

  // ---- pass 2: x, router partial products, quantised x
  const int row = lane & 15, g = lane >> 4;
  const int t = t0 + row;
  const bool tv = t < T;
  const uint16_t* hrow = p.h + size_t(tv ? t : t0) * H;  // rows past T read row t0 (never stored)
  const float r = NORM ? sr[row] : 1.0f;
  f32x4 acc[EB];
#pragma unroll
  for (int j = 0; j < EB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint16_t* wrow[EB];
#pragma unroll
  for (int j = 0; j < EB; ++j) wrow[j] = p.wr + size_t(min(16 * j + row, E - 1)) * H;  // B column = expert
  const int nb = H / 128;
  const int blo = int(long(nb) * z / S), bhi = int(long(nb) * (z + 1) / S);  // this slice's column blocks
  // every load of a 128-column block (of half a block when there are many
  // expert blocks) is issued before any of its MFMAs, and with at most 2
  // expert blocks the next block's loads go out before this one's MFMAs too
  // (two register sets), so a wave always has a block in flight
  constexpr int NS = EB > 12 ? 1 : (EB > 10 ? 2 : 4);  // MFMA steps whose loads are held at once
  struct Blk {
    u32x4 h[NS], g[NORM ? NS : 1], w[NS][EB];
  };
  auto load_blk = [&](Blk& B, int b, int s0) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int k = b * 128 + (s0 + s) * 32 + g * 8;
      B.h[s] = *reinterpret_cast<const u32x4*>(hrow + k);
      if constexpr (NORM) B.g[s] = *reinterpret_cast<const u32x4*>(p.gamma + k);
#pragma unroll
      for (int j = 0; j < EB; ++j) B.w[s][j] = *reinterpret_cast<const u32x4*>(wrow[j] + k);
    }
  };
  auto mfma_blk = [&](const Blk& B, int b, int s0) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int k = b * 128 + (s0 + s) * 32 + g * 8;
      u32x4 xb = B.h[s];
      if constexpr (NORM) xb = norm_pairs(B.h[s], B.g[s], r);
      if constexpr (AF != A_NONE) *reinterpret_cast<u32x4*>(sxt + row * 64 + (s0 + s) * 16 + g * 4) = xb;
      const bf16x8_v a = __builtin_bit_cast(bf16x8_v, xb);
#pragma unroll
      for (int j = 0; j < EB; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_v, B.w[s][j]), acc[j], 0, 0, 0);
      if (p.x_out && tv) *reinterpret_cast<u32x4*>(p.x_out + size_t(t) * H + k) = xb;
    }
  };
  // the wave's tile back as 32 consecutive columns of one row per lane:
  // lane l reads row l / 4, columns 32 (l % 4) + [0, 32)
  auto quant_blk = [&](int b) {
    if constexpr (AF == A_NONE) return;
    const int qr = lane >> 2, qs = lane & 3, qt = t0 + qr;
    const bool qv = qt < T;
    float xv[4][8];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(sxt + qr * 64 + qs * 16 + s * 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xv[s][2 * q] = __uint_as_float(v[q] << 16);
        xv[s][2 * q + 1] = __uint_as_float(v[q] & 0xffff0000u);
      }
    }
    if constexpr (AF == A_FP8_1X128) {
      if (p.xq) {
        float amax = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(xv[s][i]));
        amax = group_max<4>(amax);  // the row's 4 adjacent lanes hold its 128 columns
        const float scale = amax > 0.f ? __fdiv_rn(amax, kE4M3Max) : 1.0f;
        if (qv) {
          uint32_t c[8];
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            float a[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) a[i] = __fdiv_rn(xv[s][i], scale);
            c[2 * s] = e4m3x4_sat(a[0], a[1], a[2], a[3]);
            c[2 * s + 1] = e4m3x4_sat(a[4], a[5], a[6], a[7]);
          }
          uint8_t* dst = static_cast<uint8_t*>(p.xq) + size_t(qt) * H + b * 128 + qs * 32;
          *reinterpret_cast<u32x4*>(dst) = u32x4{c[0], c[1], c[2], c[3]};
          *reinterpret_cast<u32x4*>(dst + 16) = u32x4{c[4], c[5], c[6], c[7]};
          if (qs == 0) static_cast<float*>(p.xqs)[size_t(qt) * (H / 128) + b] = scale;
        }
      }
    } else if constexpr (AF == A_MXFP8_1X32) {
      if (p.xq && qv) {  // this lane's 32 columns are one block
        float amax = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(xv[s][i]));
        const int xe = mx_exponent(amax);
        uint32_t c[8];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          float a[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) a[i] = __builtin_amdgcn_ldexpf(xv[s][i], -xe);
          c[2 * s] = e4m3x4_sat(a[0], a[1], a[2], a[3]);
          c[2 * s + 1] = e4m3x4_sat(a[4], a[5], a[6], a[7]);
        }
        uint8_t* dst = static_cast<uint8_t*>(p.xq) + size_t(qt) * H + b * 128 + qs * 32;
        *reinterpret_cast<u32x4*>(dst) = u32x4{c[0], c[1], c[2], c[3]};
        *reinterpret_cast<u32x4*>(dst + 16) = u32x4{c[4], c[5], c[6], c[7]};
        static_cast<uint8_t*>(p.xqs)[size_t(qt) * (H / 32) + b * 4 + qs] = uint8_t(xe + 127);
      }
    }
  };
  if constexpr (EB <= 2) {  // two register sets: block b + kWv loads while block b computes
    Blk A, B;
    int b = blo + wave;
    if (b < bhi) load_blk(A, b, 0);
    for (; b < bhi; b += 2 * kWv) {
      if (b + kWv < bhi) load_blk(B, b + kWv, 0);
      mfma_blk(A, b, 0);
      quant_blk(b);
      if (b + kWv >= bhi) break;
      if (b + 2 * kWv < bhi) load_blk(A, b + 2 * kWv, 0);
      mfma_blk(B, b + kWv, 0);
      quant_blk(b + kWv);
    }
  } else {
    for (int b = blo + wave; b < bhi; b += kWv) {
      Blk A;
#pragma unroll
      for (int s0 = 0; s0 < 4; s0 += NS) {
        load_blk(A, b, s0);
        mfma_blk(A, b, s0);
      }
      quant_blk(b);
    }
  }
  // lane l holds rows 4g + i, column (expert) l % 16 of each 16x16 block
#pragma unroll
  for (int j = 0; j < EB; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) red(wave, 4 * g + i, 16 * j + row) = acc[j][i];
  __syncthreads();

  // ---- logits: the 8 waves' parts added in wave order, by all threads, into red[0]
  for (int i = tid; i < kTB * EB * 16; i += kWv * 64) {
    const int tl = i / (EB * 16), e = i % (EB * 16);
    float v = red(0, tl, e);
#pragma unroll
    for (int w = 1; w < kWv; ++w) v += red(w, tl, e);
    red(0, tl, e) = S > 1 ? v : v + sbias[e];
  }
  __syncthreads();
  if (S > 1) {
    // hand the slice's partial logits over: agent-scope stores, complete
    // before the block's counter is incremented; the workgroup that brings it
    // to S adds the S parts in slice order (its own from LDS, the others with
    // agent-scope loads) and routes the block
    float* mine = p.part + (size_t(blk) * S + z) * kTB * E;
    for (int i = tid; i < kTB * E; i += kWv * 64)
      __hip_atomic_store(mine + i, red(0, i / E, i % E), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(p.ctr + blk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == unsigned(S - 1);
    __syncthreads();
    if (!s_last) return;
    for (int i = tid; i < kTB * E; i += kWv * 64) {
      const int tl = i / E, e = i % E;
      float v = 0.f;
      for (int zz = 0; zz < S; ++zz)
        v += zz == z ? red(0, tl, e)
                     : __hip_atomic_load(p.part + (size_t(blk) * S + zz) * kTB * E + i, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
      red(0, tl, e) = v + sbias[e];
    }
    if (tid == 0) __hip_atomic_store(p.ctr + blk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
  }
  // ---- top-k: wave w routes rows 2w, 2w+1
  const TopkLayout L(p.rp, lane);
#pragma unroll 1
  for (int i = 0; i < kTB / kWv; ++i) {
    const int tl = wave * (kTB / kWv) + i, tt = t0 + tl;
    if (tt >= T) break;  // uniform
    float lg[kMpl];
#pragma unroll
    for (int j = 0; j < kMpl; ++j) {
      const int e = L.expert(p.rp, j);
      lg[j] = e >= 0 ? red(0, tl, e) : kNegInfF;
    }
    topk_select(p.rp, L, lg, sids + tl * 16, sw + tl * 16);  // lane 0 writes LDS
    if (lane < K) {
      const int e = sids[tl * 16 + lane];
      p.ids[size_t(tt) * K + lane] = e;
      p.w[size_t(tt) * K + lane] = sw[tl * 16 + lane];
      if (p.hist) atomicAdd(&scnt[e], 1);
    }
  }
  if (!p.hist) return;
  __syncthreads();
  for (int e = tid; e < E; e += kWv * 64) p.hist[size_t(blk) * E + e] = scnt[e];
}

// Stage M alone (the paths whose router does not stage x itself): one wave
// per row, x = bf16(fl32(fl32(h * gamma) * r)) with r as above.
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const uint16_t* __restrict__ h,
                                                           const uint16_t* __restrict__ gamma, float eps, int T, int H,
                                                           uint16_t* __restrict__ x) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = lane_id();
  if (t >= T) return;  // whole wave
  const uint16_t* row = h + size_t(t) * H;
  const float r = row_rms_inv(row, H, eps);
  for (int c = lane * 8; c < H; c += 512)
    *reinterpret_cast<u32x4*>(x + size_t(t) * H + c) = norm_chunk(row, gamma, c, r);
}

template <int EB>
hipError_t launch_eb(const RouteFusedParams& p, hipStream_t s) {
  const dim3 grid(unsigned((p.T + kTB - 1) / kTB * p.slices));
  const bool norm = p.gamma != nullptr;
  const int af = p.xq ? p.afmt : A_NONE;
#define MOE_RF(NORM, AF) hipLaunchKernelGGL((route_fused_kernel<EB, NORM, AF>), grid, dim3(kWv * 64), 0, s, p)
  if (norm) {
    if (af == A_FP8_1X128) MOE_RF(true, A_FP8_1X128);
    else if (af == A_MXFP8_1X32) MOE_RF(true, A_MXFP8_1X32);
    else MOE_RF(true, A_NONE);
  } else {
    if (af == A_FP8_1X128) MOE_RF(false, A_FP8_1X128);
    else if (af == A_MXFP8_1X32) MOE_RF(false, A_MXFP8_1X32);
    else MOE_RF(false, A_NONE);
  }
#undef MOE_RF
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm_rows(const uint16_t* h, const uint16_t* gamma, float eps, int T, int H, uint16_t* x,
                               hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (H % 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rmsnorm_rows_kernel, dim3((T + 3) / 4), dim3(256), 0, s, h, gamma, eps, T, H, x);
  return hipGetLastError();
}

hipError_t launch_route_fused(const RouteFusedParams& p, hipStream_t s) {
  if (p.T <= 0) return hipSuccess;
  if (p.H % 128 || p.rp.E > 256 || p.rp.K > 16 || p.slices < 1) return hipErrorInvalidValue;
  if (p.slices > 1 && (!p.part || !p.ctr || (p.T + kTB - 1) / kTB > kRouteCtrMax)) return hipErrorInvalidValue;
  switch ((p.rp.E + 15) / 16) {
    case 1: return launch_eb<1>(p, s);
    case 2: return launch_eb<2>(p, s);
    case 3: return launch_eb<3>(p, s);
    case 4: return launch_eb<4>(p, s);
    case 5: return launch_eb<5>(p, s);
    case 6: return launch_eb<6>(p, s);
    case 7: return launch_eb<7>(p, s);
    case 8: return launch_eb<8>(p, s);
    case 9: return launch_eb<9>(p, s);
    case 10: return launch_eb<10>(p, s);
    case 11: return launch_eb<11>(p, s);
    case 12: return launch_eb<12>(p, s);
    case 13: return launch_eb<13>(p, s);
    case 14: return launch_eb<14>(p, s);
    case 15: return launch_eb<15>(p, s);
    default: return launch_eb<16>(p, s);
  }
}

}  // namespace moe
