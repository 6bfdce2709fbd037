// Grouped GEMM on gfx950 matrix cores for the batched expert FFNs (stages
// P1/P2 and Q1/Q2 of the DSV2-236B-MegaKernel README flowchart at T > 1).
//
//   C[r][n] = sum_k A[r][k] * B_e[n][k]   for the rows r of expert e's segment
//
// Weight formats and the matrix-core instruction each uses:
//   bf16      v_mfma_f32_16x16x32_bf16
//   FP8_B128  v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales; one
//             instruction covers exactly one 128-deep K block, and its fp32
//             result is promoted into the accumulator with the block's
//             activation scale (per row) times weight scale (per 128 rows)
//   MXFP8     v_mfma_scale_f32_16x16x128_f8f6f4 with the e8m0 scales of A and
//             B passed per lane (lane l scales row l%16, K block l/16)
//
// Tile: 64 rows x 256 columns x 128 bytes of K per step, 4 waves each owning
// 16 rows x 256 columns.  Tiles of one step are staged in LDS with an XOR
// swizzle of the 16-byte chunks (chunk c of row r sits at c ^ (r & 7)), double
// buffered, with the next step's global loads in flight during the MFMAs.
// Rows come from a device tile list written by the dispatch kernel, so no
// expert count is read back to the host (Mixture-of-Kittens, Abstract).
//
// EPI_GATEUP: the B tile holds 128 gate rows and the 128 up rows of the same
// intermediate columns, so every lane owns g and u of the same (row, column)
// and the epilogue writes h = SiLU(g) * u directly, optionally quantised to
// e4m3 per 1x128 or 1x32 block ("From 35 to 873 tokens/s", Rounds 12-15: the
// following quantisation emitted by the producing kernel's epilogue).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int BM = kGemmBM;  // 64
constexpr int BN = 256;
constexpr int BKB = 128;     // bytes of K per step
constexpr int kLdsA = BM * BKB;
constexpr int kLdsB = BN * BKB;

template <int WF>
MOE_DEV constexpr int esz() { return WF == W_BF16 ? 2 : 1; }

MOE_DEV int swz(int row, int c) { return row * BKB + ((c ^ (row & 7)) << 4); }

template <int WF, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][kLdsA];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][kLdsB];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int tile = blockIdx.x;
  int e, m0;
  if (p.tiles) {
    if (tile >= p.ntiles[0]) return;
    e = p.tiles[2 * tile];
    m0 = p.tiles[2 * tile + 1];
  } else {
    e = 0;
    m0 = tile * BM;
    if (m0 >= p.M) return;
  }
  // segment bounds clamped to [0, M] so malformed offsets cannot address outside the rows
  const int seg0 = p.seg ? min(max(p.seg[e], 0), p.M) : 0;
  const int seg1 = p.seg ? min(max(p.seg[e + 1], seg0), p.M) : p.M;
  const int mrows = min(BM, seg1 - seg0 - m0);
  if (mrows <= 0) return;
  const int n0 = blockIdx.y * (EPI == EPI_GATEUP ? BN / 2 : BN);
  const int K = p.K;
  const int KE = BKB / esz<WF>();  // elements per step
  const int nk = K / KE;
  const size_t lda_b = size_t(p.lda) * esz<WF>();
  const size_t ldb_b = size_t(K) * esz<WF>();

#define PHYS_ROW(rl) (p.a_map ? p.a_map[seg0 + m0 + min((rl), mrows - 1)] / p.a_div : seg0 + m0 + min((rl), mrows - 1))
  const uint8_t* b0 = static_cast<const uint8_t*>(p.B0) + size_t(e) * p.b_stride * esz<WF>();
  const uint8_t* b1 = p.B1 ? static_cast<const uint8_t*>(p.B1) + size_t(e) * p.b_stride * esz<WF>() : nullptr;

  // this thread's global->LDS chunks: A 2, B 8
  const uint8_t* ga[2];
  int la[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + 256 * i, r = q >> 3, c = q & 7;
    ga[i] = static_cast<const uint8_t*>(p.A) + size_t(PHYS_ROW(r)) * lda_b + c * 16;
    la[i] = swz(r, c);
  }
  const uint8_t* gb[8];
  int lb[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = tid + 256 * i, r = q >> 3, c = q & 7;
    const uint8_t* rp;
    if (EPI == EPI_GATEUP)
      rp = r < BN / 2 ? b0 + size_t(n0 + r) * ldb_b : b1 + size_t(n0 + r - BN / 2) * ldb_b;
    else
      rp = b0 + size_t(min(n0 + r, p.N - 1)) * ldb_b;
    gb[i] = rp + c * 16;
    lb[i] = swz(r, c);
  }

  // scales
  const int arow_mfma = wave * 16 + (lane & 15);  // A row of this lane in the MFMA operand layout
  int srow[4];                                     // A rows of this lane's accumulator elements
#pragma unroll
  for (int i = 0; i < 4; ++i) srow[i] = PHYS_ROW(wave * 16 + 4 * (lane >> 4) + i);
  const int kb_per_row = K / 128;
  const float* asf = static_cast<const float*>(p.As);
  const uint32_t* asu = static_cast<const uint32_t*>(p.As);
  const int amx_row = PHYS_ROW(arow_mfma);
#undef PHYS_ROW
  const float* bsf0 = nullptr;
  const float* bsf1 = nullptr;
  const uint32_t* bsu[16];
  if (WF == W_FP8_B128) {
    const size_t sstr = p.bs_stride;
    if (EPI == EPI_GATEUP) {
      bsf0 = static_cast<const float*>(p.B0s) + e * sstr + size_t(n0 / 128) * kb_per_row;
      bsf1 = static_cast<const float*>(p.B1s) + e * sstr + size_t(n0 / 128) * kb_per_row;
    } else {
      const int nblk = p.N / 128;
      bsf0 = static_cast<const float*>(p.B0s) + e * sstr + size_t(min(n0 / 128, nblk - 1)) * kb_per_row;
      bsf1 = static_cast<const float*>(p.B0s) + e * sstr + size_t(min(n0 / 128 + 1, nblk - 1)) * kb_per_row;
    }
  }
  if (WF == W_MXFP8) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int nl = j * 16 + (lane & 15);
      int grow;
      const uint8_t* sb;
      if (EPI == EPI_GATEUP) {
        sb = static_cast<const uint8_t*>(nl < BN / 2 ? p.B0s : p.B1s);
        grow = n0 + (nl < BN / 2 ? nl : nl - BN / 2);
      } else {
        sb = static_cast<const uint8_t*>(p.B0s);
        grow = min(n0 + nl, p.N - 1);
      }
      bsu[j] = reinterpret_cast<const uint32_t*>(sb + e * p.bs_stride + size_t(grow) * (K / 32));
    }
  }

  f32x4 acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[2], rb[8];
#define GLOAD(st)                                                                          \
  do {                                                                                     \
    _Pragma("unroll") for (int i = 0; i < 2; ++i) ra[i] =                                  \
        *reinterpret_cast<const u32x4*>(ga[i] + size_t(st) * BKB);                         \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) rb[i] =                                  \
        *reinterpret_cast<const u32x4*>(gb[i] + size_t(st) * BKB);                         \
  } while (0)
#define LSTORE(bf)                                                                          \
  do {                                                                                      \
    _Pragma("unroll") for (int i = 0; i < 2; ++i) *reinterpret_cast<u32x4*>(&sA[bf][la[i]]) = ra[i]; \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(&sB[bf][lb[i]]) = rb[i]; \
  } while (0)

  GLOAD(0);
  LSTORE(0);
  __syncthreads();

  for (int s = 0; s < nk; ++s) {
    const int buf = s & 1;
    if (s + 1 < nk) GLOAD(s + 1);
    if (WF == W_BF16) {
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        const int c = ss * 4 + (lane >> 4);
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sA[buf][swz(arow_mfma, c)]);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(&sB[buf][swz(j * 16 + (lane & 15), c)]);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
        }
      }
    } else {
      // operand layout of the 16x16x128 8-bit instruction: lane group g = lane/16
      // holds K [16g, 16g+16) in bytes 0-15 and K [64+16g, 64+16g+16) in bytes
      // 16-31; the e8m0 scale of lane l covers row l%16, K block [32(l/16), +32)
      const int c0 = lane >> 4;
      i32x8 a;
      {
        const i32x4 lo = *reinterpret_cast<const i32x4*>(&sA[buf][swz(arow_mfma, c0)]);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(&sA[buf][swz(arow_mfma, c0 + 4)]);
        a = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
      if (WF == W_FP8_B128) {
        float sx[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sx[i] = asf[size_t(srow[i]) * kb_per_row + s];
        const float sb0 = bsf0[s], sb1 = bsf1[s];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int br = j * 16 + (lane & 15);
          const i32x4 lo = *reinterpret_cast<const i32x4*>(&sB[buf][swz(br, c0)]);
          const i32x4 hi = *reinterpret_cast<const i32x4*>(&sB[buf][swz(br, c0 + 4)]);
          const i32x8 b = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          const f32x4 t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0,
                                                                            0, 127, 0, 127);
          const float sbj = (j < 8) ? sb0 : sb1;
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[j][i] = fmaf(t[i], sx[i] * sbj, acc[j][i]);
        }
      } else {  // MXFP8
        const int sa = int((asu[size_t(amx_row) * kb_per_row + s] >> (8 * (lane >> 4))) & 0xffu);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int br = j * 16 + (lane & 15);
          const i32x4 lo = *reinterpret_cast<const i32x4*>(&sB[buf][swz(br, c0)]);
          const i32x4 hi = *reinterpret_cast<const i32x4*>(&sB[buf][swz(br, c0 + 4)]);
          const i32x8 b = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          const int sb = int((bsu[j][s] >> (8 * (lane >> 4))) & 0xffu);
          acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[j], 0, 0, 0, sa, 0, sb);
        }
      }
    }
    if (s + 1 < nk) LSTORE(buf ^ 1);
    __syncthreads();
  }

#undef GLOAD
#undef LSTORE
  // ------------------------------------------------------------ epilogue
  const int col_l = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = wave * 16 + 4 * (lane >> 4) + i;
    const bool rvalid = rl < mrows;
    const size_t orow = size_t(seg0 + m0 + rl);
    if (EPI == EPI_GATEUP) {
      float h[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) h[j] = silu(acc[j][i]) * acc[j + 8][i];
      if (p.C_f32) {
        if (rvalid)
#pragma unroll
          for (int j = 0; j < 8; ++j) p.C_f32[orow * p.ldc + n0 + j * 16 + col_l] = h[j];
      } else if (p.out_afmt == A_NONE) {
        if (rvalid)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            static_cast<uint16_t*>(p.C)[orow * p.ldc + n0 + j * 16 + col_l] = f32_to_bf16(h[j]);
      } else if (p.out_afmt == A_FP8_1X128) {
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(h[j]));
        amax = group_max<16>(amax);
        const float sc = amax > 0.f ? __fdiv_rn(amax, kE4M3Max) : 1.0f;
        if (rvalid) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            static_cast<uint8_t*>(p.C)[orow * p.ldc + n0 + j * 16 + col_l] = uint8_t(f32_to_e4m3(__fdiv_rn(h[j], sc)));
          if (col_l == 0) static_cast<float*>(p.Cs)[orow * (p.N / 128) + n0 / 128] = sc;
        }
      } else {  // MX 1x32: block b = columns [32b, 32b+32) = n-tiles 2b, 2b+1
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          float amax = fmaxf(fabsf(h[2 * b]), fabsf(h[2 * b + 1]));
          amax = group_max<16>(amax);
          const int xe = mx_exponent(amax);
          if (rvalid) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
              const int j = 2 * b + jj;
              static_cast<uint8_t*>(p.C)[orow * p.ldc + n0 + j * 16 + col_l] =
                  uint8_t(f32_to_e4m3(__builtin_amdgcn_ldexpf(h[j], -xe)));
            }
            if (col_l == 0) static_cast<uint8_t*>(p.Cs)[orow * (p.N / 32) + n0 / 32 + b] = uint8_t(xe + 127);
          }
        }
      }
    } else {
      if (!rvalid) continue;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int col = n0 + j * 16 + col_l;
        if (col < p.N) {
          if (EPI == EPI_F32)
            static_cast<float*>(p.C)[orow * p.ldc + col] = acc[j][i];
          else
            static_cast<uint16_t*>(p.C)[orow * p.ldc + col] = f32_to_bf16(acc[j][i]);
        }
      }
    }
  }
}

template <int WF>
hipError_t launch_epi(int epi, const GemmParams& p, dim3 grid, hipStream_t s) {
  switch (epi) {
    case EPI_F32: hipLaunchKernelGGL((gemm_kernel<WF, EPI_F32>), grid, dim3(256), 0, s, p); break;
    case EPI_BF16: hipLaunchKernelGGL((gemm_kernel<WF, EPI_BF16>), grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((gemm_kernel<WF, EPI_GATEUP>), grid, dim3(256), 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int wfmt, int epi, const GemmParams& p, hipStream_t s) {
  const int ntile = p.tiles ? p.max_tiles : (p.M + BM - 1) / BM;
  if (ntile <= 0) return hipSuccess;
  const int nper = epi == EPI_GATEUP ? BN / 2 : BN;
  const dim3 grid(unsigned(ntile), unsigned((p.N + nper - 1) / nper));
  switch (wfmt) {
    case W_BF16: return launch_epi<W_BF16>(epi, p, grid, s);
    case W_FP8_B128: return launch_epi<W_FP8_B128>(epi, p, grid, s);
    default: return launch_epi<W_MXFP8>(epi, p, grid, s);
  }
}

}  // namespace moe
