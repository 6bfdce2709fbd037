// Grouped GEMM on gfx950 matrix cores for the batched expert FFNs (stages
// P1/P2 and Q1/Q2 of the DSV2-236B-MegaKernel README flowchart at T > 1).
//
//   C[r][n] = sum_k A[r][k] * B_e[n][k]   for the rows r of expert e's segment
//
// Weight formats and the matrix-core instruction each uses:
//   bf16      v_mfma_f32_16x16x32_bf16, two per 128-byte K step
//   FP8_B128  v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales; one
//             instruction covers exactly one 128-deep K block, and its fp32
//             result is promoted into the accumulator with the block's
//             activation scale (per row) times weight scale (per 128 rows)
//   MXFP8     v_mfma_scale_f32_16x16x128_f8f6f4 with the e8m0 scales of A and
//             B passed per lane (lane l scales row l%16, K block l/16)
//
// Tile: 128 rows x 256 B-rows x 128 bytes of K per step; 4 waves, each owning
// 64 rows x 128 B-rows (4 x 8 MFMA tiles of 16x16), so every operand read from
// LDS feeds 4 or 8 MFMAs.  Tiles move HBM -> LDS with direct-to-LDS loads
// (global_load_lds_dwordx4: lane l's 16 bytes land at base + 16 l), three
// stages deep, so two steps of loads are in flight during the MFMAs of a
// third.  Each lane fetches the global chunk that belongs at its LDS slot, so
// the LDS image is swizzled (chunk c of row r sits at c ^ ((r >> 1) & 7)):
// the 16 lanes that read one operand column hit 16 distinct bank groups.
// Activation and MX weight scales travel the same way, one dword per row.
//
// Rows come from a device tile list written by the dispatch kernel, so no
// expert count is read back to the host (Mixture-of-Kittens, Abstract).  The
// flat list of (expert, n-block, m-tile) tiles is cut into 8 contiguous
// ranges, one per XCD (blocks are dispatched round robin over the XCDs): the
// tiles that run together on one XCD share their weight panel (m-tiles of the
// same n-block are adjacent) and their activation panel (same expert), so the
// XCD's L2 serves the repeats.
//
// EPI_GATEUP: B-tile rows [128w, 128w+64) are gate rows and [128w+64, 128w+128)
// the up rows of the same 64 intermediate columns, so every lane owns g and u
// of the same (row, column) and the epilogue writes h = SiLU(g) * u directly,
// optionally quantised to e4m3 per 1x128 or 1x32 block ("From 35 to 873
// tokens/s", Rounds 12-15: the next matmul's input quantised by the producer).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int BM = kGemmBM;   // 128 rows
constexpr int BNT = 256;      // B rows per tile
constexpr int BKB = 128;      // bytes of K per step
constexpr int kStages = 3;
constexpr int kLdsA = BM * BKB;    // 16 KB
constexpr int kLdsB = BNT * BKB;   // 32 KB
constexpr int kLdsAS = BM * 4;     // one scale dword per A row per step
constexpr int kLdsBS = BNT * 4;    // one scale dword per B row per step (MX)
constexpr int kMaxKSteps = 64;     // FP8_B128: K <= 8192 (checked by the host)

template <int WF>
MOE_DEV constexpr int esz() { return WF == W_BF16 ? 2 : 1; }

// LDS byte offset of 16-byte chunk c of tile row r
MOE_DEV int swz(int r, int c) { return r * BKB + ((c ^ ((r >> 1) & 7)) << 4); }

// Direct-to-LDS loads: the 64 lanes' data lands at lds_base + 16 l (x4) or
// + 4 l (x1).  lds_base is wave-uniform.  M0 is reserved for this use; nothing
// else in these kernels reads it.
MOE_DEV void dma16(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_base) : "memory");
}
MOE_DEV void dma4(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds_base) : "memory");
}
template <int N>
MOE_DEV void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
MOE_DEV void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
MOE_DEV uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(p)));
}

template <int WF>
MOE_DEV constexpr int scale_dmas() { return WF == W_MXFP8 ? 2 : (WF == W_FP8_B128 ? 1 : 0); }
template <int WF>
MOE_DEV constexpr int dmas_per_stage() { return 4 + 8 + scale_dmas<WF>(); }

template <int WF, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[kStages][kLdsA];
  __shared__ __attribute__((aligned(16))) uint8_t sB[kStages][kLdsB];
  __shared__ __attribute__((aligned(16))) uint32_t sAS[kStages][BM];
  __shared__ __attribute__((aligned(16))) uint32_t sBS[WF == W_MXFP8 ? kStages : 1][WF == W_MXFP8 ? BNT : 1];
  __shared__ float sAmax[2][BM];
  __shared__ float sWs[WF == W_FP8_B128 ? 4 : 1][2][WF == W_FP8_B128 ? kMaxKSteps : 1];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1;
  const int nper = EPI == EPI_GATEUP ? BNT / 2 : BNT;  // output columns per tile
  const int NB = (p.N + nper - 1) / nper;

  // ---------------------------------------------------------- tile schedule
  const int nt_list = p.tiles ? p.ntiles[0] : (p.M + BM - 1) / BM;
  const int KS = (EPI == EPI_F32 && p.ksplit > 1) ? p.ksplit : 1;
  const int T = nt_list * NB * KS;
  const int chunk = (T + 7) / 8;
  int idx = int(blockIdx.x % 8) * chunk + int(blockIdx.x / 8);
  if (int(blockIdx.x / 8) >= chunk || idx >= T) return;
  const int kz = idx % KS;  // K slice (split-K: slices of one tile are adjacent)
  idx /= KS;
  int e = 0, m0, nb;
  {
    const int pe = idx / NB;  // a tile-list entry of the same expert
    int be = 0, ne = nt_list;
    if (p.tiles) {
      e = p.tiles[2 * pe];
      be = pe - p.tiles[2 * pe + 1] / BM;
      const int c0 = min(max(p.seg[e], 0), p.M), c1 = min(max(p.seg[e + 1], c0), p.M);
      ne = max((c1 - c0 + BM - 1) / BM, 1);
    }
    const int local = idx - be * NB;
    nb = local / ne;
    m0 = (local % ne) * BM;
  }
  // segment bounds clamped to [0, M] so malformed offsets cannot address outside the rows
  const int seg0 = p.seg ? min(max(p.seg[e], 0), p.M) : 0;
  const int seg1 = p.seg ? min(max(p.seg[e + 1], seg0), p.M) : p.M;
  const int mrows = min(BM, seg1 - seg0 - m0);
  if (mrows <= 0) return;
  const int n0 = nb * nper;
  const int K = p.K;
  const int nk_all = K * esz<WF>() / BKB;
  const int ks0 = int(long(nk_all) * kz / KS), ks1 = int(long(nk_all) * (kz + 1) / KS);
  const int nk = ks1 - ks0;  // K steps of this slice, starting at step ks0
  const size_t lda_b = size_t(p.lda) * esz<WF>();
  const size_t ldb_b = size_t(K) * esz<WF>();
  const uint8_t* b0 = static_cast<const uint8_t*>(p.B0) + size_t(e) * p.b_stride * esz<WF>();
  const uint8_t* b1 = p.B1 ? static_cast<const uint8_t*>(p.B1) + size_t(e) * p.b_stride * esz<WF>() : nullptr;

  const int* a_map = p.a_map;
  const int a_div = p.a_div;
  const int rbase = seg0 + m0, rlast = mrows - 1;
  const int N = p.N;
  // global row of tile row rl (clamped into the segment)
#define PHYS_ROW(rl) (a_map ? a_map[rbase + min((rl), rlast)] / a_div : rbase + min((rl), rlast))

  // ---------------------------------------------------------- DMA sources
  // A: wave w loads tile rows [32w, 32w+32) as 4 blocks of 8 rows; lane L
  // fetches row 8i + L/8 of its block, chunk (L%8) ^ ((row>>1)&7).
  const uint8_t* ga[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 32 * wave + 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    ga[i] = static_cast<const uint8_t*>(p.A) + size_t(PHYS_ROW(r)) * lda_b + c * 16;
  }
  const uint8_t* gb[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = 64 * wave + 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ ((t >> 1) & 7);
    const uint8_t* base = b0;
    int br;
    if (EPI == EPI_GATEUP) {
      const int w = t >> 7, u = t & 127;
      base = u < 64 ? b0 : b1;
      br = n0 + 64 * w + (u & 63);
    } else {
      br = min(n0 + t, N - 1);
    }
    gb[i] = base + size_t(br) * ldb_b + c * 16;
  }
  // scales: A rows (waves 0,1 own rows [64w, 64w+64); waves 2,3 repeat them, so
  // every wave issues the same number of loads), MX weight rows (64 per wave)
  const int kb_a = WF == W_MXFP8 ? K / 32 : K / 128;  // scale units per A row
  const uint8_t* gas = nullptr;
  const uint8_t* gbs = nullptr;
  if (WF != W_BF16) {
    const int r = 64 * (wave & 1) + lane;
    gas = static_cast<const uint8_t*>(p.As) + size_t(PHYS_ROW(r)) * (WF == W_MXFP8 ? kb_a : kb_a * 4);
  }
  if (WF == W_MXFP8) {
    const int t = 64 * wave + lane;
    int br;
    const uint8_t* base;
    if (EPI == EPI_GATEUP) {
      const int w = t >> 7, u = t & 127;
      base = static_cast<const uint8_t*>(u < 64 ? p.B0s : p.B1s);
      br = n0 + 64 * w + (u & 63);
    } else {
      base = static_cast<const uint8_t*>(p.B0s);
      br = min(n0 + t, p.N - 1);
    }
    gbs = base + size_t(e) * p.bs_stride + size_t(br) * (K / 32);
  }
  // FP8_B128 weight scales: one per (128 B rows, 128 K); a wave's B rows sit in
  // one gate block and one up block (GATEUP) or one block.  All K steps' scales
  // go to LDS before the main loop, which then issues no global load of its own.
  if constexpr (WF == W_FP8_B128) {
    const int kb = K / 128;
    for (int q = tid; q < 4 * 2 * kb; q += 256) {
      const int w = q / (2 * kb), g = (q / kb) & 1, ks = q % kb;
      const int wnq = w >> 1;
      const float* src;
      if (EPI == EPI_GATEUP)
        src = static_cast<const float*>(g ? p.B1s : p.B0s) + size_t(e) * p.bs_stride + size_t(n0 / 128) * kb;
      else
        src = static_cast<const float*>(p.B0s) + size_t(e) * p.bs_stride +
              size_t(min((n0 + 128 * wnq) / 128, p.N / 128 - 1)) * kb;
      sWs[w][g][ks] = src[ks];
    }
    __syncthreads();
  }

#undef PHYS_ROW
  auto issue = [&](int s) {
    const int st = s % kStages;
    const size_t ko = size_t(s + ks0) * BKB;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(ga[i] + ko, lds_addr(&sA[st][(32 * wave + 8 * i) * BKB]));
#pragma unroll
    for (int i = 0; i < 8; ++i) dma16(gb[i] + ko, lds_addr(&sB[st][(64 * wave + 8 * i) * BKB]));
    if constexpr (WF == W_MXFP8) {
      dma4(gas + 4 * (s + ks0), lds_addr(&sAS[st][64 * (wave & 1)]));
      dma4(gbs + 4 * (s + ks0), lds_addr(&sBS[st][64 * wave]));
    } else if constexpr (WF == W_FP8_B128) {
      dma4(gas + 4 * (s + ks0), lds_addr(&sAS[st][64 * (wave & 1)]));
    }
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int c0 = lane >> 4;  // operand chunk of this lane group (and c0 + 4)
  const int ra = 64 * wm + (lane & 15), rb = 128 * wn + (lane & 15);

  if (nk > 0) issue(0);
  if (nk > 1) issue(1);
  for (int s = 0; s < nk; ++s) {
    const int st = s % kStages;
    if (s + 1 < nk)
      wait_vm<dmas_per_stage<WF>()>();
    else
      wait_vm<0>();
    barrier();
    if (s + 2 < nk) issue(s + 2);
    const uint8_t* A_ = sA[st];
    const uint8_t* B_ = sB[st];
    if (WF == W_BF16) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const bf16x8*>(A_ + swz(ra + 16 * i, c0 + 4 * h));
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(B_ + swz(rb + 16 * j, c0 + 4 * h));
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b, acc[i][j], 0, 0, 0);
        }
      }
    } else {
      i32x8 a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const i32x4 lo = *reinterpret_cast<const i32x4*>(A_ + swz(ra + 16 * i, c0));
        const i32x4 hi = *reinterpret_cast<const i32x4*>(A_ + swz(ra + 16 * i, c0 + 4));
        a[i] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
      if (WF == W_MXFP8) {
        int sa[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sa[i] = int((sAS[st][ra + 16 * i] >> (8 * c0)) & 0xffu);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const i32x4 lo = *reinterpret_cast<const i32x4*>(B_ + swz(rb + 16 * j, c0));
          const i32x4 hi = *reinterpret_cast<const i32x4*>(B_ + swz(rb + 16 * j, c0 + 4));
          const i32x8 b = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          const int sb = int((sBS[st][rb + 16 * j] >> (8 * c0)) & 0xffu);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i], b, acc[i][j], 0, 0, 0, sa[i], 0, sb);
        }
      } else {  // FP8_B128: unit-scale MFMA per 128-deep block, promoted with sa * sb
        const float w0 = sWs[wave][0][s + ks0], w1 = sWs[wave][1][s + ks0];
        f32x4 fa[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          fa[i] = *reinterpret_cast<const f32x4*>(&sAS[st][64 * wm + 16 * i + 4 * c0]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const i32x4 lo = *reinterpret_cast<const i32x4*>(B_ + swz(rb + 16 * j, c0));
          const i32x4 hi = *reinterpret_cast<const i32x4*>(B_ + swz(rb + 16 * j, c0 + 4));
          const i32x8 b = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          const float wj = (EPI == EPI_GATEUP && j >= 4) ? w1 : w0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f32x4 t = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i], b, f32x4{0.f, 0.f, 0.f, 0.f}, 0,
                                                                              0, 0, 127, 0, 127);
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[i][j][k] = fmaf(t[k], fa[i][k] * wj, acc[i][j][k]);
          }
        }
      }
    }
  }

  // ------------------------------------------------------------ epilogue
  // lane l holds rows 4(l/16)+k (k < 4) of each 16x16 tile, column l%16
  const int col_l = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int rl = 64 * wm + 16 * i + 4 * c0 + k;
      const bool rvalid = rl < mrows;
      const size_t orow = size_t(seg0 + m0 + rl);
      if (EPI == EPI_GATEUP) {
        float h[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) h[j] = silu(acc[i][j][k]) * acc[i][j + 4][k];
        const int cb = n0 + 64 * wn;  // first h column of this wave
        if (p.C_f32) {
          if (rvalid)
#pragma unroll
            for (int j = 0; j < 4; ++j) p.C_f32[orow * p.ldc + cb + 16 * j + col_l] = h[j];
        } else if (p.out_afmt == A_NONE) {
          if (rvalid)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              static_cast<uint16_t*>(p.C)[orow * p.ldc + cb + 16 * j + col_l] = f32_to_bf16(h[j]);
        } else if (p.out_afmt == A_MXFP8_1X32) {  // block b = columns [32b, 32b+32) of this wave's 64
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            float amax = fmaxf(fabsf(h[2 * b]), fabsf(h[2 * b + 1]));
            amax = group_max<16>(amax);
            const int xe = mx_exponent(amax);
            if (rvalid) {
#pragma unroll
              for (int jj = 0; jj < 2; ++jj) {
                const int j = 2 * b + jj;
                static_cast<uint8_t*>(p.C)[orow * p.ldc + cb + 16 * j + col_l] =
                    uint8_t(f32_to_e4m3(__builtin_amdgcn_ldexpf(h[j], -xe)));
              }
              if (col_l == 0) static_cast<uint8_t*>(p.Cs)[orow * (p.N / 32) + cb / 32 + b] = uint8_t(xe + 127);
            }
          }
        } else {  // A_FP8_1X128: the 128-column block spans both column waves
          float amax = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fabsf(h[j]));
          amax = group_max<16>(amax);
          if (col_l == 0) sAmax[wn][rl] = amax;
          __syncthreads();
          amax = fmaxf(sAmax[0][rl], sAmax[1][rl]);
          __syncthreads();
          const float sc = amax > 0.f ? __fdiv_rn(amax, kE4M3Max) : 1.0f;
          if (rvalid) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              static_cast<uint8_t*>(p.C)[orow * p.ldc + cb + 16 * j + col_l] = uint8_t(f32_to_e4m3(__fdiv_rn(h[j], sc)));
            if (col_l == 0 && wn == 0) static_cast<float*>(p.Cs)[orow * (p.N / 128) + n0 / 128] = sc;
          }
        }
      } else {
        if (!rvalid) continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int col = n0 + 128 * wn + 16 * j + col_l;
          if (col < p.N) {
            if (EPI == EPI_F32)
              static_cast<float*>(p.C)[kz * p.c_split + orow * p.ldc + col] = acc[i][j][k];
            else
              static_cast<uint16_t*>(p.C)[orow * p.ldc + col] = f32_to_bf16(acc[i][j][k]);
          }
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
  const int nper = epi == EPI_GATEUP ? BNT / 2 : BNT;
  const long tiles = long(ntile) * ((p.N + nper - 1) / nper) * (epi == EPI_F32 && p.ksplit > 1 ? p.ksplit : 1);
  const dim3 grid(unsigned((tiles + 7) / 8 * 8));  // the in-kernel schedule maps block b to XCD b % 8
  switch (wfmt) {
    case W_BF16: return launch_epi<W_BF16>(epi, p, grid, s);
    case W_FP8_B128: return launch_epi<W_FP8_B128>(epi, p, grid, s);
    default: return launch_epi<W_MXFP8>(epi, p, grid, s);
  }
}

}  // namespace moe
