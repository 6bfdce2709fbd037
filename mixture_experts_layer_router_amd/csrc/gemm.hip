// Grouped GEMM on gfx950 matrix cores for the batched expert FFNs (stages
// P1/P2 and Q1/Q2 of the DSV2-236B-MegaKernel README flowchart at T > 1).
//
//   C[r][n] = sum_k A[r][k] * B_e[n][k]   for the rows r of expert e's segment
//
// Weight formats and the matrix-core instruction each uses (32x32 output
// blocks: on gfx950 these issue at 4.4 PFLOP/s FP8 and 2.2 PFLOP/s bf16 from
// one wave per SIMD, against 3.5 and 1.25 for the 16x16 shapes):
//   bf16      v_mfma_f32_32x32x16_bf16, four per 128-byte K step
//   MXFP8     v_mfma_scale_f32_32x32x64_f8f6f4, two per step, with the e8m0
//             scales of A and B passed per lane (lane l scales row l%32 of its
//             operand for the 32-deep K block l/32 of the instruction)
//   FP8_B128  the same instruction with unit scales; the two of one 128-deep
//             K block accumulate into a temporary, which is promoted into the
//             accumulator with the block's activation scale (per row) times
//             its weight scale (per 128 B rows)
//
// Tile: 128 rows x 256 B rows x 128 bytes of K per step; 4 waves, each owning
// 64 rows x 128 B rows (2 x 4 blocks of 32x32).  Tiles move HBM -> LDS with
// direct-to-LDS loads (global_load_lds_dwordx4: lane l's 16 bytes land at
// base + 16 l), three stages deep.  The LDS image is swizzled (16-byte chunk c
// of row r sits at c ^ ((r >> 1) & 7)) so that the 16 lanes of one LDS read
// cycle hit 16 distinct bank groups.  Operand layout in registers: for slot
// c = 0..3 of a 128-byte step, lane l reads chunk 2c + l/32 of row l%32 of its
// block; an FP8 instruction for K half h takes slots 2h and 2h+1 (K bytes
// [16g, 16g+16) and [32+16g, 48+16g) of the half, g = l/32), a bf16
// instruction for K quarter q takes slot q.
//
// bf16, MXFP8 and the FP8_B128 gate/up keep two register sets of operands:
// the reads of step s+1 are issued among the MFMAs of step s, together with
// the direct-to-LDS loads of step s+3, in a fixed interleave, so the matrix
// pipe does not wait for LDS at the step boundary.  The FP8_B128 down GEMMs
// need those registers for their temporaries beside their epilogue and read
// each step's operands at the start of the step.
//
// Rows come from a device tile list written by the dispatch kernel, so no
// expert count is read back to the host (Mixture-of-Kittens, Abstract); the
// tile order is gemm_dev.h's XCD-aware schedule.  In the FP8_B128 path a wave
// whose second 32-row block lies past the tile's valid rows skips that
// block's MFMAs.  This kernel serves FP8_B128, MXFP8 with K not a multiple of
// 512, and the dense GEMMs too small to fill the chip with 256-row tiles
// (gemm2.hip serves the rest).
//
// EPI_GATEUP: B-tile rows [128w, 128w+64) are gate rows and [128w+64, 128w+128)
// the up rows of the same 64 intermediate columns, so blocks j and j+2 of a
// wave hold g and u of the same (row, column) and the epilogue writes
// h = SiLU(g) * u directly, optionally quantised to e4m3 per 1x128 or 1x32
// block ("From 35 to 873 tokens/s", Rounds 12-15: the next matmul's input
// quantised by the producer).
#include "gemm_dev.h"

namespace moe {

namespace {

using namespace gemm_dev;

constexpr int BM = kGemmBM;  // 128 rows
constexpr int BNT = 256;     // B rows per tile
constexpr int BKB = 128;     // bytes of K per step
constexpr int kStages = 3;
constexpr int kLdsA = BM * BKB;   // 16 KB
constexpr int kLdsB = BNT * BKB;  // 32 KB
static_assert(kGemmMaxK / 128 <= 64, "one 64-lane load holds a block's weight scales");

template <int WF>
MOE_DEV constexpr int scale_dmas() { return WF == W_MXFP8 ? 2 : (WF == W_FP8_B128 ? 1 : 0); }
template <int WF>
MOE_DEV constexpr int dmas_per_stage() { return 4 + 8 + scale_dmas<WF>(); }


// one step's operands of one lane: slot c of block i sits in half c%2 of
// a[i][c/2], so an FP8 instruction for K half h takes a[i][h] whole
struct Frag {
  i32x8 a[2][2];  // [32-row block i][K half]
  i32x8 b[4][2];  // [32-row B block j][K half]
  uint32_t sa[2], sb[4];  // MXFP8: the four e8m0 scales of the step, one byte per K block;
                          // FP8_B128: sa[i] holds the fp32 activation scale of the lane's row of block i
  float w[2];             // FP8_B128: the step's weight scales of the wave's gate (or only) and up blocks
};
MOE_DEV void set_slot(i32x8& v, int c, i32x4 x) {
  if (c & 1)
    v.hi = x;
  else
    v.lo = x;
}
MOE_DEV i32x4 get_slot(const i32x8& v, int c) { return (c & 1) ? v.hi : v.lo; }

template <int WF, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * (kLdsA + kLdsB)];
  __shared__ __attribute__((aligned(16))) uint32_t sAS[kStages][BM];
  __shared__ __attribute__((aligned(16))) uint32_t sBS[WF == W_MXFP8 ? kStages : 1][WF == W_MXFP8 ? BNT : 1];
  __shared__ float sAmax[2][BM];
  __shared__ __attribute__((aligned(16))) float sWs[WF == W_FP8_B128 ? 4 : 1][2][WF == W_FP8_B128 ? 64 : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int g = lane >> 5, l32 = lane & 31;
  const int nper = EPI == EPI_GATEUP ? BNT / 2 : BNT;  // output columns per tile
  const int KS = (EPI == EPI_F32 && p.ksplit > 1) ? p.ksplit : 1;
  const Tile tl = tile_of(p, BM, nper, KS, int(blockIdx.x));
  if (!tl.valid) return;
  const int e = tl.e, m0 = tl.m0, n0 = tl.n0, seg0 = tl.seg0, mrows = tl.mrows, kz = tl.kz;
  const int K = p.K;
  const int N = p.N;
  const int nk_all = K * esz<WF>() / BKB;
  const int ks0 = int(long(nk_all) * kz / KS), ks1 = int(long(nk_all) * (kz + 1) / KS);
  const int nk = ks1 - ks0;  // K steps of this slice, starting at step ks0
  const uint32_t lda_b = uint32_t(p.lda) * esz<WF>();
  const uint32_t ldb_b = uint32_t(K) * esz<WF>();

  const int* a_map = p.a_map;
  const int a_div = p.a_div;
  const int rbase = seg0 + m0, rlast = mrows - 1;
  // global row of tile row rl (clamped into the segment)
#define PHYS_ROW(rl) uint32_t(a_map ? a_map[rbase + min((rl), rlast)] / a_div : rbase + min((rl), rlast))

  // ---------------------------------------------------------- DMA sources
  // A: wave w loads tile rows [32w, 32w+32) as 4 blocks of 8 rows; lane L
  // fetches row 8i + L/8 of its block, chunk (L%8) ^ ((row>>1)&7).
  const uint8_t* a_base = uniform_ptr(p.A);
  uint32_t oa[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 32 * wave + 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    oa[i] = PHYS_ROW(r) * lda_b + c * 16;
  }
  // B: wave w loads tile B rows [64w, 64w+64); for EPI_GATEUP these are gate
  // rows (w even) or up rows (w odd) of intermediate columns n0 + 64 (w/2) + [0, 64)
  const uint8_t* b_base;
  uint32_t ob[8];
  {
    const void* bsrc = (EPI == EPI_GATEUP && (wave & 1)) ? p.B1 : p.B0;
    b_base = uniform_ptr(static_cast<const uint8_t*>(bsrc) + size_t(e) * p.b_stride * esz<WF>());
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = 64 * wave + 8 * i + (lane >> 3);
      const int c = (lane & 7) ^ ((t >> 1) & 7);
      const int br = EPI == EPI_GATEUP ? n0 + 64 * wn + 8 * i + (lane >> 3) : min(n0 + t, N - 1);
      ob[i] = uint32_t(br) * ldb_b + c * 16;
    }
  }
  // scales: A rows (waves 0,1 own rows [64w, 64w+64); waves 2,3 repeat them, so
  // every wave issues the same number of loads), MX weight rows (64 per wave)
  const uint8_t* as_base = nullptr;
  const uint8_t* bs_base = nullptr;
  uint32_t oas = 0, obs = 0;
  if constexpr (WF != W_BF16) {
    as_base = uniform_ptr(p.As);
    const int r = 64 * wm + lane;
    oas = PHYS_ROW(r) * (WF == W_MXFP8 ? uint32_t(K / 32) : uint32_t(K / 128) * 4u);
  }
  if constexpr (WF == W_MXFP8) {
    const void* ssrc = (EPI == EPI_GATEUP && (wave & 1)) ? p.B1s : p.B0s;
    bs_base = uniform_ptr(static_cast<const uint8_t*>(ssrc) + size_t(e) * p.bs_stride);
    const int br = EPI == EPI_GATEUP ? n0 + 64 * wn + lane : min(n0 + 64 * wave + lane, N - 1);
    obs = uint32_t(br) * uint32_t(K / 32);
  }
#undef PHYS_ROW
  // FP8_B128 weight scales: one per (128 B rows, 128 K); a wave's B rows sit in
  // one gate block and one up block (GATEUP) or one block.  Each wave loads
  // every K step's scales of its blocks (K/128 <= 64: one direct-to-LDS load
  // per block, lane l fetching step l) ahead of the prologue's tile loads, so
  // the prologue's wait covers them and the main loop issues no other load.
  const uint8_t* ws_base[2] = {nullptr, nullptr};
  uint32_t ows = 0;
  if constexpr (WF == W_FP8_B128) {
    const int kb = K / 128;
    ows = uint32_t(min(lane, kb - 1)) * 4u;
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      const float* src;
      if (EPI == EPI_GATEUP)
        src = static_cast<const float*>(gg ? p.B1s : p.B0s) + size_t(e) * p.bs_stride + size_t(n0 / 128) * kb;
      else
        src = static_cast<const float*>(p.B0s) + size_t(e) * p.bs_stride +
              size_t(min((n0 + 128 * wn) / 128, N / 128 - 1)) * kb;
      ws_base[gg] = uniform_ptr(src);
    }
  }
  auto wscale_dma = [&]() {
    if constexpr (WF == W_FP8_B128) {
      dma4(ows, ws_base[0], lds_addr(&sWs[wave][0][0]));
      if constexpr (EPI == EPI_GATEUP) dma4(ows, ws_base[1], lds_addr(&sWs[wave][1][0]));
    }
  };

  const uint32_t lds_a0 = lds_addr(smem), lds_b0 = lds_a0 + kStages * kLdsA;
  // direct-to-LDS load d of K step kstep into stage st
  auto dma_op = [&](int d, int st, int kstep) {
    if (d < 4) {
      dma16(oa[d], a_base + size_t(kstep) * BKB, lds_a0 + st * kLdsA + (32 * wave + 8 * d) * BKB);
    } else if (d < 12) {
      dma16(ob[d - 4], b_base + size_t(kstep) * BKB, lds_b0 + st * kLdsB + (64 * wave + 8 * (d - 4)) * BKB);
    } else if (d == 12) {
      dma4(oas, as_base + 4 * kstep, lds_addr(&sAS[st][64 * wm]));
    } else if constexpr (WF == W_MXFP8) {
      dma4(obs, bs_base + 4 * kstep, lds_addr(&sBS[st][64 * wave]));
    }
  };
  constexpr int DPS = dmas_per_stage<WF>();
  auto issue = [&](int s) {
#pragma unroll
    for (int d = 0; d < DPS; ++d) dma_op(d, s % kStages, s + ks0);
  };

  // LDS operand reads: lane's row within its block is l32; slot c reads chunk 2c + g
  int colo[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) colo[c] = ((2 * c + g) ^ ((l32 >> 1) & 7)) << 4;
  const int rowA = (64 * wm + l32) * BKB, rowB = (128 * wn + l32) * BKB;
  // read r of a step: A slots (i, c) for i < NI, then B slots (j, c), then MX scales
  auto read_op = [&](int r, Frag& f, int st, auto ni_t) {
    constexpr int NI = decltype(ni_t)::value;
    const uint8_t* As_ = smem + st * kLdsA;
    const uint8_t* Bs_ = smem + kStages * kLdsA + st * kLdsB;
    if (r < NI * 4) {
      const int i = r / 4, c = r % 4;
      set_slot(f.a[i][c >> 1], c, *reinterpret_cast<const i32x4*>(As_ + rowA + 32 * BKB * i + colo[c]));
    } else if (r < NI * 4 + 16) {
      const int j = (r - NI * 4) / 4, c = (r - NI * 4) % 4;
      set_slot(f.b[j][c >> 1], c, *reinterpret_cast<const i32x4*>(Bs_ + rowB + 32 * BKB * j + colo[c]));
    } else if (r < NI * 5 + 16) {
      const int i = r - NI * 4 - 16;
      f.sa[i] = sAS[st][64 * wm + 32 * i + l32];
    } else {
      const int j = r - NI * 5 - 16;
      f.sb[j] = sBS[WF == W_MXFP8 ? st : 0][WF == W_MXFP8 ? 128 * wn + 32 * j + l32 : 0];
    }
  };

  // zero for FP8_B128; the pipelined formats' first step writes it without reading it
  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // MFMA m of a step (bf16 / MXFP8): K part outermost, so the two MFMAs on one
  // accumulator are NI*4 instructions apart.  In the first step the first
  // MFMA of each accumulator starts from zero (no zero-filled registers).
  // B blocks of this wave that hold columns below N (the others are not computed)
  const int nJ = EPI == EPI_GATEUP ? 4 : min(max((N - n0 - 128 * wn + 31) / 32, 0), 4);
  auto mfma_op = [&](int m, const Frag& f, auto ni_t, auto first_t) {
    constexpr int NI = decltype(ni_t)::value;
    const int kq = m / (NI * 4), i = (m / 4) % NI, j = m % 4;
    if (j >= nJ) return;
    f32x16 c = acc[i][j];
    if (decltype(first_t)::value && kq == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) c[r] = 0.f;
    }
    if constexpr (WF == W_BF16) {
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16(get_slot(f.a[i][kq >> 1], kq)),
                                                          as_bf16(get_slot(f.b[j][kq >> 1], kq)), c, 0, 0, 0);
    } else {
      const int sh = 8 * (2 * kq + g);
      const int sa = int((f.sa[i] >> sh) & 0xffu), sb = int((f.sb[j] >> sh) & 0xffu);
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i][kq], f.b[j][kq], c, 0, 0, 0, sa, 0, sb);
    }
  };

  // ------------------------------------------------------------ main loop
  const bool two = 64 * wm + 32 < mrows;  // this wave's second row block holds valid rows
  if constexpr (WF == W_FP8_B128) {
    // One 128-byte step is one 128-deep scale block.  The matrix instruction
    // takes the weight rows as its first operand, so a lane's 16 results of a
    // block are 16 output columns of one row: the promotion scale of a block
    // is one number per lane (the row's activation scale times the block's
    // weight scale).  Blocks b = 2 NI h + 2 i + jj (B half h, row block i,
    // j = 2 h + jj) go in pairs: both first-K-half MFMAs of a pair write a
    // temporary t[b % 4], then both second halves accumulate onto it.  The
    // promotion acc += t * scale is cut into chunks of 8 elements, chunk k of
    // the step (block k/2) issued after MFMA k+3, the last three after the
    // first MFMAs of the next step: between two MFMAs a wave issues in order,
    // so at most one chunk of VALU work sits between them and the matrix pipe
    // keeps busy.  A temporary is rewritten by the block four after its own,
    // at least one MFMA after its last chunk.  The operands of step s+1 are
    // read among the MFMAs of step s, the loads of step s+3 issued among them
    // too.
    auto run = [&](auto ni_t) {
      constexpr int NI = decltype(ni_t)::value;
      constexpr int NBS = 4 * NI;               // blocks per step
      constexpr int NM = 2 * NBS;               // MFMAs per step
      constexpr int NR = NI * 4 + 16 + NI;      // LDS reads: A slots, B slots, activation scales
      constexpr int kLag = 3;                   // chunk k follows MFMA k + kLag
      f32x16 t[4];
      float sc[NI][2];      // this step's promotion scales per (i, h)
      float sc_last = 0.f;  // the previous step's scale of its last pair (i = NI-1, h = 1)
      auto read_w = [&](Frag& f, int ks) {  // weight scales of K step ks (of this slice)
        f.w[0] = sWs[wave][0][ks + ks0];
        f.w[1] = sWs[wave][EPI == EPI_GATEUP ? 1 : 0][ks + ks0];
      };
      auto chunk = [&](int k, float scale) {
        const int b = k / 2, c = k % 2;
        const int h = b / (2 * NI), i = (b / 2) % NI, j = 2 * h + (b & 1);
#pragma unroll
        for (int r = 8 * c; r < 8 * c + 8; ++r) acc[i][j][r] = fmaf(t[b % 4][r], scale, acc[i][j][r]);
      };
      auto step = [&](int s, Frag& cur, Frag& nxt, auto first_t) {
        wait_lgkm0();    // cur is in registers: this wave no longer reads stage s
        wait_vm<DPS>();  // this wave's loads of step s+1 have landed
        barrier();       // ... and every wave's; stage s % 3 is free for step s+3
        const int stn = (s + 1) % kStages, std_ = s % kStages;
        const int kd = min(s + 3, nk - 1) + ks0;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          sc[i][0] = __uint_as_float(cur.sa[i]) * cur.w[0];
          sc[i][1] = __uint_as_float(cur.sa[i]) * cur.w[1];
        }
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          const int p4 = m / 4, q = m % 2, kq = (m / 2) % 2;
          const int b = 2 * p4 + q;
          const int h = b / (2 * NI), i = (b / 2) % NI, j = 2 * h + (b & 1);
          if (kq == 0) {
            f32x16 z;
#pragma unroll
            for (int r = 0; r < 16; ++r) z[r] = 0.f;
            t[b % 4] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cur.b[j][0], cur.a[i][0], z, 0, 0, 0, 127, 0, 127);
          } else {
            t[b % 4] =
                __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cur.b[j][1], cur.a[i][1], t[b % 4], 0, 0, 0, 127, 0, 127);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int r = (m * NR) / NM; r < ((m + 1) * NR) / NM; ++r) read_op(r, nxt, stn, ni_t);
          if (m == NM / 2) read_w(nxt, min(s + 1, nk - 1));
#pragma unroll
          for (int d = (m * DPS) / NM; d < ((m + 1) * DPS) / NM; ++d) dma_op(d, std_, kd);
          __builtin_amdgcn_sched_barrier(0);
          if (m >= kLag) {
            const int k = m - kLag, bk = k / 2;
            chunk(k, sc[(bk / 2) % NI][bk / (2 * NI)]);
          } else if constexpr (!decltype(first_t)::value) {
            chunk(m - kLag + NM, sc_last);  // the previous step's last pair
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        sc_last = sc[NI - 1][1];
      };
      Frag f0, f1;
      wscale_dma();
      issue(0);
      issue(min(1, nk - 1));
      issue(min(2, nk - 1));
      wait_vm<2 * DPS>();  // the weight scales and step 0
      barrier();
#pragma unroll
      for (int r = 0; r < NR; ++r) read_op(r, f0, 0, ni_t);
      read_w(f0, 0);
      const std::true_type first{};
      const std::false_type later{};
      step(0, f0, f1, first);
      int s = 1;
      for (; s + 1 < nk; s += 2) {
        step(s, f1, f0, later);
        step(s + 1, f0, f1, later);
      }
      if (s < nk) step(s, f1, f0, later);
#pragma unroll
      for (int k = NM - kLag; k < NM; ++k) chunk(k, sc_last);  // the last step's pending chunks
    };
    if (nk > 0) {
      if (two)
        run(IC<2>{});
      else
        run(IC<1>{});
    }
  } else {
    auto run = [&](auto ni_t) {
      constexpr int NI = decltype(ni_t)::value;
      constexpr int NM = WF == W_BF16 ? NI * 16 : NI * 8;                // MFMAs per step
      constexpr int NR = NI * 4 + 16 + (WF == W_MXFP8 ? NI + 4 : 0);     // LDS reads per step
      // step s: MFMAs on cur (read during step s-1) interleaved with the reads
      // of step s+1 into nxt and the direct-to-LDS loads of step s+3
      // Every step issues its direct-to-LDS loads; past the last K step they
      // reload the last step into a stage that is not read again (L2 hits),
      // which keeps one instance of the step in the loop and every wait count
      // fixed.
      auto step = [&](int s, Frag& cur, Frag& nxt, auto first_t) {
        wait_lgkm0();  // cur is in registers: this wave no longer reads stage s
        wait_vm<DPS>();  // this wave's loads of step s+1 have landed
        barrier();       // ... and every wave's; stage s % 3 is free for step s+3
        const int stn = (s + 1) % kStages, std_ = s % kStages;
        const int kd = min(s + 3, nk - 1) + ks0;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          mfma_op(m, cur, ni_t, first_t);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int r = (m * NR) / NM; r < ((m + 1) * NR) / NM; ++r) read_op(r, nxt, stn, ni_t);
#pragma unroll
          for (int d = (m * DPS) / NM; d < ((m + 1) * DPS) / NM; ++d) dma_op(d, std_, kd);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      Frag f0, f1;
      issue(0);
      issue(min(1, nk - 1));
      issue(min(2, nk - 1));
      wait_vm<2 * DPS>();
      barrier();
#pragma unroll
      for (int r = 0; r < NR; ++r) read_op(r, f0, 0, ni_t);
      step(0, f0, f1, std::true_type{});
      int s = 1;
      for (; s + 1 < nk; s += 2) {
        step(s, f1, f0, std::false_type{});
        step(s + 1, f0, f1, std::false_type{});
      }
      if (s < nk) step(s, f1, f0, std::false_type{});
    };
    if (nk > 0) run(IC<2>{});
  }
  wait_vm<0>();

  // ------------------------------------------------------------ epilogue
  // lane l holds column l%32 of each 32x32 block, rows 8(r/4) + 4(l/32) + r%4
  auto row_of = [&](int i, int r) { return 64 * wm + 32 * i + 8 * (r >> 2) + 4 * g + (r & 3); };
  if constexpr (EPI == EPI_GATEUP) {
    // h = SiLU(g) * u in place of the gate blocks
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][jj][r] = silu(acc[i][jj][r]) * acc[i][jj + 2][r];
    // Stage the tile's h (128 rows x 128 columns, fp32) through LDS, so that
    // each thread finishes 64 columns of one row in registers: block maxima
    // without cross-lane reductions (a 1x128 block is two threads, combined
    // through LDS), the hardware e4m3 pack, and 16-byte stores.
    constexpr int RSF = 132;  // floats per staged row: 16-byte reads of 16 consecutive rows hit distinct banks
    float* hb = reinterpret_cast<float*>(smem);
    wait_vm<0>();
    __syncthreads();  // every wave is done with the stages
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        if constexpr (WF == W_FP8_B128) {  // lane: row 64 wm + 32 i + l%32, columns 8 q + 4 (l/32) + [0, 4)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<f32x4*>(hb + (64 * wm + 32 * i + l32) * RSF + 64 * wn + 32 * jj + 8 * q + 4 * g) =
                f32x4{acc[i][jj][4 * q], acc[i][jj][4 * q + 1], acc[i][jj][4 * q + 2], acc[i][jj][4 * q + 3]};
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) hb[row_of(i, r) * RSF + 64 * wn + 32 * jj + l32] = acc[i][jj][r];
        }
      }
    __syncthreads();
    const int row = tid & 127, half = tid >> 7;  // this thread: h columns n0 + 64 half + [0, 64) of tile row `row`
    f32x4 v[16];
#pragma unroll
    for (int q4 = 0; q4 < 16; ++q4) v[q4] = *reinterpret_cast<const f32x4*>(hb + row * RSF + 64 * half + 4 * q4);
    float m = 0.f;
#pragma unroll
    for (int q4 = 0; q4 < 16; ++q4)
      m = fmaxf(m, fmaxf(fmaxf(fabsf(v[q4][0]), fabsf(v[q4][1])), fmaxf(fabsf(v[q4][2]), fabsf(v[q4][3]))));
    if (!p.C_f32 && p.out_afmt == A_FP8_1X128) {  // the 128-column block is both halves of the row
      sAmax[half][row] = m;
      __syncthreads();
      m = fmaxf(sAmax[0][row], sAmax[1][row]);
    }
    if (row < mrows) {
      const size_t orow = size_t(seg0 + m0 + row);
      const int col = n0 + 64 * half;
      if (p.C_f32) {
#pragma unroll
        for (int q4 = 0; q4 < 16; ++q4) *reinterpret_cast<f32x4*>(p.C_f32 + orow * p.ldc + col + 4 * q4) = v[q4];
      } else if (p.out_afmt == A_NONE) {
        uint16_t* dst = static_cast<uint16_t*>(p.C) + orow * p.ldc + col;
#pragma unroll
        for (int q8 = 0; q8 < 8; ++q8) {
          i32x4 o;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const f32x4& x = v[2 * q8 + t / 2];
            const int cc = 2 * (t & 1);
            o[t] = int(uint32_t(f32_to_bf16(x[cc])) | (uint32_t(f32_to_bf16(x[cc + 1])) << 16));
          }
          *reinterpret_cast<i32x4*>(dst + 8 * q8) = o;
        }
      } else {
        uint8_t* dst = static_cast<uint8_t*>(p.C) + orow * p.ldc + col;
        if (p.out_afmt == A_MXFP8_1X32) {  // two 1x32 blocks: columns [32b, 32b+32)
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            float am = 0.f;
#pragma unroll
            for (int q4 = 8 * b; q4 < 8 * b + 8; ++q4)
              am = fmaxf(am, fmaxf(fmaxf(fabsf(v[q4][0]), fabsf(v[q4][1])), fmaxf(fabsf(v[q4][2]), fabsf(v[q4][3]))));
            const int xe = mx_exponent(am);
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
              i32x4 o;
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                const f32x4& x = v[8 * b + 4 * q2 + t];
                o[t] = int(e4m3x4_sat(__builtin_amdgcn_ldexpf(x[0], -xe), __builtin_amdgcn_ldexpf(x[1], -xe),
                                      __builtin_amdgcn_ldexpf(x[2], -xe), __builtin_amdgcn_ldexpf(x[3], -xe)));
              }
              *reinterpret_cast<i32x4*>(dst + 32 * b + 16 * q2) = o;
            }
            static_cast<uint8_t*>(p.Cs)[orow * (N / 32) + col / 32 + b] = uint8_t(xe + 127);
          }
        } else {  // 1x128: s = fl32(amax / 448), codes of fl32(v / s)
          const float sc = m > 0.f ? __fdiv_rn(m, kE4M3Max) : 1.0f;
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2) {
            i32x4 o;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const f32x4& x = v[4 * q2 + t];
              o[t] = int(e4m3x4_sat(__fdiv_rn(x[0], sc), __fdiv_rn(x[1], sc), __fdiv_rn(x[2], sc),
                                    __fdiv_rn(x[3], sc)));
            }
            *reinterpret_cast<i32x4*>(dst + 16 * q2) = o;
          }
          if (half == 0) static_cast<float*>(p.Cs)[orow * (N / 128) + n0 / 128] = sc;
        }
      }
    }
  } else if constexpr (WF == W_FP8_B128) {
    // lane: row 64 wm + 32 i + l%32, columns 32 j + 8 q + 4 (l/32) + [0, 4) of the wave's 128
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int rl = 64 * wm + 32 * i + l32;
      if (rl >= mrows) continue;
      const size_t orow = size_t(seg0 + m0 + rl);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = n0 + 128 * wn + 32 * j + 8 * q + 4 * g;
          if (col >= N) continue;
          const f32x4 v{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          if (EPI == EPI_F32) {
            *reinterpret_cast<f32x4*>(static_cast<float*>(p.C) + kz * p.c_split + orow * p.ldc + col) = v;
          } else {
            const uint32_t lo = uint32_t(f32_to_bf16(v[0])) | (uint32_t(f32_to_bf16(v[1])) << 16);
            const uint32_t hi = uint32_t(f32_to_bf16(v[2])) | (uint32_t(f32_to_bf16(v[3])) << 16);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.C) + orow * p.ldc + col) = uint2{lo, hi};
          }
        }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = row_of(i, r);
        if (rl >= mrows) continue;
        const size_t orow = size_t(seg0 + m0 + rl);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = n0 + 128 * wn + 32 * j + l32;
          if (col < N) {
            if (EPI == EPI_F32)
              static_cast<float*>(p.C)[kz * p.c_split + orow * p.ldc + col] = acc[i][j][r];
            else
              static_cast<uint16_t*>(p.C)[orow * p.ldc + col] = f32_to_bf16(acc[i][j][r]);
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
  // FP8_B128: every K step's weight scales sit in one 64-entry LDS row per block
  if (wfmt == W_FP8_B128 && (p.K > kGemmMaxK || p.K % 128)) return hipErrorInvalidValue;
  if (gemm2_chosen(wfmt, epi, p)) return launch_gemm2(wfmt, epi, p, s);
  const int ntile = p.tiles ? p.max_tiles : (p.M + BM - 1) / BM;
  if (ntile <= 0) return hipSuccess;
  // the kernels address A rows and one group's B rows with 32-bit byte offsets
  const long es = wfmt == W_BF16 ? 2 : 1;
  const long a_rows = p.a_map ? (long(p.M) + p.a_div - 1) / p.a_div : long(p.M);
  if (a_rows * p.lda * es >= (1L << 32) || long(p.N) * p.K * es >= (1L << 32)) return hipErrorInvalidValue;
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
