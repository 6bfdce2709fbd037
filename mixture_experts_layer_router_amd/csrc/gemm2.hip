// Grouped GEMM, large-tile variant, for bf16 and MXFP8 weights (stages P1/P2
// and Q1/Q2 of the DSV2-236B-MegaKernel README flowchart at batched sizes):
//
//   C[r][n] = sum_k A[r][k] * B_e[n][k]   for the rows r of expert e's segment
//
// Tile: 256 rows x 256 B rows, 64 bytes of K per step, 4 waves each owning
// 128 x 128 (4 x 4 blocks of 32x32), plus up to 32 extra rows (tile rows
// 256-287, one 32-row block) when an expert's segment holds more than 256
// rows: each wave computes that block against two of the B blocks it
// already holds, so a 257-288-row segment streams its weight panel once
// instead of running a second, nearly empty tile (a tile's time follows the
// bytes it loads, so such a tail tile cost about half a full one).
//
// Measured on MI355X, a CU moves about 64 bytes per clock from L2 into LDS
// when each load instruction covers whole 128-byte row segments (8 rows x
// 128 B), but only about 32 when it covers 16 rows x 64 B; this tile needs
// 32 bytes per clock at the full FP8 matrix rate (a 128 x 256 tile needs
// 47).  So the loads move 128 bytes of each row, two K steps, at a time:
// two LDS buffers (A 288 rows and B 256 rows x 128 B each), double-buffered
// per step pair.  The loads of pair q+2 are issued among the MFMAs of the
// odd step that starts pair q's second half, into the buffer pair q has just
// released, and waited for two steps later.  The operand reads of step s+1
// go among the MFMAs of step s: the A blocks and one B block into a second
// register set, the other B blocks and the extra A block into the registers
// they replace, right after their last MFMA of step s.
//
//   bf16   v_mfma_f32_32x32x16_bf16, two per block per step
//   MXFP8  v_mfma_scale_f32_32x32x64_f8f6f4, one per block per step, with the
//          e8m0 scales of A and B per lane (lane l scales row l%32 for the
//          32-deep K block l/32 of the instruction)
//
// LDS image: row r of a buffer holds its 128 bytes (steps 2q, 2q+1) as 8
// chunks of 16, chunk c at c ^ ((r >> 1) & 7), so the 16 lanes of one LDS
// read cycle (16 rows, one chunk) hit 16 distinct bank groups.  Lane l's
// operand for a block in step half h is chunk 4h + l/32 (bytes 0-15) and
// chunk 4h + 2 + l/32 (bytes 16-31) of row l%32: K bytes [16g, 16g+16) and
// [32+16g, 48+16g) of the step, the instruction's K layout.
//
// MX scales (one e8m0 byte per 32 K of a row) are loaded once per 8 steps
// (512 K): 16 bytes per row per load, into one of two LDS buffers, so the
// scale loads add an eighth of the tile loads' cache-line requests instead of
// matching them.  Group g + 1 is loaded at step 8g into the buffer group g - 1
// used; every wave finished reading group g - 1 before the barrier of step
// 8g - 1.  K must be a multiple of 512 (the host checks).
//
// A wave of row half wm keeps B block j of its column half in its register
// slot j ^ wm, so the extra block's operands are always slots 0 and 2
// (compile-time register indices) and slots j, j + 2 still pair the same
// columns of gate and up.
//
// EPI_GATEUP: B-tile rows [128w, 128w+64) are gate rows and [128w+64,
// 128w+128) the up rows of the same 64 intermediate columns, so blocks j and
// j+2 of a wave hold g and u of the same (row, column) and the epilogue writes
// h = SiLU(g) * u, as bf16, fp32 or MXFP8 codes per 1x32 block ("From 35 to
// 873 tokens/s", Rounds 12-15).  The other epilogues stage the fp32 / bf16
// tile through LDS and store whole 16-byte row chunks.
#include <algorithm>

#include "gemm_dev.h"

namespace moe {

namespace {

using namespace gemm_dev;

constexpr int BM = kGemm2BM;     // 256 main rows
constexpr int BMX = kGemm2Rows;  // 288: main rows + the extra block
constexpr int BNT = 256;         // B rows per tile
constexpr int BKB = 64;          // bytes of K per step
constexpr int RB = 2 * BKB;      // bytes per LDS row: a step pair
constexpr int kBufs = 2;         // LDS buffers (step pairs)
constexpr int kLdsA = BMX * RB;  // 36 KB
constexpr int kLdsB = BNT * RB;  // 32 KB
constexpr int kSG = 8;           // K steps per MX scale group (512 K)
constexpr int kSBuf = 2;         // MX scale group buffers
constexpr int kDPP = 17;         // tile loads per wave per step pair: 8 A, 8 B, 1 extra A
static_assert(BMX - BM == 32, "the extra rows are one 32-row MFMA block");

// Operands of one K step.  The A blocks, B register slot 3 and the A scales
// are double-buffered: read among the first MFMAs of the step before.  B slots
// 0-2, the extra A block and their scales are single-buffered: the MFMAs of a
// step go B slot by B slot, and each slot's operands for the next step are
// read right after that slot's last MFMA (slot 3 last, so it cannot wait).
struct Frag {
  i32x8 a[4];  // [32-row block i]: chunk g | chunk 2+g of the step's 64 bytes
  i32x8 b3;    // B register slot 3 (B block 3 ^ wm)
  uint32_t sa[4], sb3;  // MXFP8: e8m0 byte of the lane's row for its K block
};
struct Single {
  i32x8 b[3];  // B register slots 0-2 (B blocks j ^ wm)
  i32x8 ax;    // the extra 32-row block (tile rows 256-287)
  uint32_t sb[3], sax;
};

// LDS of one workgroup: the operand buffers, then (MXFP8) the scale buffers
// of A (288 rows and 32 rows of room for the extra rows' 64-lane load) and B
constexpr int kLdsOps = kBufs * (kLdsA + kLdsB);
constexpr int kLdsSA = kSBuf * (BMX + 32) * 16;
constexpr int kLdsSB = kSBuf * BNT * 16;
constexpr int kLdsAll = kLdsOps + kLdsSA + kLdsSB;

// One workgroup's tile of the GEMM p; bid is its index among p's workgroups
// (see tile_of), lds its kLdsAll bytes of LDS (1 KB aligned).
template <int WF, int EPI>
MOE_DEV void gemm2_body(const GemmParams& p, uint8_t* lds, int bid) {
  constexpr bool MX = WF == W_MXFP8;
  uint8_t* const smem = lds;
  auto& sSA = *reinterpret_cast<uint8_t(*)[kSBuf][(BMX + 32) * 16]>(lds + kLdsOps);
  auto& sSB = *reinterpret_cast<uint8_t(*)[kSBuf][BNT * 16]>(lds + kLdsOps + kLdsSA);


  const int tid = threadIdx.x;
  int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  int g = lane >> 5, l32 = lane & 31;
  constexpr int nper = EPI == EPI_GATEUP ? BNT / 2 : BNT;  // output columns per tile
  const int KS = (EPI == EPI_F32 && p.ksplit > 1) ? p.ksplit : 1;
  const Tile tl = tile_of(p, BM, nper, KS, bid);
  if (!tl.valid) return;
  const int e = tl.e, m0 = tl.m0, n0 = tl.n0, seg0 = tl.seg0, mrows = tl.mrows, kz = tl.kz;
  const int K = p.K, N = p.N;
  const int np_all = K * esz<WF>() / RB;
  const int kp0 = int(long(np_all) * kz / KS), kp1 = int(long(np_all) * (kz + 1) / KS);
  const int npair = kp1 - kp0;  // step pairs of this slice, starting at pair kp0
  if (npair <= 0) return;
  const int nk = 2 * npair;
  const uint32_t lda_b = uint32_t(p.lda) * esz<WF>();
  const uint32_t ldb_b = uint32_t(K) * esz<WF>();

  const int* a_map = p.a_map;
  const int a_div = p.a_div;
  const int rbase = seg0 + m0, rlast = mrows - 1;
#define PHYS_ROW(rl) uint32_t(a_map ? a_map[rbase + min((rl), rlast)] / a_div : rbase + min((rl), rlast))

  // ---------------------------------------------------------- load sources
  // A: wave w loads tile rows [64w, 64w+64) as 8 blocks of 8; lane L fetches
  // row 8k + L/8 of block k, chunk (L%8) ^ ((row>>1)&7).  Blocks wholly past
  // the segment's rows are not loaded (their MFMA rows are never stored).
  const uint8_t* a_base = uniform_ptr(p.A);
  uint32_t oa[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int r = 64 * wave + 8 * k + (lane >> 3);
    oa[k] = PHYS_ROW(r) * lda_b + (((lane & 7) ^ ((r >> 1) & 7)) << 4);
  }
  const int na_blk = min(max((mrows - 64 * wave + 7) / 8, 0), 8);
  // the extra rows: wave w loads tile rows 256 + 8w + [0, 8)
  uint32_t oax;
  {
    const int r = BM + 8 * wave + (lane >> 3);
    oax = PHYS_ROW(r) * lda_b + (((lane & 7) ^ ((r >> 1) & 7)) << 4);
  }
  const bool ldx = mrows > BM + 8 * wave;  // this wave's extra load holds valid rows
  const bool hasX = mrows > BM;            // the tile has extra rows
  // B: wave w loads tile B rows [64w, 64w+64); for EPI_GATEUP these are gate
  // rows (w even) or up rows (w odd) of intermediate columns n0 + 64 (w/2) + [0, 64)
  // Block k's offset is formed at issue (a few VALU operations among the
  // MFMAs) rather than kept in a register per block.
  const uint8_t* b_base;
  {
    const void* bsrc = (EPI == EPI_GATEUP && (wave & 1)) ? p.B1 : p.B0;
    b_base = uniform_ptr(static_cast<const uint8_t*>(bsrc) + size_t(e) * p.b_stride * esz<WF>());
  }
  const int brow0 = (EPI == EPI_GATEUP ? n0 + 64 * wn : n0 + 64 * wave) + (lane >> 3);  // block 0's row
  auto ob_of = [&](int k) {  // tile B row t = 64 wave + 8k + L/8: (t >> 1) & 7 = (4k + L/16) & 7
    const int br = EPI == EPI_GATEUP ? brow0 + 8 * k : min(brow0 + 8 * k, N - 1);
    return uint32_t(br) * ldb_b + (((lane & 7) ^ ((4 * k + (lane >> 4)) & 7)) << 4);
  };
  // MX scales: wave w loads the 16 bytes of A rows and B rows [64w, 64w+64) of a group
  const uint8_t* as_base = nullptr;
  const uint8_t* bs_base = nullptr;
  uint32_t oas = 0, obs = 0, oasx = 0;
  if constexpr (MX) {
    as_base = uniform_ptr(p.As);
    oas = PHYS_ROW(64 * wave + lane) * uint32_t(K / 32);
    oasx = PHYS_ROW(BM + lane) * uint32_t(K / 32);  // wave 0 loads the extra rows' scales
    const void* ssrc = (EPI == EPI_GATEUP && (wave & 1)) ? p.B1s : p.B0s;
    bs_base = uniform_ptr(static_cast<const uint8_t*>(ssrc) + size_t(e) * p.bs_stride);
    const int br = EPI == EPI_GATEUP ? n0 + 64 * wn + lane : min(n0 + 64 * wave + lane, N - 1);
    obs = uint32_t(br) * uint32_t(K / 32);
  }
#undef PHYS_ROW

  const uint32_t lds_a0 = lds_addr(smem), lds_b0 = lds_a0 + kBufs * kLdsA;
  const int ngroups = (nk + kSG - 1) / kSG;
  // load d of pair q into buffer q % 2.  The steady-state waits drain every
  // tile load, so loads past the last pair and of A blocks past the rows are
  // skipped there; the prologue (full) issues all 16, clamped to the last
  // pair, which keeps its wait count exact.
  auto tile_dma = [&](int d, int q, bool full) {
    if (!full && (q >= npair || (d < 8 && d >= na_blk))) return;  // (d == 16: see below)
    const int buf = q & 1, qq = min(q, npair - 1) + kp0;
    if (d == 16) {
      if (!full && !ldx) return;
      dma16(oax, a_base + size_t(qq) * RB, lds_a0 + buf * kLdsA + (BM + 8 * wave) * RB);
    } else if (d < 8) {
      dma16(oa[d], a_base + size_t(qq) * RB, lds_a0 + buf * kLdsA + (64 * wave + 8 * d) * RB);
    } else {
      dma16(ob_of(d - 8), b_base + size_t(qq) * RB, lds_b0 + buf * kLdsB + (64 * wave + 8 * (d - 8)) * RB);
    }
  };
  // scale group q (clamped) into buffer q % 2: 2 loads per wave, 3 in wave 0
  auto scale_dma = [&](int q) {
    if constexpr (MX) {
      const int qq = min(q, ngroups - 1), buf = q % kSBuf;
      dma16(oas, as_base + 16 * qq, lds_addr(&sSA[buf][64 * wave * 16]));
      dma16(obs, bs_base + 16 * qq, lds_addr(&sSB[buf][64 * wave * 16]));
      if (wave == 0) dma16(oasx, as_base + 16 * qq, lds_addr(&sSA[buf][BM * 16]));
    }
  };
  // wait for every load but the scale loads issued last
  auto wait_but_scales = [&]() {
    if (wave == 0)
      wait_vm<3>();
    else
      wait_vm<2>();
  };

  // LDS operand reads: block i of the lane's rows, chunks 4h+g and 4h+2+g
  const int f = (l32 >> 1) & 7;
  // the wave's A row blocks interleave with the other row half's: block i
  // covers tile rows 64 i + 32 wm + [0, 32), so a partial tile's blocks are
  // shared by both halves
  const int rowA = (32 * wm + l32) * RB, rowB = (128 * wn + l32) * RB, rowX = (BM + l32) * RB;
  const int srowA = (32 * wm + l32) * 16 + g, srowB = (128 * wn + l32) * 16 + g, srowX = (BM + l32) * 16 + g;
  // A buffer, B buffer, the two chunk offsets and the scale byte of step t
  struct StepAddr {
    const uint8_t *As, *Bs;
    int colo0, colo1, sbuf, byte;
  };
  auto addr_of = [&](int t) {
    const int buf = (t >> 1) & 1, h = t & 1;
    return StepAddr{smem + buf * kLdsA, smem + kBufs * kLdsA + buf * kLdsB, ((4 * h + g) ^ f) << 4,
                    ((4 * h + 2 + g) ^ f) << 4, (t / kSG) % kSBuf, 2 * (t % kSG)};
  };
  auto rd = [&](const uint8_t* base, int hi, const StepAddr& sa) {
    return *reinterpret_cast<const i32x4*>(base + (hi ? sa.colo1 : sa.colo0));
  };
  // double-buffered read r of step t's operands
  constexpr int ND = 10 + (MX ? 5 : 0);
  auto read_dbl = [&](int r, Frag& fr, int t) {
    const StepAddr sa = addr_of(t);
    if (r < 8) {
      const i32x4 v = rd(sa.As + rowA + 64 * RB * (r / 2), r & 1, sa);
      if (r & 1)
        fr.a[r / 2].hi = v;
      else
        fr.a[r / 2].lo = v;
    } else if (r < 10) {
      const i32x4 v = rd(sa.Bs + rowB + 32 * RB * (3 ^ wm), r & 1, sa);
      if (r & 1)
        fr.b3.hi = v;
      else
        fr.b3.lo = v;
    } else if constexpr (MX) {
      if (r < 14)
        fr.sa[r - 10] = sSA[sa.sbuf][srowA + 64 * 16 * (r - 10) + sa.byte];
      else
        fr.sb3 = sSB[sa.sbuf][srowB + 32 * 16 * (3 ^ wm) + sa.byte];
    }
  };
  // single-buffered reads of B slot j (and, with slot 2, the extra block) for step t
  auto read_single = [&](int j, Single& sg, int t) {
    const StepAddr sa = addr_of(t);
    sg.b[j].lo = rd(sa.Bs + rowB + 32 * RB * (j ^ wm), 0, sa);
    sg.b[j].hi = rd(sa.Bs + rowB + 32 * RB * (j ^ wm), 1, sa);
    if constexpr (MX) sg.sb[j] = sSB[sa.sbuf][srowB + 32 * 16 * (j ^ wm) + sa.byte];
    if (j == 2 && hasX) {
      sg.ax.lo = rd(sa.As + rowX, 0, sa);
      sg.ax.hi = rd(sa.As + rowX, 1, sa);
      if constexpr (MX) sg.sax = sSA[sa.sbuf][srowX + sa.byte];
    }
  };

  // this wave's blocks that hold valid rows (block i is tile block 2 i + wm): blocks at or past nI are skipped
  const int nI = min(max(((mrows + 31) / 32 - wm + 1) / 2, 0), 4);
  f32x16 acc[4][4], accx[2];  // accx[x]: the extra block against register slot 2x
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int r = 0; r < 16; ++r) accx[x][r] = 0.f;
  // One MFMA: block (i, slot j) or the extra block against slot 2x, K half q
  // (bf16: two per block per step).  In the first step each accumulator's
  // first MFMA starts from zero.
  constexpr int QN = MX ? 1 : 2;   // MFMAs per block per step
  constexpr int NM = 18 * QN;      // MFMA slots per step: 16 blocks + 2 extra
  auto mfma_main = [&](int i, int j, int q, const Frag& cur, const Single& sg, auto first_t) {
    if (i >= nI) return;
    const i32x8& b = j == 3 ? cur.b3 : sg.b[j];
    f32x16 c = acc[i][j];
    if (decltype(first_t)::value && q == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) c[r] = 0.f;
    }
    if constexpr (MX) {
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cur.a[i], b, c, 0, 0, 0, int(cur.sa[i]), 0,
                                                                  int(j == 3 ? cur.sb3 : sg.sb[j]));
    } else {
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16(q ? cur.a[i].hi : cur.a[i].lo),
                                                          as_bf16(q ? b.hi : b.lo), c, 0, 0, 0);
    }
  };
  auto mfma_x = [&](int x, int q, const Single& sg, auto first_t) {
    if (!hasX) return;
    f32x16 c = accx[x];
    if (decltype(first_t)::value && q == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) c[r] = 0.f;
    }
    if constexpr (MX) {
      accx[x] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(sg.ax, sg.b[2 * x], c, 0, 0, 0, int(sg.sax), 0,
                                                                int(sg.sb[2 * x]));
    } else {
      accx[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16(q ? sg.ax.hi : sg.ax.lo),
                                                        as_bf16(q ? sg.b[2 * x].hi : sg.b[2 * x].lo), c, 0, 0, 0);
    }
  };

  // step s: the MFMAs on cur and sg (slot by slot: the 4 blocks of slot j,
  // after slots 0 and 2 the extra block), with the double-buffered reads of
  // step s+1 into nxt among the first half of them and each single-buffered
  // slot re-read for step s+1 after its last MFMA.  An odd step s = 2q+1 first
  // waits for pair q+1 (read from step s on) and then, pair q's buffer being
  // released by every wave, issues the loads of pair q+2 into it, one per
  // MFMA.  MX scale groups are loaded at the steps = 0 mod 8.  Loads complete
  // in issue order, so the wait leaves out exactly the scale loads issued at
  // step s-1 (at step 1, the step-1 case is peeled at compile time).
  auto step = [&](int s, Frag& cur, Frag& nxt, Single& sg, auto first_t, auto odd_t, auto step1_t) {
    constexpr bool odd = decltype(odd_t)::value;
    wait_lgkm0();  // this wave no longer reads step s's half
    if constexpr (odd) {
      if constexpr (decltype(step1_t)::value) {
        if constexpr (MX)
          wait_but_scales();
        else
          wait_vm<0>();
      } else if (MX && ((s - 1) & (kSG - 1)) == 0) {
        wait_but_scales();
      } else {
        wait_vm<0>();
      }
      barrier();  // every wave's loads of pair q+1 have landed; pair q's buffer is free
    } else {
      if (MX && (s & (kSG - 1)) == 0) scale_dma(s / kSG + 1);
    }
    const int q2 = (s >> 1) + 2;
    constexpr int NH = NM / 2;
    int m = 0;  // MFMA slot (compile-time after unrolling)
    auto after = [&](int m) {
      if (m < NH) {
#pragma unroll
        for (int r = (m * ND) / NH; r < ((m + 1) * ND) / NH; ++r) read_dbl(r, nxt, s + 1);
      }
      if constexpr (odd) {
#pragma unroll
        for (int d = (m * kDPP) / NM; d < ((m + 1) * kDPP) / NM; ++d) tile_dma(d, q2, false);
      }
    };
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int q = 0; q < QN; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          mfma_main(i, j, q, cur, sg, first_t);
          __builtin_amdgcn_sched_barrier(0);
          after(m++);
          __builtin_amdgcn_sched_barrier(0);
        }
      if (j == 0 || j == 2) {
#pragma unroll
        for (int q = 0; q < QN; ++q) {
          mfma_x(j / 2, q, sg, first_t);
          __builtin_amdgcn_sched_barrier(0);
          after(m++);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (j < 3) {
        read_single(j, sg, s + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // ------------------------------------------------------------ main loop
  Frag f0, f1;
  Single sg;
  if constexpr (MX) scale_dma(0);
#pragma unroll
  for (int q = 0; q < kBufs; ++q)
#pragma unroll
    for (int d = 0; d < kDPP; ++d) tile_dma(d, q, true);
  wait_vm<kDPP>();  // pair 0 and scale group 0 (the loads of pair 1 may be in flight)
  barrier();
#pragma unroll
  for (int r = 0; r < ND; ++r) read_dbl(r, f0, 0);
#pragma unroll
  for (int j = 0; j < 3; ++j) read_single(j, sg, 0);
  const std::false_type no{};
  const std::true_type yes{};
  step(0, f0, f1, sg, yes, no, no);
  step(1, f1, f0, sg, no, yes, yes);  // nk >= 2
  for (int s = 2; s + 1 < nk; s += 2) {  // nk is even: steps come in (even, odd) pairs
    step(s, f0, f1, sg, no, no, no);
    step(s + 1, f1, f0, sg, no, yes, no);
  }
  wait_vm<0>();
  wait_lgkm0();
  barrier();  // the buffers are free for the epilogue

  // ------------------------------------------------------------ epilogue
  // lane l holds column l%32 of each 32x32 block, rows 8(r/4) + 4(l/32) + r%4.
  // The lane index is re-derived here behind an empty asm, so the compiler
  // cannot hoist the epilogue's per-lane addresses above the K loop, where
  // they would hold registers through it.
  {
    int l = lane;
    asm volatile("" : "+v"(l));
    lane = l;
    g = l >> 5;
    l32 = l & 31;
  }
  if constexpr (EPI == EPI_GATEUP) {
    // Stage the wave's h (128 rows x 64 columns, fp32) through LDS, 64 rows
    // at a time, so that each lane finishes whole 32-column row blocks in
    // registers: the MX block maximum without cross-lane reductions, and
    // 16-byte stores.  One wave writes and reads its own region; its LDS
    // operations complete in order.
    constexpr int RSF = 68;  // floats per staged row (64 + 4: conflict-free 16-byte reads)
    float* wsf = reinterpret_cast<float*>(smem) + wave * (64 * RSF);
    const int cb = n0 + 64 * wn;  // first h column of this wave
    const int omode = p.C_f32 ? 0 : (p.out_afmt == A_NONE ? 1 : 2);
    // store 32 consecutive h values of tile row rl from column col
    auto store_h = [&](int rl, int col, const f32x4 (&v)[8]) {
      const size_t orow = size_t(seg0 + m0 + rl);
      if (omode == 0) {
#pragma unroll
        for (int q = 0; q < 8; ++q) *reinterpret_cast<f32x4*>(p.C_f32 + orow * p.ldc + col + 4 * q) = v[q];
      } else if (omode == 1) {
        uint16_t* dst = static_cast<uint16_t*>(p.C) + orow * p.ldc + col;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          i32x4 o;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const f32x4& x = v[2 * q + t / 2];
            const int c = 2 * (t & 1);
            o[t] = int(uint32_t(f32_to_bf16(x[c])) | (uint32_t(f32_to_bf16(x[c + 1])) << 16));
          }
          *reinterpret_cast<i32x4*>(dst + 8 * q) = o;
        }
      } else {  // MXFP8 1x32: this lane's 32 values are one block
        float amax = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q)
          amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[q][0]), fabsf(v[q][1])), fmaxf(fabsf(v[q][2]), fabsf(v[q][3]))));
        const int xe = mx_exponent(amax);
        uint8_t* dst = static_cast<uint8_t*>(p.C) + orow * p.ldc + col;
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          i32x4 o;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const f32x4& x = v[4 * q2 + t];
            o[t] = int(e4m3x4_sat(__builtin_amdgcn_ldexpf(x[0], -xe), __builtin_amdgcn_ldexpf(x[1], -xe),
                                  __builtin_amdgcn_ldexpf(x[2], -xe), __builtin_amdgcn_ldexpf(x[3], -xe)));
          }
          *reinterpret_cast<i32x4*>(dst + 16 * q2) = o;
        }
        static_cast<uint8_t*>(p.Cs)[orow * (N / 32) + col / 32] = uint8_t(xe + 127);
      }
    };
    // the extra rows: h of tile rows 256-287, the wave's column block wm;
    // lane l < 32 finishes row 256 + l
    if (hasX) {  // first, so the extra accumulators are free before the main blocks
#pragma unroll
      for (int r = 0; r < 16; ++r) wsf[(8 * (r >> 2) + 4 * g + (r & 3)) * RSF + l32] = silu(accx[0][r]) * accx[1][r];
      f32x4 v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = *reinterpret_cast<const f32x4*>(wsf + l32 * RSF + 4 * q);
      if (lane < 32 && BM + lane < mrows) store_h(BM + lane, cb + 32 * wm, v);
    }
    // register slot jj holds the wave's h column block jj ^ wm
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            wsf[(32 * ii + 8 * (r >> 2) + 4 * g + (r & 3)) * RSF + 32 * (jj ^ wm) + l32] =
                silu(acc[2 * h + ii][jj][r]) * acc[2 * h + ii][jj + 2][r];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int b = lane + 64 * k, row = b >> 1, half = b & 1;
        const int rl = 128 * h + 64 * (row >> 5) + 32 * wm + (row & 31);  // staged block 2 h + row / 32
        f32x4 v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = *reinterpret_cast<const f32x4*>(wsf + row * RSF + 32 * half + 4 * q);
        if (rl < mrows) store_h(rl, cb + 32 * half, v);
      }
    }
  } else {
    // stage the wave's 128 x 128 block through LDS, one 32-row block at a
    // time (at most 4 x 32 x 528 bytes), and store whole 16-byte row chunks
    constexpr int ES = EPI == EPI_F32 ? 4 : 2;
    constexpr int RS = 128 * ES + 16;  // LDS row stride (bytes), padded
    constexpr int CPR = 128 * ES / 16;  // 16-byte chunks per row
    uint8_t* ws = smem + wave * (32 * RS);
    const int cw = n0 + 128 * wn;  // first output column of this wave
    // stage one 32x32 block for column block cb
    auto stage = [&](const f32x16& a, int cb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        uint8_t* d = ws + (8 * (r >> 2) + 4 * g + (r & 3)) * RS + (32 * cb + l32) * ES;
        if (EPI == EPI_F32)
          *reinterpret_cast<float*>(d) = a[r];
        else
          *reinterpret_cast<uint16_t*>(d) = f32_to_bf16(a[r]);
      }
    };
    // store the staged rows row0 + [0, 32) (the column blocks in cmask)
    auto store_rows = [&](int row0, int cmask) {
#pragma unroll 4
      for (int c = lane; c < 32 * CPR; c += 64) {
        const int rl = c / CPR, cc = c % CPR;
        const int row = row0 + rl;
        if (row >= mrows || !((cmask >> (cc * (16 / ES) / 32)) & 1)) continue;
        const int col = cw + cc * (16 / ES);
        const i32x4 v = *reinterpret_cast<const i32x4*>(ws + rl * RS + cc * 16);
        const size_t orow = size_t(seg0 + m0 + row);
        uint8_t* dst = static_cast<uint8_t*>(p.C) + (size_t(kz) * p.c_split + orow * p.ldc + col) * ES;
        if (col + 16 / ES <= N) {
          *reinterpret_cast<i32x4*>(dst) = v;
        } else {
          for (int q = 0; q < 16 / ES && col + q < N; ++q)
            for (int b = 0; b < ES; ++b) dst[q * ES + b] = reinterpret_cast<const uint8_t*>(&v)[q * ES + b];
        }
      }
    };
    if (hasX) {  // the extra rows: column blocks wm (slot 0) and 2 + wm (slot 2)
      stage(accx[0], wm);
      stage(accx[1], 2 + wm);
      store_rows(BM, (1 << wm) | (4 << wm));
    }
    // register slot j holds the wave's column block j ^ wm
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) stage(acc[i][j], j ^ wm);
      store_rows(64 * i + 32 * wm, 0xf);
    }
  }
}

template <int WF, int EPI>
__global__ __launch_bounds__(256) void gemm2_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsAll];
  gemm2_body<WF, EPI>(p, lds, int(blockIdx.x));
}

// Two GEMMs in one launch: workgroups [0, n1) run p1, the rest p2 (n1 is a
// multiple of 8, so both keep their XCD-aware tile order).  A GEMM whose
// tiles leave part of the last wave idle then shares that wave with the
// other's tiles instead of running after it.
template <int WF1, int EPI1, int WF2, int EPI2>
__global__ __launch_bounds__(256) void gemm2_dual_kernel(GemmParams p1, int n1, GemmParams p2) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsAll];
  if (int(blockIdx.x) < n1)
    gemm2_body<WF1, EPI1>(p1, lds, int(blockIdx.x));
  else
    gemm2_body<WF2, EPI2>(p2, lds, int(blockIdx.x) - n1);
}

template <int WF>
hipError_t launch_epi(int epi, const GemmParams& p, dim3 grid, hipStream_t s) {
  switch (epi) {
    case EPI_F32: hipLaunchKernelGGL((gemm2_kernel<WF, EPI_F32>), grid, dim3(256), 0, s, p); break;
    case EPI_BF16: hipLaunchKernelGGL((gemm2_kernel<WF, EPI_BF16>), grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((gemm2_kernel<WF, EPI_GATEUP>), grid, dim3(256), 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm2_dual(int wf1, const GemmParams& p1, int wf2, const GemmParams& p2, hipStream_t s) {
  auto tiles_of = [](int wf, const GemmParams& p) -> long {
    const int ntile = p.tiles ? p.max_tiles : (p.M + BM - 1) / BM;
    if (ntile <= 0) return 0;
    const long es = wf == W_BF16 ? 2 : 1;
    const long a_rows = p.a_map ? (long(p.M) + p.a_div - 1) / p.a_div : long(p.M);
    if (a_rows * p.lda * es >= (1L << 32) || long(p.N) * p.K * es >= (1L << 32)) return -1;
    return (long(ntile) * ((p.N + BNT - 1) / BNT) + 7) / 8 * 8;
  };
  if (!gemm2_serves(wf1, p1.K, EPI_BF16, A_NONE, p1.ksplit) || !gemm2_serves(wf2, p2.K, EPI_BF16, A_NONE, p2.ksplit))
    return hipErrorInvalidValue;
  const long n1 = tiles_of(wf1, p1), n2 = tiles_of(wf2, p2);
  if (n1 < 0 || n2 < 0) return hipErrorInvalidValue;
  if (n1 + n2 == 0) return hipSuccess;
  const dim3 grid(unsigned(n1 + n2));
  const int n1i = int(n1);
  if (wf1 == W_BF16 && wf2 == W_MXFP8)
    hipLaunchKernelGGL((gemm2_dual_kernel<W_BF16, EPI_BF16, W_MXFP8, EPI_BF16>), grid, dim3(256), 0, s, p1, n1i, p2);
  else if (wf1 == W_MXFP8 && wf2 == W_MXFP8)
    hipLaunchKernelGGL((gemm2_dual_kernel<W_MXFP8, EPI_BF16, W_MXFP8, EPI_BF16>), grid, dim3(256), 0, s, p1, n1i, p2);
  else if (wf1 == W_BF16 && wf2 == W_BF16)
    hipLaunchKernelGGL((gemm2_dual_kernel<W_BF16, EPI_BF16, W_BF16, EPI_BF16>), grid, dim3(256), 0, s, p1, n1i, p2);
  else
    hipLaunchKernelGGL((gemm2_dual_kernel<W_MXFP8, EPI_BF16, W_BF16, EPI_BF16>), grid, dim3(256), 0, s, p1, n1i, p2);
  return hipGetLastError();
}

bool gemm2_serves(int wfmt, int K, int epi, int out_afmt, int ksplit) {
  if (wfmt == W_BF16) return K % 64 == 0 && (epi != EPI_GATEUP || out_afmt == A_NONE);
  if (wfmt == W_MXFP8) return K % 512 == 0 && ksplit <= 1 && (epi != EPI_GATEUP || out_afmt != A_FP8_1X128);
  return false;
}

bool gemm2_chosen(int wfmt, int epi, const GemmParams& p) {
  if (p.tiles) return p.bm == kGemm2BM;
  if (!gemm2_serves(wfmt, p.K, epi, p.C_f32 ? A_NONE : p.out_afmt, p.ksplit)) return false;
  const int nper = epi == EPI_GATEUP ? BNT / 2 : BNT;
  const long t2 = long((p.M + BM - 1) / BM) * ((p.N + nper - 1) / nper) * std::max(p.ksplit, 1);
  return t2 >= 224;  // about the CU count: fewer large tiles would leave CUs idle
}

hipError_t launch_gemm2(int wfmt, int epi, const GemmParams& p, hipStream_t s) {
  const int ntile = p.tiles ? p.max_tiles : (p.M + BM - 1) / BM;
  if (ntile <= 0) return hipSuccess;
  if (!gemm2_serves(wfmt, p.K, epi, p.C_f32 ? A_NONE : p.out_afmt, p.ksplit)) return hipErrorInvalidValue;
  // the kernels address A rows and one group's B rows with 32-bit byte offsets
  const long es = wfmt == W_BF16 ? 2 : 1;
  const long a_rows = p.a_map ? (long(p.M) + p.a_div - 1) / p.a_div : long(p.M);
  if (a_rows * p.lda * es >= (1L << 32) || long(p.N) * p.K * es >= (1L << 32)) return hipErrorInvalidValue;
  const int nper = epi == EPI_GATEUP ? BNT / 2 : BNT;
  const long tiles = long(ntile) * ((p.N + nper - 1) / nper) * (epi == EPI_F32 && p.ksplit > 1 ? p.ksplit : 1);
  const dim3 grid(unsigned((tiles + 7) / 8 * 8));  // the in-kernel schedule maps block b to XCD b % 8
  return wfmt == W_BF16 ? launch_epi<W_BF16>(epi, p, grid, s) : launch_epi<W_MXFP8>(epi, p, grid, s);
}

}  // namespace moe
