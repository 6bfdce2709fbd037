// Device helpers of the grouped GEMM kernels (gemm.hip, gemm2.hip): direct
// HBM -> LDS loads, wait counters, the workgroup barrier, wave-uniform
// pointers, and the grouped tile schedule.
#pragma once
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace gemm_dev {

template <int N>
using IC = std::integral_constant<int, N>;

template <int WF>
MOE_DEV constexpr int esz() { return WF == W_BF16 ? 2 : 1; }

// Direct-to-LDS loads from base + off: the 64 lanes' data lands at
// lds + 16 l (x4) or + 4 l (x1).  base and lds are wave-uniform.  M0 is
// reserved for this use; nothing else in these kernels reads it.
MOE_DEV void dma16(uint32_t off, const uint8_t* base, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory");
}
MOE_DEV void dma4(uint32_t off, const uint8_t* base, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory");
}
template <int N>
MOE_DEV void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
MOE_DEV void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
MOE_DEV void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
MOE_DEV uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(p)));
}
MOE_DEV const uint8_t* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(v)));
  const uint64_t hi = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(v >> 32)));
  return reinterpret_cast<const uint8_t*>((hi << 32) | lo);
}
MOE_DEV bf16x8 as_bf16(i32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// max over the 32 lanes of each half wave; every lane of the half gets it
MOE_DEV float half_max(float v) {
  v = group_max<16>(v);
  return fmaxf(v, __shfl_xor(v, 16, 64));
}

// One workgroup's tile of the grouped GEMM.  The flat list of (expert,
// n-block, m-tile) tiles (times the K slices) is cut into 8 contiguous
// ranges, one per XCD (blocks are dispatched round robin over the XCDs), so
// the tiles that run together on one XCD share their weight panel (m-tiles of
// the same n-block are adjacent) and their activation panel (same expert).
// Without a tile list (one group of M rows) the list runs over groups of 4
// m-tiles, n-block-major inside a group: the 32 tiles that run together on an
// XCD cover 4 activation panels and 8 weight panels instead of 16 and 2.
struct Tile {
  int e, m0, n0, kz, seg0, mrows;
  bool valid;
};
// bid: the workgroup's index among the launch's workgroups of this GEMM
// (blockIdx.x, or its offset in a launch shared with another GEMM, which
// keeps bid % 8 = blockIdx.x % 8 when that offset is a multiple of 8).
MOE_DEV Tile tile_of(const GemmParams& p, int bm, int nper, int ks, int bid) {
  Tile t{};
  const int NB = (p.N + nper - 1) / nper;
  const int nt_list = p.tiles ? p.ntiles[0] : (p.M + bm - 1) / bm;
  const int T = nt_list * NB * ks;
  const int chunk = (T + 7) / 8;
  int idx = (bid % 8) * chunk + bid / 8;
  if (bid / 8 >= chunk || idx >= T) return t;
  t.kz = idx % ks;  // K slice (split-K: slices of one tile are adjacent)
  idx /= ks;
  int e = 0, nb, m0, step = bm;
  {
    const int pe = idx / NB;  // a tile-list entry of the same expert
    int be = 0, ne = nt_list;
    if (p.tiles) {
      e = p.tiles[2 * pe];
      const int c0 = min(max(p.seg[e], 0), p.M), c1 = min(max(p.seg[e + 1], c0), p.M);
      ne = max(tile_split(c1 - c0, bm, &step), 1);
      be = pe - p.tiles[2 * pe + 1] / step;
    }
    const int local = idx - be * NB;
    if (p.tiles) {  // one expert's m-tiles of an n-block are adjacent
      nb = local / ne;
      m0 = (local % ne) * step;
    } else {  // one group: groups of 4 m-tiles, n-block-major within a group
      const int gm = 4, grp = local / (gm * NB), rest = local - grp * gm * NB;
      const int gsz = min(gm, ne - grp * gm);
      nb = rest / gsz;
      m0 = (grp * gm + rest % gsz) * bm;
    }
  }
  // segment bounds clamped to [0, M] so malformed offsets cannot address outside the rows
  const int seg0 = p.seg ? min(max(p.seg[e], 0), p.M) : 0;
  const int seg1 = p.seg ? min(max(p.seg[e + 1], seg0), p.M) : p.M;
  t.e = e;
  t.m0 = m0;
  t.n0 = nb * nper;
  t.seg0 = seg0;
  t.mrows = min(step, seg1 - seg0 - m0);
  t.valid = t.mrows > 0;
  return t;
}

}  // namespace gemm_dev
}  // namespace moe
