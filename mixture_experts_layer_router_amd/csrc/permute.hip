// Dispatch of the T*K (token, slot) pairs into per-expert segments, on the
// GPU and without any host round trip (Mixture-of-Kittens, Abstract and
// Figure 1: GPU-side dispatch scheduling, no CPU-GPU synchronisation).
//
// Two launches over chunks of 1024 slots, one workgroup per chunk: each
// chunk's per-expert counts, then a stable scatter in which every workgroup
// reduces those counts itself (expert totals, the counts of the chunks before
// its own, an exclusive scan over the experts), so no workgroup ever waits for
// another.  Within a wave, the slots of one expert are found with ballots (an
// 8-bit bit-sliced match): the count takes one LDS add per (wave, expert)
// instead of one per slot, and a slot's rank among equal experts is a
// popcount; one 16-lane row per expert turns the waves' counts into each
// wave's first position.  The order is the flat slot order: integer-only and
// deterministic.  A single chunk needs only the second launch.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kMaxE = 256;
constexpr int kWaves = 16;  // one row of 16 lanes covers an expert's per-wave counts
constexpr int kChunk = 1024;  // slots per workgroup, one per thread

MOE_DEV int wave_incl_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

// Exclusive scan of cnt[0..E) into out[0..E] by wave 0 (E <= 256).
MOE_DEV void scan_experts(const int* cnt, int E, int* out_lds, int* out_glob) {
  const int lane = lane_id();
  int v[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int e = lane * 4 + i;
    v[i] = e < E ? cnt[e] : 0;
    sum += v[i];
  }
  int incl = wave_incl_scan(sum);
  int run = incl - sum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int e = lane * 4 + i;
    if (e < E) {
      if (out_lds) out_lds[e] = run;
      if (out_glob) out_glob[e] = run;
    }
    run += v[i];
  }
  if (lane == 63 && out_glob) out_glob[E] = incl;
}

MOE_DEV void write_tiles(const int* cnt, int E, int bm, int* tiles, int* ntiles, int* scratch) {
  // scratch[e] = exclusive prefix of the experts' tile counts; wave 0 scans, all threads write
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int lane = tid;
    int v[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = lane * 4 + i;
      v[i] = e < E ? tile_count(cnt[e], bm) : 0;
      sum += v[i];
    }
    int incl = wave_incl_scan(sum);
    int run = incl - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = lane * 4 + i;
      if (e < E) scratch[e] = run;
      run += v[i];
    }
    if (lane == 63) ntiles[0] = incl;
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    int step;
    const int n = tile_split(cnt[e], bm, &step), b = scratch[e];
    for (int i = 0; i < n; ++i) {
      tiles[2 * (b + i)] = e;
      tiles[2 * (b + i) + 1] = i * step;
    }
  }
}

// inclusive prefix sum over each row of 16 lanes (DPP row shifts; lanes
// shifted in from outside the row add 0)
MOE_DEV int row16_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  return v;
}

// lanes of this wave holding the same valid expert as this lane (an 8-bit
// bit-sliced match of ballots), as a lane mask
MOE_DEV uint64_t same_expert_lanes(int e, bool valid) {
  uint64_t m = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bb = __ballot(valid && bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

// Per-chunk expert counts: chunk c (1024 slots) writes hist[c][0..E).
__global__ __launch_bounds__(1024) void permute_count_kernel(const int* __restrict__ ids, int TK, int E,
                                                             int* __restrict__ hist) {
  __shared__ int cnt[kMaxE];
  const int tid = threadIdx.x, lane = tid & 63, c = blockIdx.x;
  const int p = c * kChunk + tid;
  const int e = p < TK ? ids[p] : -1;
  const bool valid = e >= 0 && e < E;
  if (tid < kMaxE) cnt[tid] = 0;
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const uint64_t m = same_expert_lanes(e, valid);
  if (valid && __popcll(m & lt_mask) == 0) atomicAdd(&cnt[e], __popcll(m));
  __syncthreads();
  for (int i = tid; i < E; i += kChunk) hist[size_t(c) * E + i] = cnt[i];
}

// Stable scatter of one chunk of per_wg slots.  The counts come in hist rows
// of `fine` slots each (per_wg is a multiple of fine, at most 1024): every
// workgroup reduces them itself (the expert totals, and the counts of the
// rows before its own chunk), so no workgroup waits for another; workgroup 0
// also writes the offsets and the tile list.  With a single chunk (hist NULL)
// the counts come from the chunk.
__global__ __launch_bounds__(1024) void permute_scatter_kernel(const int* __restrict__ ids, int TK, int E,
                                                               const int* __restrict__ hist, int nchunks, int fine,
                                                               int per_wg, int* __restrict__ offsets,
                                                               int* __restrict__ perm_src, int* __restrict__ inv_pos,
                                                               int* tiles, int* ntiles, int bm) {
  __shared__ int part[2][4][kMaxE];    // [before, total][quarter][expert]
  __shared__ int tot[kMaxE];           // slots of each expert
  __shared__ int first[kMaxE];         // position of this chunk's first slot of each expert
  __shared__ int wcnt[kMaxE][kWaves];  // per (expert, wave): count, then first position
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, c = blockIdx.x;
  const int p = c * per_wg + tid;
  const bool mine = tid < per_wg && p < TK;
  const int e = mine ? ids[p] : -1;
  const bool valid = e >= 0 && e < E;
  const int rows_before = c * (per_wg / fine);  // hist rows wholly before this chunk
  for (int i = tid; i < kMaxE * kWaves; i += kChunk) (&wcnt[0][0])[i] = 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const uint64_t m = same_expert_lanes(e, valid);
  const int rank = __popcll(m & lt_mask);
  if (hist) {
    // thread (q, x) sums expert x over the chunks q, q + 4, ...
    const int x = tid & (kMaxE - 1), q = tid >> 8;
    int before = 0, total = 0;
    if (x < E) {
#pragma unroll 4
      for (int cc = q; cc < nchunks; cc += 4) {
        const int v = hist[size_t(cc) * E + x];
        total += v;
        before += cc < rows_before ? v : 0;
      }
    }
    part[0][q][x] = before;
    part[1][q][x] = total;
    __syncthreads();
    if (tid < kMaxE) {
      tot[tid] = part[1][0][tid] + part[1][1][tid] + part[1][2][tid] + part[1][3][tid];
      first[tid] = part[0][0][tid] + part[0][1][tid] + part[0][2][tid] + part[0][3][tid];
    }
  } else {
    if (tid < kMaxE) tot[tid] = first[tid] = 0;
    __syncthreads();
    if (valid && rank == 0) atomicAdd(&tot[e], __popcll(m));
  }
  __syncthreads();
  // expert offsets (exclusive scan of the totals) into part[0][0]
  if (tid < 64) scan_experts(tot, E, &part[0][0][0], c == 0 ? offsets : nullptr);
  if (valid && rank == 0) wcnt[e][wave] = __popcll(m);
  __syncthreads();
  // one 16-lane row per expert: the waves' counts, scanned across the row
  for (int i = tid; i < E * kWaves; i += kChunk) {
    const int x = i / kWaves;
    const int n = wcnt[x][i % kWaves];
    wcnt[x][i % kWaves] = part[0][0][x] + first[x] + row16_incl_scan(n) - n;
  }
  __syncthreads();
  if (valid) {
    const int pos = wcnt[e][wave] + rank;
    perm_src[pos] = p;
    inv_pos[p] = pos;
  } else if (mine) {
    inv_pos[p] = -1;
  }
  if (c == 0 && tiles) write_tiles(tot, E, bm, tiles, ntiles, &part[1][0][0]);
}

__global__ __launch_bounds__(256) void build_tiles_kernel(const int* __restrict__ offsets, int E, int rows, int bm,
                                                          int* tiles, int* ntiles) {
  __shared__ int cnt[kMaxE];
  __shared__ int scratch[kMaxE];
  // counts from offsets clamped to [0, rows]: at most ceil(rows/bm) + E tiles
  for (int e = threadIdx.x; e < E; e += 256) {
    const int a = min(max(offsets[e], 0), rows);
    const int b = min(max(offsets[e + 1], a), rows);
    cnt[e] = b - a;
  }
  __syncthreads();
  write_tiles(cnt, E, bm, tiles, ntiles, scratch);
}

// Debug check of a dispatch (one workgroup, reads only, never traps): ORs
// into *flags bit 0 if offsets[0] != 0 or offsets decrease, bit 1 if
// offsets[E] != TK, bit 2 for an id outside [0, E), bit 3 if perm_src is not
// a bijection of [0, TK) with inv_pos its inverse, bit 4 if a position holds
// a slot of another expert or a segment is not in ascending slot order, bit
// 5 if the tile list does not cover each segment in order with
// tile_count(cnt, bm) tiles at the row step tile_step(cnt, bm).
__global__ __launch_bounds__(256) void validate_dispatch_kernel(const int* __restrict__ ids, int TK, int E,
                                                                const int* __restrict__ off,
                                                                const int* __restrict__ perm,
                                                                const int* __restrict__ inv,
                                                                const int* __restrict__ tiles,
                                                                const int* __restrict__ ntiles, int maxt, int bm,
                                                                int* flags) {
  __shared__ int s_bits, s_want;
  const int tid = threadIdx.x;
  if (tid == 0) s_bits = s_want = 0;
  __syncthreads();
  int bits = 0, want = 0;
  for (int e = tid; e <= E; e += 256) {
    if (e == 0 && off[0] != 0) bits |= 1;
    if (e < E && off[e] > off[e + 1]) bits |= 1;
    if (e == E && off[E] != TK) bits |= 2;
    if (e < E) want += tile_count(max(off[e + 1] - off[e], 0), bm);
  }
  for (int i = tid; i < TK; i += 256) {
    const int id = ids[i];
    if (id < 0 || id >= E) bits |= 4;
    const int p = perm[i];
    if (p < 0 || p >= TK || inv[p] != i) {
      bits |= 8;
      continue;
    }
    int lo = 0, hi = E - 1;  // the segment holding position i: largest e with off[e] <= i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    if (ids[p] != lo) bits |= 16;
    if (i + 1 < off[lo + 1] && i + 1 < TK && perm[i + 1] <= p) bits |= 16;
  }
  const int n_raw = ntiles[0], n = min(max(n_raw, 0), maxt);  // the list holds at most maxt entries
  if (tid == 0 && n != n_raw) bits |= 32;
  for (int j = tid; j < n; j += 256) {
    const int e = tiles[2 * j], m0 = tiles[2 * j + 1];
    if (e < 0 || e >= E) {
      bits |= 32;
      continue;
    }
    const int cnt = off[e + 1] - off[e], step = tile_step(cnt, bm);
    const bool first = j == 0 || tiles[2 * (j - 1)] != e;
    if (m0 < 0 || m0 >= cnt || (first ? m0 != 0 : m0 != tiles[2 * (j - 1) + 1] + step)) bits |= 32;
  }
  if (bits) atomicOr(&s_bits, bits);
  if (want) atomicAdd(&s_want, want);
  __syncthreads();
  if (tid == 0) {
    if (s_want != n) s_bits |= 32;
    if (s_bits) atomicOr(flags, s_bits);
  }
}

}  // namespace

hipError_t launch_permute(const int* ids, int TK, int E, int* hist, int* offsets, int* perm_src, int* inv_pos,
                          int* tiles, int* ntiles, int bm, hipStream_t s) {
  const int nchunks = (TK + kChunk - 1) / kChunk;
  if (nchunks > 1) {
    hipLaunchKernelGGL(permute_count_kernel, dim3(nchunks), dim3(kChunk), 0, s, ids, TK, E, hist);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(nchunks), dim3(kChunk), 0, s, ids, TK, E,
                     nchunks > 1 ? hist : nullptr, nchunks, kChunk, kChunk, offsets, perm_src, inv_pos, tiles, ntiles,
                     bm);
  return hipGetLastError();
}

hipError_t launch_permute_scatter(const int* ids, int TK, int E, const int* hist, int fine, int* offsets,
                                  int* perm_src, int* inv_pos, int* tiles, int* ntiles, int bm, hipStream_t s) {
  if (TK <= 0) return hipSuccess;
  if (fine <= 0 || fine > kChunk) return hipErrorInvalidValue;
  const int per_wg = fine * (kChunk / fine);
  const int nwg = (TK + per_wg - 1) / per_wg, nrows = (TK + fine - 1) / fine;
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(nwg), dim3(kChunk), 0, s, ids, TK, E, hist, nrows, fine, per_wg,
                     offsets, perm_src, inv_pos, tiles, ntiles, bm);
  return hipGetLastError();
}

hipError_t launch_validate_dispatch(const int* ids, int TK, int E, const int* offsets, const int* perm, const int* inv,
                                   const int* tiles, const int* ntiles, int maxt, int bm, int* flags, hipStream_t s) {
  hipLaunchKernelGGL(validate_dispatch_kernel, dim3(1), dim3(256), 0, s, ids, TK, E, offsets, perm, inv, tiles, ntiles,
                     maxt, bm, flags);
  return hipGetLastError();
}

hipError_t launch_build_tiles(const int* offsets, int E, int rows, int bm, int* tiles, int* ntiles, hipStream_t s) {
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(256), 0, s, offsets, E, rows, bm, tiles, ntiles);
  return hipGetLastError();
}

}  // namespace moe
