// Dispatch of the T*K (token, slot) pairs into per-expert segments, on the
// GPU and without any host round trip (Mixture-of-Kittens, Abstract and
// Figure 1: GPU-side dispatch scheduling, no CPU-GPU synchronisation).
//
// One workgroup of 1024 threads: an LDS histogram, an exclusive scan over
// the experts, then a stable scatter in chunks of 1024 slots.  Within a chunk
// a slot's rank among equal experts comes from wave ballots (an 8-bit
// bit-sliced match) plus the counts of the earlier waves, so the order is the
// flat slot order: integer-only and deterministic.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kMaxE = 256;
constexpr int kWaves = 16;

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
  // scratch[e] = exclusive prefix of ceil(cnt/bm); wave 0 scans, all threads write
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int lane = tid;
    int v[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = lane * 4 + i;
      v[i] = e < E ? (cnt[e] + bm - 1) / bm : 0;
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
    int n = (cnt[e] + bm - 1) / bm, b = scratch[e];
    for (int i = 0; i < n; ++i) {
      tiles[2 * (b + i)] = e;
      tiles[2 * (b + i) + 1] = i * bm;
    }
  }
}

__global__ __launch_bounds__(1024) void permute_kernel(const int* __restrict__ ids, int TK, int E,
                                                       int* __restrict__ offsets, int* __restrict__ perm_src,
                                                       int* __restrict__ inv_pos, int* tiles, int* ntiles,
                                                       int bm) {
  __shared__ int cnt[kMaxE];
  __shared__ int base[kMaxE];
  __shared__ int wcnt[kWaves][kMaxE];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < kMaxE; i += 1024) cnt[i] = 0;
  for (int i = tid; i < kWaves * kMaxE; i += 1024) (&wcnt[0][0])[i] = 0;
  __syncthreads();
  for (int p = tid; p < TK; p += 1024) {
    int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (tid < 64) scan_experts(cnt, E, base, offsets);
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c0 = 0; c0 < TK; c0 += 1024) {
    const int p = c0 + tid;
    int e = p < TK ? ids[p] : -1;
    const bool valid = e >= 0 && e < E;
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (e >> b) & 1;
      uint64_t bb = __ballot(valid && bit);
      m &= bit ? bb : ~bb;
    }
    const int rank = __popcll(m & lt_mask);
    if (valid && rank == 0) wcnt[wave][e] = __popcll(m);
    __syncthreads();
    if (valid) {
      int pos = base[e] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
      perm_src[pos] = p;
      inv_pos[p] = pos;
    } else if (p < TK) {
      inv_pos[p] = -1;
    }
    __syncthreads();
    if (tid < E) {
      int s = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        s += wcnt[w][tid];
        wcnt[w][tid] = 0;
      }
      base[tid] += s;
    }
    __syncthreads();
  }
  if (tiles) write_tiles(cnt, E, bm, tiles, ntiles, &wcnt[0][0]);
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

}  // namespace

hipError_t launch_permute(const int* ids, int TK, int E, int* offsets, int* perm_src, int* inv_pos, int* tiles,
                          int* ntiles, int bm, hipStream_t s) {
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(1024), 0, s, ids, TK, E, offsets, perm_src, inv_pos, tiles,
                     ntiles, bm);
  return hipGetLastError();
}

hipError_t launch_build_tiles(const int* offsets, int E, int rows, int bm, int* tiles, int* ntiles, hipStream_t s) {
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(256), 0, s, offsets, E, rows, bm, tiles, ntiles);
  return hipGetLastError();
}

}  // namespace moe
