// Dispatch of the T*K (token, slot) pairs into per-expert segments, on the
// GPU and without any host round trip (Mixture-of-Kittens, Abstract and
// Figure 1: GPU-side dispatch scheduling, no CPU-GPU synchronisation).
//
// One workgroup of 1024 threads: a histogram, an exclusive scan over the
// experts, then a stable scatter in chunks of 1024 slots.  Within a wave, the
// slots of one expert are found with ballots (an 8-bit bit-sliced match), so
// the histogram takes one LDS add per (wave, expert) instead of one per slot,
// and a slot's rank among equal experts is a popcount; per chunk, one thread
// per expert turns the waves' counts into each wave's first position.  The
// order is the flat slot order: integer-only and deterministic.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kMaxE = 256;
constexpr int kWaves = 16;  // one row of 16 lanes covers an expert's per-wave counts
constexpr int kGroup = 24;  // chunks of 1024 slots whose ids a thread holds at once

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

// Workgroup barrier for LDS traffic only: __syncthreads() also waits for the
// thread's outstanding global stores (a workgroup-scope release), which in the
// chunk loop would put the store latency of every chunk on the critical path.
MOE_DEV void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
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

__global__ __launch_bounds__(1024) void permute_kernel(const int* __restrict__ ids, int TK, int E,
                                                       int* __restrict__ offsets, int* __restrict__ perm_src,
                                                       int* __restrict__ inv_pos, int* tiles, int* ntiles,
                                                       int bm) {
  __shared__ int cnt[kMaxE];
  __shared__ int base[kMaxE];
  __shared__ int wcnt[kMaxE][kWaves];  // this chunk's count per (expert, wave)
  __shared__ int wpre[kMaxE][kWaves];  // ... and the position of its first slot
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < kMaxE; i += 1024) cnt[i] = 0;
  for (int i = tid; i < kWaves * kMaxE; i += 1024) (&wcnt[0][0])[i] = 0;
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // the slots are taken kGroup chunks of 1024 at a time; a thread loads its
  // ids of the whole group at once (one memory latency, not one per chunk)
  const int nchunks = (TK + 1023) / 1024;
  auto load_group = [&](int g0, int (&idv)[kGroup]) {
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      const int p = (g0 + k) * 1024 + tid;
      idv[k] = (g0 + k < nchunks && p < TK) ? ids[p] : -1;
    }
    // wait for the loads here, in a form the compiler tracks: loads and stores
    // share one counter, and without this the chunk loop would wait for its
    // own scattered stores before every use of an id
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  };
  // histogram: one LDS add per (wave, expert present in the wave's 64 slots)
  for (int g0 = 0; g0 < nchunks; g0 += kGroup) {
    int idv[kGroup];
    load_group(g0, idv);
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      if (g0 + k >= nchunks) break;  // uniform
      const int e = idv[k];
      const bool valid = e >= 0 && e < E;
      const uint64_t m = same_expert_lanes(e, valid);
      if (valid && __popcll(m & lt_mask) == 0) atomicAdd(&cnt[e], __popcll(m));
    }
  }
  __syncthreads();
  if (tid < 64) scan_experts(cnt, E, base, offsets);
  __syncthreads();
  // stable scatter, 1024 slots at a time: a slot's position is its expert's
  // running base, plus the counts of the earlier waves of the chunk, plus its
  // rank among the equal slots of its wave
  for (int g0 = 0; g0 < nchunks; g0 += kGroup) {
    int idv[kGroup];
    load_group(g0, idv);
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      if (g0 + k >= nchunks) break;  // uniform
      const int p = (g0 + k) * 1024 + tid;
      const int e = idv[k];
      const bool valid = e >= 0 && e < E;
      const uint64_t m = same_expert_lanes(e, valid);
      const int rank = __popcll(m & lt_mask);
      if (valid && rank == 0) wcnt[e][wave] = __popcll(m);
      lds_barrier();
      // one 16-lane row per expert: its waves' counts, scanned across the row
      for (int i = tid; i < E * kWaves; i += 1024) {
        const int x = i / kWaves, w = i % kWaves;
        const int n = wcnt[x][w];
        const int incl = row16_incl_scan(n);
        const int b = base[x];
        wpre[x][w] = b + incl - n;
        wcnt[x][w] = 0;
        if (w == kWaves - 1) base[x] = b + incl;
      }
      lds_barrier();
      if (valid) {
        const int pos = wpre[e][wave] + rank;
        perm_src[pos] = p;
        inv_pos[p] = pos;
      } else if (p < TK) {
        inv_pos[p] = -1;
      }
    }
  }
  lds_barrier();
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
