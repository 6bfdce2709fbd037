// Backward pass of the MoE layer (Mixture-of-Kittens, Table 1: the MoE
// layer's backward beside its forward), bf16 weights, unquantised
// activations.  Kernels:
//
//   bwd_gemm_kernel   C (+)= sum_k A(m, k) B(k, n) in bf16 MFMAs, fp32 accumulate,
//                     for the two shapes the backward needs beyond the forward:
//                     NN   rows m of an expert segment (tile list), A[m][k]
//                          row-major, B stored [k][n] (the forward weight read
//                          along its output dimension): dh = dY Wd, dX = dg Wg
//                          + du Wu (two passes), the router's dl Wr;
//                     TN   the reduction runs over an expert's segment rows:
//                          A(m, k) = P[k][m], B(k, n) = Q[k][n]: the weight
//                          gradients dY^T h, dg^T X, du^T X, dl^T x.
//                     64 x 64 tiles, 32-deep K steps staged through LDS as
//                     [m][k] and [n][k] (k-major operands are transposed on the
//                     way in), 4 waves x 2 x 2 v_mfma_f32_16x16x32_bf16 blocks.
//   swiglu_fwd_kernel h = SiLU(g) u (bf16), from the recomputed fp32 g and u
//   swiglu_bwd_kernel dg = dh u SiLU'(g), du = dh SiLU(g) (bf16)
//   combine_bwd_kernel   per (token, slot): dw = <dy, Y_slot>, dY_slot = w dy
//   router_bwd_kernel    per token: softmax backward of w = scale * s[ids]
//   dx_sum_kernel        dx[t] = sum_j dX_slot + dX_shared + dl Wr, fixed order
//   colsum_kernel        d_bias = sum over tokens of dl
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int BM = 64, BN = 64, BK = 32;
constexpr int LDSP = BK + 8;  // bf16 per LDS row (padded: 80 bytes)

typedef __bf16 bf16x8_b __attribute__((ext_vector_type(8)));

// One 64 x 32 operand tile into LDS as [row][k] (row = m for A, n for B).
//   KMAJ false: element (row, k) at src[row_phys(row) * ld + k]   (k contiguous)
//   KMAJ true:  element (row, k) at src[k_phys(k) * ld + row]     (row contiguous)
// Rows past nrow and k past nk load zeros.  256 threads, 8 elements each;
// 16-byte loads when the leading dimension keeps them aligned (ld % 8 == 0).
template <bool KMAJ, class RowMap, class KMap>
MOE_DEV void load_tile(uint16_t (*dst)[LDSP], const uint16_t* src, long ld, int row0, int nrow, int k0, int nk,
                       RowMap row_phys, KMap k_phys) {
  const int tid = threadIdx.x;
  if constexpr (!KMAJ) {
    const int r = tid >> 2, c = (tid & 3) * 8;  // row r, k = c .. c+7
    u32x4 v = u32x4{0, 0, 0, 0};
    if (r < nrow - row0 && c < nk - k0) {
      const uint16_t* s = src + row_phys(row0 + r) * ld + k0 + c;
      if (c + 8 <= nk - k0 && (ld & 7) == 0) {
        v = *reinterpret_cast<const u32x4*>(s);
      } else {
        uint16_t t[8] = {};
        for (int i = 0; i < 8 && c + i < nk - k0; ++i) t[i] = s[i];
        for (int q = 0; q < 4; ++q) v[q] = uint32_t(t[2 * q]) | (uint32_t(t[2 * q + 1]) << 16);
      }
    }
    *reinterpret_cast<u32x4*>(&dst[r][c]) = v;
  } else {
    const int k = tid >> 3, r = (tid & 7) * 8;  // k row of the source, rows r .. r+7
    uint16_t t[8] = {};
    if (k < nk - k0 && r < nrow - row0) {
      const uint16_t* s = src + k_phys(k0 + k) * ld + row0 + r;
      if (r + 8 <= nrow - row0 && (ld & 7) == 0) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(s);
        for (int q = 0; q < 4; ++q) {
          t[2 * q] = uint16_t(v[q] & 0xffffu);
          t[2 * q + 1] = uint16_t(v[q] >> 16);
        }
      } else {
        for (int i = 0; i < 8 && r + i < nrow - row0; ++i) t[i] = s[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[r + i][k] = t[i];
  }
}

template <bool TN, bool OUT_BF16>
__global__ __launch_bounds__(256) void bwd_gemm_kernel(BwdGemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[BM][LDSP];
  __shared__ __attribute__((aligned(16))) uint16_t sB[BN][LDSP];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1;
  const int NB = (p.N + BN - 1) / BN;
  int e = 0, m0, n0, rows, seg0 = 0;
  long kbeg = 0, kend = p.K;
  if constexpr (TN) {
    // grid: (m tile, n tile) x groups; k runs over the group's segment rows
    const int MB = (p.M + BM - 1) / BM;
    const int per = MB * NB;
    e = blockIdx.x / per;
    const int rest = blockIdx.x % per;
    m0 = (rest / NB) * BM;
    n0 = (rest % NB) * BN;
    rows = p.M;
    if (p.seg) {
      kbeg = min(max(p.seg[e], 0), p.rows);
      kend = min(max(p.seg[e + 1], int(kbeg)), p.rows);
    } else {
      kbeg = 0;
      kend = p.rows;
    }
  } else {
    // grid: tile list entries (or row tiles of one group) x n tiles
    const int tix = blockIdx.x / NB;
    n0 = (blockIdx.x % NB) * BN;
    if (p.tiles) {
      if (tix >= p.ntiles[0]) return;
      e = p.tiles[2 * tix];
      m0 = p.tiles[2 * tix + 1];
      seg0 = min(max(p.seg[e], 0), p.rows);
      const int seg1 = min(max(p.seg[e + 1], seg0), p.rows);
      rows = seg1 - seg0;
    } else {
      m0 = tix * BM;
      rows = p.rows;
    }
    if (m0 >= rows) return;
  }
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int r16 = lane & 15, g = lane >> 4;
  for (int pass = 0; pass < p.npass; ++pass) {
    const uint16_t* A = pass ? p.A1 : p.A0;
    const uint16_t* B = pass ? p.B1 : p.B0;
    if constexpr (TN) {
      // A(m, k) = P[k][m] (P rows: permuted rows, optionally gathered), B(k, n) = Q[k][n]
      const int* amap = p.a_map;
      const int adiv = p.a_div;
      const int* bmap = p.b_map;
      const int bdiv = p.b_div;
      auto kp_a = [&](long k) -> long { return amap ? long(amap[k] / adiv) : k; };
      auto kp_b = [&](long k) -> long { return bmap ? long(bmap[k] / bdiv) : k; };
      auto id = [](int r) -> long { return r; };
      for (long k0 = kbeg; k0 < kend; k0 += BK) {
        __syncthreads();
        load_tile<true>(sA, A, p.lda, m0, p.M, int(k0 - kbeg), int(kend - kbeg), id,
                        [&](int k) { return kp_a(kbeg + k); });
        load_tile<true>(sB, B, p.ldb, n0, p.N, int(k0 - kbeg), int(kend - kbeg), id,
                        [&](int k) { return kp_b(kbeg + k); });
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const bf16x8_b a = *reinterpret_cast<const bf16x8_b*>(&sA[32 * wm + 16 * i + r16][8 * g]);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const bf16x8_b b = *reinterpret_cast<const bf16x8_b*>(&sB[32 * wn + 16 * j + r16][8 * g]);
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i][j], 0, 0, 0);
          }
        }
      }
    } else {
      // A[m][k] row-major (rows of the segment, optionally gathered), B(k, n) = Bg[k][n] of the group
      const uint16_t* Bg = B + long(e) * p.b_stride;
      const int* amap = p.a_map;
      const int adiv = p.a_div;
      auto rp = [&](int r) -> long {
        const long q = seg0 + r;
        return amap ? long(amap[q] / adiv) : q;
      };
      auto id = [](int k) -> long { return k; };
      const int Kp = pass ? p.K1 : p.K;
      for (int k0 = 0; k0 < Kp; k0 += BK) {
        __syncthreads();
        load_tile<false>(sA, A, p.lda, m0, rows, k0, Kp, rp, id);
        load_tile<true>(sB, Bg, p.ldb, n0, p.N, k0, Kp, id, id);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const bf16x8_b a = *reinterpret_cast<const bf16x8_b*>(&sA[32 * wm + 16 * i + r16][8 * g]);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const bf16x8_b b = *reinterpret_cast<const bf16x8_b*>(&sB[32 * wn + 16 * j + r16][8 * g]);
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i][j], 0, 0, 0);
          }
        }
      }
    }
  }
  // lane l holds rows 4g + q, column l % 16 of each 16 x 16 block
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + 32 * wm + 16 * i + 4 * g + q, n = n0 + 32 * wn + 16 * j + r16;
        if (m >= rows || n >= p.N) continue;
        const long off = TN ? long(e) * p.c_stride + long(m) * p.ldc + n : (long(seg0) + m) * p.ldc + n;
        if constexpr (OUT_BF16)
          static_cast<uint16_t*>(p.C)[off] = f32_to_bf16(acc[i][j][q]);
        else
          static_cast<float*>(p.C)[off] = acc[i][j][q];
      }
}

// ---------------------------------------------------------------------------
// bwd_gemm_tr_kernel: the same two shapes on 128 x 128 tiles, 32-deep K steps,
// 4 waves x 2 x 2 blocks of v_mfma_f32_32x32x16_bf16.  Operands stay in LDS in
// the layout they have in memory: a k-contiguous operand (NN's A) as
// [row][k], a k-major one (NN's B, both TN operands) as [k][row], whose MFMA
// fragments (8 consecutive k of one row per lane) come from two transposing
// LDS reads (ds_read_b64_tr_b16: within each 16-lane group, lane i receives
// element i % 4 of the 8 bytes read by lane 4 j + i / 4 as its element j, so
// lanes that point at [kb + s/4][rb + 4 (s%4)] give lane i rows rb + i at
// k = kb .. kb+3).  The next step's tiles are loaded into registers while
// the current step's MFMAs run, then stored into the other LDS buffer: one
// barrier per step.  Requires every leading dimension, K (NN) and the
// row/column counts to be multiples of 8 (16-byte loads); the launcher
// falls back to bwd_gemm_kernel otherwise.
constexpr int TT = 128, TK = 32;
constexpr int KCP = TK + 8;   // bf16 per row of a [row][k] tile (80 bytes: 16-byte reads spread over banks)
constexpr int RCP = TT + 16;  // bf16 per k-row of a [k][row] tile (288 bytes)

typedef short v4i16 __attribute__((ext_vector_type(4)));

// thread's 32 bytes of a [row][k] tile: row t/2, k 16 (t%2) + [0, 16)
template <class RowMap>
MOE_DEV void kc_load(u32x4 (&v)[2], const uint16_t* src, long ld, int nrow, int k0, int K, RowMap row_phys) {
  const int t = threadIdx.x, r = t >> 1;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int kk = k0 + 16 * (t & 1) + 8 * q;
    v[q] = (r < nrow && kk < K) ? *reinterpret_cast<const u32x4*>(src + row_phys(r) * ld + kk) : u32x4{0, 0, 0, 0};
  }
}
MOE_DEV void kc_store(uint16_t* tile, const u32x4 (&v)[2]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 2; ++q) *reinterpret_cast<u32x4*>(tile + (t >> 1) * KCP + 16 * (t & 1) + 8 * q) = v[q];
}
// thread's 32 bytes of a [k][row] tile: k t/8, rows 16 (t%8) + [0, 16) (row0..row0+127 of the source)
template <class KMap>
MOE_DEV void rc_load(u32x4 (&v)[2], const uint16_t* src, long ld, int row0, int nrow, int k, int kend, KMap k_phys) {
  const int t = threadIdx.x, kr = k + (t >> 3);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = 16 * (t & 7) + 8 * q;
    v[q] = (kr < kend && row0 + r < nrow) ? *reinterpret_cast<const u32x4*>(src + k_phys(kr) * ld + row0 + r)
                                          : u32x4{0, 0, 0, 0};
  }
}
MOE_DEV void rc_store(uint16_t* tile, const u32x4 (&v)[2]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 2; ++q) *reinterpret_cast<u32x4*>(tile + (t >> 3) * RCP + 16 * (t & 7) + 8 * q) = v[q];
}
// MFMA fragment (rows rb + lane % 32, k = 16 h + 8 (lane / 32) + [0, 8)) of a [row][k] tile
MOE_DEV bf16x8_b kc_frag(const uint16_t* tile, int rb, int h) {
  const int l = lane_id();
  return *reinterpret_cast<const bf16x8_b*>(tile + (rb + (l & 31)) * KCP + 16 * h + 8 * (l >> 5));
}
// ... of a [k][row] tile, by two transposing reads
MOE_DEV bf16x8_b rc_frag(const uint16_t* tile, int rb, int h) {
  const int l = lane_id(), gg = l >> 4, sl = l & 15;
  const uint16_t* base = tile + (16 * h + 8 * (gg >> 1) + (sl >> 2)) * RCP + rb + 16 * (gg & 1) + 4 * (sl & 3);
  typedef __attribute__((address_space(3))) v4i16 lds_v4;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(base));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(base + 4 * RCP));
  const short e[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_b, e);
}

template <bool TN, bool OUT_BF16>
__global__ __launch_bounds__(256) void bwd_gemm_tr_kernel(BwdGemmParams p) {
  // NN: A [row][k] (TT x KCP), B [k][n] (TK x RCP); TN: both [k][row]
  constexpr int A_ELEMS = TN ? TK * RCP : TT * KCP;
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][A_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][TK * RCP];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1;
  const int NB = (p.N + TT - 1) / TT;
  int e = 0, m0, n0, rows, seg0 = 0;
  long kbeg = 0, kend = p.K;
  if constexpr (TN) {
    const int MB = (p.M + TT - 1) / TT;
    const int per = MB * NB;
    e = blockIdx.x / per;
    const int rest = blockIdx.x % per;
    m0 = (rest / NB) * TT;
    n0 = (rest % NB) * TT;
    rows = p.M;
    if (p.seg) {
      kbeg = min(max(p.seg[e], 0), p.rows);
      kend = min(max(p.seg[e + 1], int(kbeg)), p.rows);
    } else {
      kend = p.rows;
    }
  } else {
    const int tix = blockIdx.x / NB;
    n0 = (blockIdx.x % NB) * TT;
    if (p.tiles) {
      if (tix >= p.ntiles[0]) return;
      e = p.tiles[2 * tix];
      m0 = p.tiles[2 * tix + 1];
      seg0 = min(max(p.seg[e], 0), p.rows);
      const int seg1 = min(max(p.seg[e + 1], seg0), p.rows);
      rows = seg1 - seg0;
    } else {
      m0 = tix * TT;
      rows = p.rows;
    }
    if (m0 >= rows) return;
  }
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  for (int pass = 0; pass < p.npass; ++pass) {
    const uint16_t* A = pass ? p.A1 : p.A0;
    const uint16_t* B = pass ? p.B1 : p.B0;
    const uint16_t* Bg = TN ? B : B + long(e) * p.b_stride;
    const int* amap = p.a_map;
    const int adiv = p.a_div;
    const int* bmap = p.b_map;
    const int bdiv = p.b_div;
    // NN: A rows of the segment (optionally gathered); TN: source rows of the k index
    auto a_row = [&](int r) -> long {
      const long q = seg0 + m0 + r;
      return amap ? long(amap[q] / adiv) : q;
    };
    auto ka = [&](int k) -> long { return amap ? long(amap[k] / adiv) : k; };
    auto kb = [&](int k) -> long { return bmap ? long(bmap[k] / bdiv) : k; };
    auto kid = [](int k) -> long { return k; };
    const int Kp = TN ? int(kend - kbeg) : (pass ? p.K1 : p.K);
    const int nsteps = (Kp + TK - 1) / TK;
    if (nsteps <= 0) continue;
    u32x4 ra[2], rb[2];
    auto load = [&](int st) {
      const int k = st * TK;
      if constexpr (TN) {
        rc_load(ra, A, p.lda, m0, p.M, int(kbeg) + k, int(kend), ka);
        rc_load(rb, B, p.ldb, n0, p.N, int(kbeg) + k, int(kend), kb);
      } else {
        kc_load(ra, A, p.lda, rows - m0, k, Kp, a_row);
        rc_load(rb, Bg, p.ldb, n0, p.N, k, Kp, kid);
      }
    };
    auto store = [&](int buf) {
      if constexpr (TN) rc_store(sA[buf], ra);
      else kc_store(sA[buf], ra);
      rc_store(sB[buf], rb);
    };
    __syncthreads();  // the previous pass's last reads of both buffers are done
    load(0);
    store(0);
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
      const int buf = st & 1;
      const bool more = st + 1 < nsteps;
      if (more) load(st + 1);
#pragma unroll
      for (int h = 0; h < TK / 16; ++h) {
        bf16x8_b a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          a[i] = TN ? rc_frag(sA[buf], 64 * wm + 32 * i, h) : kc_frag(sA[buf], 64 * wm + 32 * i, h);
#pragma unroll
        for (int j = 0; j < 2; ++j) b[j] = rc_frag(sB[buf], 64 * wn + 32 * j, h);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
      if (more) store(buf ^ 1);
      __syncthreads();
    }
  }
  // lane l: column l % 32, rows 8 (r / 4) + 4 (l / 32) + r % 4 of each 32 x 32 block
  const int g = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
        const int n = n0 + 64 * wn + 32 * j + l32;
        if (m >= rows || n >= p.N) continue;
        const long off = TN ? long(e) * p.c_stride + long(m) * p.ldc + n : (long(seg0) + m) * p.ldc + n;
        if constexpr (OUT_BF16)
          static_cast<uint16_t*>(p.C)[off] = f32_to_bf16(acc[i][j][r]);
        else
          static_cast<float*>(p.C)[off] = acc[i][j][r];
      }
}

MOE_DEV float sig(float g) { return 1.0f / (1.0f + __expf(-g)); }

__global__ void swiglu_fwd_kernel(const float* __restrict__ g, const float* __restrict__ u, long n,
                                  uint16_t* __restrict__ h) {
  const long i = long(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) h[i] = f32_to_bf16(silu(g[i]) * u[i]);
}

__global__ void swiglu_bwd_kernel(const float* __restrict__ g, const float* __restrict__ u,
                                  const float* __restrict__ dh, long n, uint16_t* __restrict__ dg,
                                  uint16_t* __restrict__ du) {
  const long i = long(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float gv = g[i], s = sig(gv), d = dh[i];
  du[i] = f32_to_bf16(d * gv * s);
  dg[i] = f32_to_bf16(d * u[i] * (s * (1.0f + gv * (1.0f - s))));
}

// one workgroup per (token, slot): dw = <dy[t], Y[pos]> (fixed order: lanes
// stride, then a wave sum and the 4 waves in order), dY[pos] = bf16(w dy[t])
__global__ __launch_bounds__(256) void combine_bwd_kernel(const uint16_t* __restrict__ dy, const float* __restrict__ Y,
                                                          const int* __restrict__ inv_pos, const float* __restrict__ w,
                                                          int K, int H, float* __restrict__ dw,
                                                          uint16_t* __restrict__ dY) {
  __shared__ float part[4];
  const int p = blockIdx.x, t = p / K, pos = inv_pos[p];
  const float wp = w[p];
  float acc = 0.f;
  for (int c = threadIdx.x; c < H; c += 256) {
    const float d = bf16_to_f32(dy[size_t(t) * H + c]);
    if (pos >= 0) {
      acc = fmaf(d, Y[size_t(pos) * H + c], acc);
      dY[size_t(pos) * H + c] = f32_to_bf16(wp * d);
    }
  }
  acc = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) dw[p] = ((part[0] + part[1]) + part[2]) + part[3];
}

// one wave per token: s = softmax(logits + bias) over all experts,
// ds = scale * dw on the selected experts, dl = s (ds - sum s ds)
__global__ __launch_bounds__(256) void router_bwd_kernel(const float* __restrict__ logits,
                                                         const float* __restrict__ bias, const int* __restrict__ ids,
                                                         const float* __restrict__ dw, int T, int E, int K,
                                                         float scale, float* __restrict__ dl,
                                                         uint16_t* __restrict__ dl_bf) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = lane_id();
  if (t >= T) return;
  float l[4], ds[4];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    l[i] = e < E ? logits[size_t(t) * E + e] + (bias ? bias[e] : 0.f) : -INFINITY;
    mx = fmaxf(mx, l[i]);
    ds[i] = 0.f;
    for (int j = 0; j < K; ++j)
      if (ids[t * K + j] == e) ds[i] = scale * dw[t * K + j];
  }
  mx = wave_max(mx);
  float se = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) se += lane + 64 * i < E ? __expf(l[i] - mx) : 0.f;
  se = wave_sum(se);
  float s[4], sds = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s[i] = lane + 64 * i < E ? __expf(l[i] - mx) / se : 0.f;
    sds += s[i] * ds[i];
  }
  sds = wave_sum(sds);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      const float v = s[i] * (ds[i] - sds);
      dl[size_t(t) * E + e] = v;
      dl_bf[size_t(t) * E + e] = f32_to_bf16(v);
    }
  }
}

// dx[t][c] = bf16( sum_j dXr[inv_pos[t*K+j]][c] + dXs[t][c] + dXw[t][c] ), in that order
__global__ void dx_sum_kernel(const float* __restrict__ dXr, const int* __restrict__ inv_pos, int K,
                              const float* __restrict__ dXs, const float* __restrict__ dXw, int T, int H,
                              uint16_t* __restrict__ dx) {
  const long i = long(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= long(T) * H) return;
  const int t = int(i / H), c = int(i % H);
  float v = 0.f;
  for (int j = 0; j < K; ++j) {
    const int pos = inv_pos[t * K + j];
    if (pos >= 0) v += dXr[size_t(pos) * H + c];
  }
  if (dXs) v += dXs[i];
  v += dXw[i];
  dx[i] = f32_to_bf16(v);
}

// out[e] = sum over t of dl[t][e]: one workgroup per expert; thread i sums
// tokens i, i + 256, ... in order, then a fixed-order tree over the threads
__global__ __launch_bounds__(256) void colsum_kernel(const float* __restrict__ dl, int T, int E, float* __restrict__ out) {
  __shared__ float part[256];
  const int e = blockIdx.x;
  float v = 0.f;
  for (int t = threadIdx.x; t < T; t += 256) v += dl[size_t(t) * E + e];
  part[threadIdx.x] = v;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (int(threadIdx.x) < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[e] = part[0];
}

}  // namespace

hipError_t launch_bwd_gemm(bool tn, bool out_bf16, const BwdGemmParams& p, int n_groups, hipStream_t s) {
  // the 128 x 128 transposing-read kernel needs 16-byte aligned rows everywhere
  const bool tr = p.lda % 8 == 0 && p.ldb % 8 == 0 && p.N % 8 == 0 && p.b_stride % 8 == 0 &&
                  (tn ? p.M % 8 == 0 : (p.K % 8 == 0 && (p.npass < 2 || p.K1 % 8 == 0)));
  if (p.tiles && !tr) return hipErrorInvalidValue;  // tile lists hold 128-row tiles
  const int tile = tr ? TT : BM;
  const long NB = (p.N + tile - 1) / tile;
  long blocks;
  if (tn) blocks = long(n_groups) * ((p.M + tile - 1) / tile) * NB;
  else blocks = (p.tiles ? long(p.max_tiles) : long((p.rows + tile - 1) / tile)) * NB;
  if (blocks <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(blocks));
  if (tr) {
    if (tn) {
      if (out_bf16) hipLaunchKernelGGL((bwd_gemm_tr_kernel<true, true>), grid, dim3(256), 0, s, p);
      else hipLaunchKernelGGL((bwd_gemm_tr_kernel<true, false>), grid, dim3(256), 0, s, p);
    } else {
      if (out_bf16) hipLaunchKernelGGL((bwd_gemm_tr_kernel<false, true>), grid, dim3(256), 0, s, p);
      else hipLaunchKernelGGL((bwd_gemm_tr_kernel<false, false>), grid, dim3(256), 0, s, p);
    }
  } else if (tn) {
    if (out_bf16) hipLaunchKernelGGL((bwd_gemm_kernel<true, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((bwd_gemm_kernel<true, false>), grid, dim3(256), 0, s, p);
  } else {
    if (out_bf16) hipLaunchKernelGGL((bwd_gemm_kernel<false, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((bwd_gemm_kernel<false, false>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_swiglu_fwd(const float* g, const float* u, long n, uint16_t* h, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_fwd_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, g, u, n, h);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const float* g, const float* u, const float* dh, long n, uint16_t* dg, uint16_t* du,
                             hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, g, u, dh, n, dg, du);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const uint16_t* dy, const float* Y, const int* inv_pos, const float* w, int T, int K,
                              int H, float* dw, uint16_t* dY, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(combine_bwd_kernel, dim3(unsigned(T * K)), dim3(256), 0, s, dy, Y, inv_pos, w, K, H, dw, dY);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const float* logits, const float* bias, const int* ids, const float* dw, int T, int E,
                             int K, float scale, float* dl, uint16_t* dl_bf, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (E > 256) return hipErrorInvalidValue;
  hipLaunchKernelGGL(router_bwd_kernel, dim3(unsigned((T + 3) / 4)), dim3(256), 0, s, logits, bias, ids, dw, T, E, K,
                     scale, dl, dl_bf);
  return hipGetLastError();
}

hipError_t launch_dx_sum(const float* dXr, const int* inv_pos, int K, const float* dXs, const float* dXw, int T, int H,
                         uint16_t* dx, hipStream_t s) {
  const long n = long(T) * H;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(dx_sum_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, dXr, inv_pos, K, dXs, dXw, T, H,
                     dx);
  return hipGetLastError();
}

hipError_t launch_colsum(const float* dl, int T, int E, float* out, hipStream_t s) {
  if (E <= 0) return hipSuccess;
  hipLaunchKernelGGL(colsum_kernel, dim3(unsigned(E)), dim3(256), 0, s, dl, T, E, out);
  return hipGetLastError();
}

}  // namespace moe
