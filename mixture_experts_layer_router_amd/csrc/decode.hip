// Single-launch small-batch MoE layer (T <= 8, bf16 activations, one weight
// format for routed and shared experts): stages N, O, P1/Q1, P2/Q2 and the
// sum of R of the DSV2-236B-MegaKernel README flowchart in one persistent
// launch, so HBM keeps streaming weights across what would otherwise be four
// kernel boundaries (each costs a ramp and a tail of a few microseconds).
//
// Router rows come first: workgroup e < E computes row e of the logits
// (all tokens) as soon as it starts; the lowest block indices are dispatched
// first, and the routing is what every routed item waits for.  The logits
// are handed over tagged: each is a 64-bit word holding the launch's tag
// (from an epoch word that the last workgroup out advances) beside the float,
// and a workgroup that needs the routing polls the E words of each token
// until all carry this launch's tag.  That costs one round trip after the
// last router row, where counting the rows and raising a flag would cost
// three (two atomics and the flag read) on a memory system busy with weight
// streams.  The rest of the work is a list of items in dependency order:
//   SU  shared gate/up         (8 intermediate columns of every token from 3
//                               tokens on, else of one token)
//   RG  routed gate/up         (8 intermediate columns of one distinct expert
//                               for every slot that chose it from 3 tokens
//                               on, else of one (token, slot))
//   DN  down + combine         (4 output rows of one token: the shared and
//                               the K routed down matrices as one long dot)
// From 3 tokens on a gate/up weight row is thus read once per launch, not
// once per token or slot (8 tokens: 256 -> 233 us per layer).
// RG needs all router rows (each workgroup runs the top-k itself from the
// logits); DN needs the routing for its weight addresses and SU + RG for h.
// A DN item issues its weight loads first and only then waits for h, so the
// down weights stream while the last gate/up items finish.  Item i sits in
// queue i % kQ.  With at most 16 items per workgroup (1 to 4 tokens) the
// schedule is static: the j-th workgroup of queue q (workgroup b = q + kQ j)
// takes the queue's items j, j + nq, j + 2 nq, ... (nq workgroups per queue)
// in order; one device-scope atomic claim per item cost 2.7 us more per B=1
// layer (48.1 against 45.4 us).  With more items (8 tokens: about 26 per
// workgroup) the round robin balances worse than claims (240 against 235 us),
// so workgroup b claims the items of queue q in order with one atomic each.
// An item waits only for the router rows (which wait for nothing) or for
// earlier items, and every workgroup takes its items in increasing order, so
// the earliest unfinished item always belongs to a workgroup that can run
// it.  Static: the launch completes once all its workgroups have been
// resident; claims: once max(E, kQ) of them are resident at a time (the
// router rows' workgroups are the first dispatched, and each queue needs a
// server).  The grid is the device's resident capacity, so either holds
// unless a kernel on another stream keeps CUs busy beyond the waits' bound.
//
// Same-address device-scope atomics serialise at about 12 ns each, so a
// workgroup counts its finished items of a phase in a register and adds them
// to the phase's counter in one atomic when its run of items of that phase
// ends (its next item belongs to another phase, or there is none); whoever
// brings the counter to the phase's item count raises the phase's ready flag.
// Waiters poll only the flag (a line no atomic touches).  A workgroup never
// waits while it holds uncounted items, so nothing waits on itself.
// Cross-workgroup data (ids / weights, h) is written with device-scope
// atomic stores; a producer waits for its stores (vmcnt(0)) before its
// increment.  A consumer reads the data with plain loads after seeing the
// flag: its XCD's L2 cannot hold those lines yet, since nothing reads them
// before the flag rises and every launch starts with clean L2s.  No L2
// writeback or invalidate is needed.  The tagged logits, which are polled
// before they are ready, are read with device-scope loads instead.  Waits
// are bounded (about 0.2 s): a wait that gives up sets the error word and the
// workgroup writes NaN for its outputs.  The last workgroup to exit resets
// every counter and flag and advances the epoch.
#include <algorithm>

#include "gemv_dev.h"

namespace moe {

namespace {

constexpr int kQ = 32;         // queues, and most stripes of a counter
constexpr int kLine = 32;      // words per 128-byte line
constexpr int kUR = 2;         // intermediate columns per wave in a gate/up item
constexpr int kUpCols = 4 * kUR;
constexpr int kSUR = 2;        // ... in a shared gate/up item
constexpr int kSUpCols = 4 * kSUR;
constexpr int kDR = 4;         // output rows of a down item
constexpr int kDJ = 3;         // down chunks per wave held in registers at once
constexpr int kPhases = 2;     // phases that signal completion: SU, RG
constexpr uint64_t kWaitTicks = 20000000;  // s_memrealtime runs at 100 MHz: 0.2 s

// Counter block (one counter per 128-byte line, word 0 of the line):
//   line 0: error word, epoch word         lines 1..kQ: queue heads (dynamic schedule)
//   per phase f: stripe summary, ready flag
//   exit stripes (kQ) and exit summary
//   per phase f: item counters of the kQ stripes
struct Ctr {
  unsigned* base;
  MOE_DEV unsigned* error() const { return base; }
  MOE_DEV unsigned* epoch() const { return base + kFusedEpochWord; }
  // tagged router logits [T][E] (64-bit words, past the counter lines)
  MOE_DEV uint64_t* tagged() const { return reinterpret_cast<uint64_t*>(base + kFusedTagOff / 4); }
  MOE_DEV unsigned* head(int q) const { return base + (1 + q) * kLine; }
  MOE_DEV unsigned* count(int f) const { return base + (1 + kQ + 2 * f) * kLine; }
  MOE_DEV unsigned* flag(int f) const { return base + (2 + kQ + 2 * f) * kLine; }
  MOE_DEV unsigned* exit_stripe(int s) const { return base + (1 + kQ + 2 * kPhases + s) * kLine; }
  MOE_DEV unsigned* exit_summary() const { return exit_stripe(kQ); }
  MOE_DEV unsigned* stripe(int f, int s) const { return base + (2 + 2 * kQ + 2 * kPhases + f * kQ + s) * kLine; }
};
constexpr int kCtrLines = 2 + 2 * kQ + 2 * kPhases + kPhases * kQ;
static_assert(kCtrLines * kLine * 4 <= kFusedTagOff, "counter lines");
static_assert(kFusedTagOff + kRouteGemvMaxT * 256 * 8 <= kFusedCtrBytes, "tagged logits");
static_assert(kFusedErrorWord == 0 && kFusedEpochWord < kLine, "line 0 words");

MOE_DEV unsigned atomic_add(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
MOE_DEV unsigned atomic_inc(unsigned* p) { return atomic_add(p, 1u); }
template <class V>
MOE_DEV void store_agent(V* p, V v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// waits for completion of this thread's earlier global stores; the memory
// clobber keeps the compiler from moving any store past it
MOE_DEV void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Items i in [a, b) with i % kQ == q: the items of that range in queue q.
MOE_DEV unsigned in_queue(int a, int b, int q) {
  auto upto = [q](int x) { return x > q ? unsigned((x - q + kQ - 1) / kQ) : 0u; };
  return upto(b) - upto(a);
}

// Counts `cnt` finished items of phase f, whose items are [a, b), run by a
// workgroup of queue q.  A phase is counted in kQ stripes, one per queue (a
// stripe's item count is known), so no counter takes more than the
// increments of one queue's workgroups: same-address atomics serialise.  The
// workgroup that completes a stripe counts it in the phase's summary, and
// the one that completes the last stripe raises the flag.  Every thread calls
// it; the workgroup's stores are complete before thread 0 counts the items.
MOE_DEV void count_items(const Ctr& c, int f, int q, int cnt, int a, int b) {
  stores_done();
  __syncthreads();
  if (threadIdx.x == 0)
    if (atomic_add(c.stripe(f, q), unsigned(cnt)) + unsigned(cnt) == in_queue(a, b, q))
      if (atomic_inc(c.count(f)) + 1 == unsigned(min(b - a, kQ))) store_agent(c.flag(f), 1u);
}

// Bounded wait for phase f's ready flag; false if it gave up.
MOE_DEV bool wait_flag(const Ctr& c, int f, int* s_ok) {
  if (threadIdx.x == 0) {
    int ok = 1;
    if (__hip_atomic_load(c.flag(f), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (__hip_atomic_load(c.flag(f), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
        __builtin_amdgcn_s_sleep(1);
        if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
          store_agent(c.error(), 1u);
          ok = 0;
          break;
        }
      }
    }
    *s_ok = ok;
  }
  __syncthreads();
  return *s_ok != 0;
}

// One wave: token row `row` of the tagged logits into the top-k layout
// (+ bias), once every expert's word carries `tag`.  Bounded like wait_flag;
// false (and the error word set) if it gave up.  Agent-scope loads: a line
// this XCD's L2 held from before the producer's store would show an old tag.
MOE_DEV bool load_tagged_logits(const RouteParams& rp, const TopkLayout& L, const uint64_t* row, const float* bias,
                                unsigned tag, float (&lg)[kMpl], unsigned* err) {
  uint64_t v[kMpl];
  bool mine = true;
#pragma unroll
  for (int j = 0; j < kMpl; ++j) {
    const int e = L.expert(rp, j);
    v[j] = e >= 0 ? __hip_atomic_load(row + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
    mine &= e < 0 || unsigned(v[j] >> 32) == tag;
  }
  bool ok = true;
  if (!__all(mine)) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    do {
      __builtin_amdgcn_s_sleep(1);
      mine = true;
#pragma unroll
      for (int j = 0; j < kMpl; ++j) {
        const int e = L.expert(rp, j);
        if (e >= 0 && unsigned(v[j] >> 32) != tag)
          v[j] = __hip_atomic_load(row + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        mine &= e < 0 || unsigned(v[j] >> 32) == tag;
      }
      if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
        ok = false;
        break;
      }
    } while (!__all(mine));
  }
  if (!ok && lane_id() == 0) store_agent(err, 1u);
#pragma unroll
  for (int j = 0; j < kMpl; ++j) {
    const int e = L.expert(rp, j);
    lg[j] = e >= 0 ? __uint_as_float(unsigned(v[j])) + (bias ? bias[e] : 0.0f) : kNegInfF;
  }
  return ok;
}

// sum of the 4 waves' partial row sums; thread r < R gets row r
template <int R>
MOE_DEV float rows_reduce(float (&acc)[R], float (*dpart)[kDR], int wave, int lane) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float v = wave_sum(acc[r]);
    if (lane == r) dpart[wave][r] = v;
  }
  __syncthreads();
  float v = 0.f;
  if (threadIdx.x < R) {
    v = dpart[0][threadIdx.x];
#pragma unroll
    for (int w = 1; w < 4; ++w) v += dpart[w][threadIdx.x];
  }
  return v;
}

// Weights (and scales, with the routing weight folded in) of one down chunk
// for kDR rows; the activations are loaded later, when they exist.
template <int WF>
struct DnStage {
  u32x4 w[kDR];
  float sc[WF == W_MXFP8 ? kDR : 1];
};

template <int WF>
MOE_DEV void dn_load_w(DnStage<WF>& st, const DownSrc& s, int n0) {
#pragma unroll
  for (int r = 0; r < kDR; ++r) st.w[r] = *reinterpret_cast<const u32x4*>(s.w + size_t(r) * s.L * Fmt<WF>::ES);
  if (WF == W_MXFP8) {
#pragma unroll
    for (int r = 0; r < kDR; ++r) st.sc[r] = s.f * wscale<WF>(s.s, n0 + r, s.off, s.L);
  } else {
    st.sc[0] = s.f * wscale<WF>(s.s, n0, s.off, s.L);
  }
}

// lanes whose chunk column lies past the end (ok false) add 0
template <int WF>
MOE_DEV void dn_math(const DnStage<WF>& st, const DownSrc& s, float (&acc)[kDR]) {
  float h[Fmt<WF>::EPL];
  load_x<true, Fmt<WF>::EPL>(s.h, 0, h);
#pragma unroll
  for (int r = 0; r < kDR; ++r) {
    const float sc = s.ok ? st.sc[WF == W_MXFP8 ? r : 0] : 0.0f;
    acc[r] = fmaf(dot_chunk<WF>(st.w[r], h), sc, acc[r]);
  }
}

// a global-memory pointer the caller knows to be the same in every lane, in
// scalar registers; typed as global so that loads through it are global
// loads (a generic pointer would make them flat loads, which also count in
// the LDS counter, so every wait for an LDS read of x would wait for them)
#define MOE_GLOBAL __attribute__((address_space(1)))
MOE_DEV const MOE_GLOBAL uint8_t* uni(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(v)));
  const uint64_t hi = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(v >> 32)));
  return reinterpret_cast<const MOE_GLOBAL uint8_t*>((hi << 32) | lo);
}


// 16 bytes of x as bf16 pairs, from LDS or (x in global memory) with a global load
MOE_DEV u32x4 ldx4(const uint32_t* p) { return *reinterpret_cast<const u32x4*>(p); }
MOE_DEV u32x4 ldx4(const MOE_GLOBAL uint32_t* p) { return *reinterpret_cast<const MOE_GLOBAL u32x4*>(p); }

// h[j][i0 .. i0+NR) = SiLU(x_j.Wg^T) * (x_j.Wu^T) for nt <= MAXT token rows
// (bf16 pairs; x row j at xrow(j), in LDS or global memory; h row j at
// hrow(j)).  Each weight chunk is read once, turned into bf16 pairs once
// (the same pairs and sum order as dot_chunk_bx) and dotted with the x of
// every token, so a matrix row that several tokens need streams from HBM
// once.  One 1 KB chunk per row is in flight per round, so a wave's requests
// spread over its item (that streams better than all of an item's loads at
// once: 48.0 against 50.3 us per B=1 layer).  h is stored with agent-scope
// atomic stores (read by other workgroups inside the launch once the phase
// is published), lane NR * j + r storing h[j][i0 + r]; pre() runs once
// every load has been consumed and before the store.
constexpr int kXG = 4;  // tokens whose x chunk a gate/up wave holds at once
template <int WF, int NR, int MAXT, class XRow, class HRow, class Pre>
MOE_DEV void gate_up_multi(XRow xrow, int nt, int H, const void* g, const void* u, const void* gs, const void* us,
                           int i0, HRow hrow, Pre pre) {
  constexpr int CW = Fmt<WF>::CW, EPL = Fmt<WF>::EPL, ES = Fmt<WF>::ES;
  constexpr int NS = WF == W_MXFP8 ? NR : 1;  // scales per chunk (FP8_B128: the rows share a 128-row block)
  static_assert(NR * MAXT <= 64, "one lane per stored h value");
  const int lane = lane_id();
  const MOE_GLOBAL uint8_t* gb[NR];
  const MOE_GLOBAL uint8_t* ub[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    gb[r] = uni(static_cast<const uint8_t*>(g) + size_t(i0 + r) * H * ES);
    ub[r] = uni(static_cast<const uint8_t*>(u) + size_t(i0 + r) * H * ES);
  }
  const MOE_GLOBAL uint8_t* gsb = nullptr;
  const MOE_GLOBAL uint8_t* usb = nullptr;
  if (WF == W_FP8_B128) {
    gsb = uni(static_cast<const uint8_t*>(gs) + size_t(i0 >> 7) * (H >> 7) * 4);
    usb = uni(static_cast<const uint8_t*>(us) + size_t(i0 >> 7) * (H >> 7) * 4);
  }
  float ag[NR][MAXT], au[NR][MAXT];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int j = 0; j < MAXT; ++j) ag[r][j] = au[r][j] = 0.f;
  const int kl = lane * EPL;
  for (int k0 = 0; k0 < H; k0 += CW) {
    const bool valid = k0 + kl < H;  // lanes past the row end add 0
    const uint32_t k = uint32_t(min(k0 + kl, H - EPL));
    u32x4 wg[NR], wu[NR];
    float sg[NS], su[NS];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      wg[r] = *reinterpret_cast<const MOE_GLOBAL u32x4*>(gb[r] + k * ES);
      wu[r] = *reinterpret_cast<const MOE_GLOBAL u32x4*>(ub[r] + k * ES);
    }
    if (WF == W_FP8_B128) {
      sg[0] = *reinterpret_cast<const MOE_GLOBAL float*>(gsb + (k >> 7) * 4);
      su[0] = *reinterpret_cast<const MOE_GLOBAL float*>(usb + (k >> 7) * 4);
    } else {
#pragma unroll
      for (int r = 0; r < NS; ++r) {
        sg[r] = wscale<WF>(gs, i0 + r, int(k), H);
        su[r] = wscale<WF>(us, i0 + r, int(k), H);
      }
    }
    uint32_t pg[NR][EPL / 2], pu[NR][EPL / 2];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      bf16_pairs<WF>(wg[r], pg[r]);
      bf16_pairs<WF>(wu[r], pu[r]);
    }
    // x of at most kXG tokens in registers at once
#pragma unroll
    for (int j0 = 0; j0 < MAXT; j0 += kXG) {
      if (j0 >= nt) break;  // uniform
      uint32_t xp[kXG][EPL / 2];
#pragma unroll
      for (int jj = 0; jj < kXG; ++jj) {
        if (j0 + jj >= nt || j0 + jj >= MAXT) break;
        const auto xr = xrow(j0 + jj);
#pragma unroll
        for (int i = 0; i < EPL / 8; ++i) {
          const u32x4 v = ldx4(xr + k / 2 + 4 * i);
#pragma unroll
          for (int q = 0; q < 4; ++q) xp[jj][4 * i + q] = v[q];
        }
      }
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float sgr = valid ? sg[NS > 1 ? r : 0] : 0.0f;
        const float sur = valid ? su[NS > 1 ? r : 0] : 0.0f;
#pragma unroll
        for (int jj = 0; jj < kXG; ++jj) {
          const int j = j0 + jj;
          if (j >= nt || j >= MAXT) break;
          ag[r][j] = fmaf(dot_pairs<EPL / 2>(pg[r], xp[jj]), sgr, ag[r][j]);
          au[r][j] = fmaf(dot_pairs<EPL / 2>(pu[r], xp[jj]), sur, au[r][j]);
        }
      }
    }
  }
  float mine = 0.f;
#pragma unroll
  for (int j = 0; j < MAXT; ++j) {
    if (j >= nt) break;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float gv = wave_sum(ag[r][j]);
      const float uv = wave_sum(au[r][j]);
      if (lane == NR * j + r) mine = silu(gv) * uv;
    }
  }
  pre();
  if (lane < NR * nt) {
    const int j = lane / NR, r = lane % NR;
    __hip_atomic_store(hrow(j) + i0 + r, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// XG: x is read from global memory (L2) instead of being staged in LDS, for
// T * H * 2 above kFusedXLdsMax: staging 80 KB per workgroup would leave one
// workgroup per CU, too few loads in flight; x is then already normalised.
template <int WF, bool XG, int MAXT>
__global__ __launch_bounds__(256, 3) void fused_decode_kernel(FusedDecodeParams p) {
  // the T rows of x as bf16 pairs (T * H * 2 bytes of dynamic LDS; none with XG)
  extern __shared__ __attribute__((aligned(16))) uint32_t sx[];
  __shared__ float part[4][MAXT];
  __shared__ float dpart[4][kDR];
  __shared__ int sids[MAXT * 16];
  __shared__ float sw[MAXT * 16];
  // the distinct routed experts of the launch in ascending id order, and per
  // distinct expert u its slots (token-major order) and their number
  __shared__ int s_uexp[MAXT * 16], s_unt[MAXT * 16], s_uslot[MAXT * 16][MAXT];
  __shared__ unsigned s_bits[8];
  __shared__ int s_nuniq;
  __shared__ unsigned s_next;
  __shared__ int s_ok, s_last, s_rok;
  const DecodeParams& d = p.d;
  const Ctr c{p.ctr};
  const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
  const int T = d.T, H = d.H, K = d.rp.K, E = d.rp.E, I = p.I, Is = d.Is;
  // from 3 tokens on, a shared gate/up item serves every token and a routed
  // one every slot of one distinct expert (each weight row read once); at 1
  // and 2 tokens the second reads come from the caches and the items stay
  // per token and per slot (measured: 2 tokens 81 against 84 us)
  const bool dedup = T > 2;
  const int n[4] = {E, Is ? (dedup ? 1 : T) * (Is / kSUpCols) : 0, T * K * (I / kUpCols), T * (H / kDR)};
  const int b1 = 0, b2 = b1 + n[1], b3 = b2 + n[2];  // queue items: SU, RG, DN (R is static)
  const unsigned total = unsigned(b3 + n[3]);
  const int q = blockIdx.x % kQ;
  // per-workgroup state (uniform across the workgroup)
  bool have_topk = false, have_dn_deps = false, poisoned = false;
  int pend_f = 0, pend_n = 0;  // finished items of phase pend_f not yet counted
  auto phase_of = [&](int i) { return i < b2 ? 0 : (i < b3 ? 1 : 2); };
  const unsigned epoch = __hip_atomic_load(c.epoch(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned tag = epoch % 0xffffffffu + 1u;  // in [1, 0xffffffff]: a zero-filled word is never ready
  const MOE_GLOBAL uint32_t* xg = reinterpret_cast<const MOE_GLOBAL uint32_t*>(uni(d.x));
  auto xrow = [&](int t) {
    if constexpr (XG) return xg + size_t(t) * H / 2;
    else return static_cast<const uint32_t*>(sx) + size_t(t) * H / 2;
  };
  if constexpr (XG) {
  } else if (d.gamma) {  // stage M: every workgroup normalises the T rows into LDS itself (wave t: row t's r)
    __shared__ float srms[MAXT];
    for (int t = wave; t < T; t += 4) {
      const float r = row_rms_inv(d.x + size_t(t) * H, H, d.eps);
      if (lane == 0) srms[t] = r;
    }
    __syncthreads();
    for (int i = tid; i < T * H / 8; i += 256) {
      const int t = (i * 8) / H;
      const u32x4 xb = norm_chunk(d.x + size_t(t) * H, d.gamma, i * 8 - t * H, srms[t]);
      reinterpret_cast<u32x4*>(sx)[i] = xb;
      if (blockIdx.x == 0 && d.x_out) reinterpret_cast<u32x4*>(d.x_out)[i] = xb;
    }
  } else {
    for (int i = tid; i < T * H / 8; i += 256)
      reinterpret_cast<u32x4*>(sx)[i] = reinterpret_cast<const u32x4*>(d.x)[i];
  }
  if (tid == 0) s_rok = 1;
  __syncthreads();

  // R: workgroup e < E computes router row e before it joins the queues (the
  // lowest block indices are dispatched first, so the routing, which every
  // routed item waits for, starts at once)
  // static schedule: workgroup b is the (b / kQ)-th of queue q's nq
  // workgroups and takes the queue's items b / kQ + nq r, r = 0, 1, ...;
  // dynamic: it claims them (the first claim before its router row)
  const unsigned nq = unsigned(int(gridDim.x) / kQ + (q < int(gridDim.x) % kQ));
  const bool stat = total <= 16u * unsigned(gridDim.x);
  if (!stat && tid == 0) s_next = q + kQ * atomic_inc(c.head(q));
  if (int(blockIdx.x) < E)
    router_row<MAXT>(d.x, T, d.wr, d.rp, blockIdx.x, nullptr, part, false, XG ? nullptr : sx, c.tagged(), tag);
  __syncthreads();
  unsigned item = stat ? blockIdx.x : s_next, next = 0, round = 0;
  __syncthreads();  // thread 0 writes s_next again only after every thread has read it
  while (item < total) {
    // the next item (claimed now); thread 0 hands it to the workgroup
    // (s_next) once this item's loads are consumed and before its stores are
    // issued: stores share the counter that the wait for the claim's value
    // uses, so a later hand-over would also wait for the stores to complete
    ++round;
    if (tid == 0) next = stat ? blockIdx.x / kQ + nq * round : atomic_inc(c.head(q));
    auto hand_over = [&] {
      if (tid == 0) s_next = q + kQ * next;
    };
    const int it = int(item);
    if (it < b2) {  // SU: 8 shared intermediate columns of every token (dedup), else of one token
      const int i = it - b1, per = Is / kSUpCols;
      const int t0 = dedup ? 0 : i / per, c0 = (dedup ? i : i % per) * kSUpCols + wave * kSUR;
      gate_up_multi<WF, kSUR, MAXT>([&](int j) { return xrow(t0 + j); }, dedup ? T : 1, H, d.sg, d.su, d.sgs, d.sus,
                                    c0, [&](int j) { return d.hs + size_t(t0 + j) * Is; }, hand_over);
    } else {
      if (!have_topk) {  // every workgroup routes all T tokens itself (wave w: tokens w, w + 4)
        for (int tt = wave; tt < T; tt += 4) {
          const TopkLayout L(d.rp, lane);
          float lg[kMpl];
          if (!load_tagged_logits(d.rp, L, c.tagged() + size_t(tt) * E, d.bias, tag, lg, c.error()) && lane == 0)
            s_rok = 0;
          topk_select(d.rp, L, lg, sids + tt * K, sw + tt * K);
        }
        __syncthreads();  // every token's ids are in LDS
        // the distinct experts (ids clamped into [0, E) as every consumer
        // of an id does) and the slots that chose each
        if (MAXT == 1 || !dedup) {  // one routed item per slot
          if (tid < T * K) {
            s_uexp[tid] = min(max(sids[tid], 0), E - 1);
            s_unt[tid] = 1;
            s_uslot[tid][0] = tid;
          }
          if (tid == 0) s_nuniq = T * K;
        } else {
          if (tid < 8) s_bits[tid] = 0u;
          __syncthreads();  // s_bits is zero
          const int TK = T * K;
          const int e_mine = tid < TK ? min(max(sids[tid], 0), E - 1) : 0;
          if (tid < TK) atomicOr(&s_bits[e_mine >> 5], 1u << (e_mine & 31));
          __syncthreads();
          if (tid < TK) {
            int u = __popc(s_bits[e_mine >> 5] & ((1u << (e_mine & 31)) - 1u));
            for (int w = 0; w < (e_mine >> 5); ++w) u += __popc(s_bits[w]);
            int j = 0, cnt = 0;
            for (int s2 = 0; s2 < TK; ++s2) {
              const bool same = min(max(sids[s2], 0), E - 1) == e_mine;
              j += same && s2 < tid;
              cnt += same;
            }
            s_uslot[u][j] = tid;
            if (j == 0) {
              s_uexp[u] = e_mine;
              s_unt[u] = cnt;
            }
          }
          if (tid == 0) {
            int nu = 0;
            for (int w = 0; w < 8; ++w) nu += __popc(s_bits[w]);
            s_nuniq = nu;
          }
        }
        __syncthreads();
        poisoned |= s_rok == 0;
        have_topk = true;
      }
      if (it < b3) {  // RG: 8 routed intermediate columns of one distinct expert for every slot that chose
                      // it (dedup), else of one slot
        const int i = it - b2;
        if (i == 0 && tid < T * K) {  // one workgroup publishes the routing
          store_agent(d.ids + tid, sids[tid]);
          store_agent(d.w + tid, sw[tid]);
        }
        const int per = I / kUpCols;
        const int u = i / per, c0 = (i % per) * kUpCols + wave * kUR;
        if (u < s_nuniq) {  // items past the distinct experts (T * K of them at most) have no work
          const int e = s_uexp[u];
          const size_t ws = wstride<WF>(I, H), ss = sstride<WF>(I, H);
          const uint8_t* ge = static_cast<const uint8_t*>(p.g) + e * ws;
          const uint8_t* ue = static_cast<const uint8_t*>(p.u) + e * ws;
          const uint8_t* gse = p.gs ? static_cast<const uint8_t*>(p.gs) + e * ss : nullptr;
          const uint8_t* use = p.us ? static_cast<const uint8_t*>(p.us) + e * ss : nullptr;
          gate_up_multi<WF, kUR, MAXT>([&](int j) { return xrow(s_uslot[u][j] / K); }, s_unt[u], H, ge, ue, gse, use,
                                       c0, [&](int j) { return p.h + size_t(s_uslot[u][j]) * I; }, hand_over);
        } else {
          hand_over();
        }
      } else {  // DN: kDR output rows of one token over [shared Is | routed K*I]
        const int i = it - b3, nb = H / kDR;
        const int t = i / nb, n0 = (i % nb) * kDR;
        GemvDownParams g{};
        g.H = H;
        g.K = K;
        g.I = I;
        g.Is = Is;
        g.h = p.h;
        g.hs = d.hs;
        g.d = p.dn;
        g.ds = p.dns;
        g.sd = d.sd;
        g.sds = d.sds;
        constexpr int CW = Fmt<WF>::CW;
        const int nsh = (Is + CW - 1) / CW, ntot = nsh + (K * I + CW - 1) / CW;
        const float inv_i = 1.0f / float(I);
        const int* sid = sids + t * K;
        const float* swt = sw + t * K;
        auto src = [&](int ch) {
          const int cc = min(ch, ntot - 1);
          DownSrc s = cc < nsh ? shared_src<WF>(g, t, n0, cc) : routed_src<WF>(g, t, n0, cc - nsh, K, inv_i, sid, swt);
          s.ok = s.ok && ch < ntot;
          return s;
        };
        float acc[kDR] = {};
        {  // this wave's first kDJ chunks: weights in flight before the wait for h
          DnStage<WF> st[kDJ];
          DownSrc s[kDJ];
#pragma unroll
          for (int j = 0; j < kDJ; ++j) {
            s[j] = src(wave + 4 * j);
            dn_load_w<WF>(st[j], s[j], n0);
          }
          if (!have_dn_deps) {
            if (Is) poisoned |= !wait_flag(c, 0, &s_ok);
            poisoned |= !wait_flag(c, 1, &s_ok);
            have_dn_deps = true;
          }
#pragma unroll
          for (int j = 0; j < kDJ; ++j) dn_math<WF>(st[j], s[j], acc);
        }
        for (int c0 = wave + 4 * kDJ; c0 < ntot; c0 += 4 * kDJ) {  // the rest, if any (no barrier inside)
          DnStage<WF> st[kDJ];
          DownSrc s[kDJ];
#pragma unroll
          for (int j = 0; j < kDJ; ++j) {
            s[j] = src(c0 + 4 * j);
            dn_load_w<WF>(st[j], s[j], n0);
          }
#pragma unroll
          for (int j = 0; j < kDJ; ++j) dn_math<WF>(st[j], s[j], acc);
        }
        const float v = rows_reduce<kDR>(acc, dpart, wave, lane);
        hand_over();
        if (tid < kDR) p.out[size_t(t) * H + n0 + tid] = poisoned ? uint16_t(0x7fc0) : f32_to_bf16(v);
      }
    }
    const int f = phase_of(it);
    if (f < 2) {
      pend_f = f;
      ++pend_n;
    }
    __syncthreads();
    item = s_next;
    __syncthreads();  // s_next is rewritten only after every thread has read it
    if (pend_n && (item >= total || phase_of(int(item)) != pend_f)) {  // end of a run: count it
      count_items(c, pend_f, q, pend_n, pend_f == 0 ? b1 : b2, pend_f == 0 ? b2 : b3);
      pend_n = 0;
    }
  }
  // exit count; the last workgroup out resets the counters and advances the
  // epoch (the next launch on this workspace starts after this one ends)
  if (tid == 0) {
    const int G = int(gridDim.x), s = blockIdx.x % kQ;
    const unsigned cnt = unsigned(G / kQ + (s < G % kQ));
    int last = 0;
    if (atomic_inc(c.exit_stripe(s)) + 1 == cnt) last = atomic_inc(c.exit_summary()) + 1 == unsigned(min(G, kQ));
    s_last = last;
  }
  __syncthreads();
  if (s_last) {
    for (int l = 1 + tid; l < kCtrLines; l += 256) store_agent(c.base + l * kLine, 0u);
    // modulo 0xffffffff: the epoch never reaches 0xffffffff, so consecutive
    // launches always get different tags (tag = epoch + 1)
    if (tid == 0) store_agent(c.epoch(), (epoch + 1u) % 0xffffffffu);
  }
}

template <int WF, bool XG, int MAXT>
hipError_t launch_fused(const FusedDecodeParams& p, hipStream_t s) {
  const size_t lds = XG ? 0 : size_t(p.d.T) * p.d.H * 2;
  if (lds > size_t(kFusedXLdsMax) || p.d.H % 8 || p.d.T > MAXT || (XG && p.d.gamma))
    return hipErrorInvalidValue;
  // resident capacity of the device for this LDS size (more workgroups would only queue)
  static int grid_for_dev[64] = {};
  static size_t lds_for_dev[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int grid = dev < 64 && lds_for_dev[dev] == lds + 1 ? grid_for_dev[dev] : 0;
  if (grid == 0) {
    int per_cu = 0, cus = 0;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fused_decode_kernel<WF, XG, MAXT>, 256, lds)) !=
        hipSuccess)
      return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    grid = std::max(std::max(per_cu, 1) * cus, kQ);
    if (dev < 64) {
      grid_for_dev[dev] = grid;
      lds_for_dev[dev] = lds + 1;  // +1: a cached size of 0 is not "unset"
    }
  }
  grid = std::max(grid, p.d.rp.E);  // one workgroup per router row
  hipLaunchKernelGGL((fused_decode_kernel<WF, XG, MAXT>), dim3(grid), dim3(256), lds, s, p);
  return hipGetLastError();
}

template <int WF>
hipError_t launch_fused_x(const FusedDecodeParams& p, hipStream_t s) {
  if (size_t(p.d.T) * p.d.H * 2 > size_t(kFusedXLdsMax)) return launch_fused<WF, true, kRouteGemvMaxT>(p, s);
  if (p.d.T == 1) return launch_fused<WF, false, 1>(p, s);
  if (p.d.T <= 4) return launch_fused<WF, false, 4>(p, s);
  return launch_fused<WF, false, kRouteGemvMaxT>(p, s);
}

}  // namespace

hipError_t launch_fused_decode(const FusedDecodeParams& p, hipStream_t s) {
  if (p.d.Is && p.d.swfmt != p.wfmt) return hipErrorInvalidValue;
  switch (p.wfmt) {
    case W_BF16: return launch_fused_x<W_BF16>(p, s);
    case W_FP8_B128: return launch_fused_x<W_FP8_B128>(p, s);
    default: return launch_fused_x<W_MXFP8>(p, s);
  }
}

}  // namespace moe
