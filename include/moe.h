/*
 * moe.h - C ABI of a single-GPU Mixture-of-Experts layer forward for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer is the MoE block of the DSV2-236B-MegaKernel README's flowchart
 * ("What runs inside the single launch", stages N, O, P1/Q1, P2/Q2 and the
 * sum of stage R), with every expert resident on the one GPU:
 *
 *   logits = x . Wr^T (+ bias)                          (stage N)
 *   s      = softmax(logits) over all experts;           (stage O)
 *            keep the topk_groups groups with the largest max member score,
 *            take the topk experts of those groups, w = route_scale * s
 *   dispatch of the T*topk (token, slot) pairs into per-expert segments
 *            (Mixture-of-Kittens, Figure 1: GPU-side dispatch scheduling)
 *   per expert e: h = SiLU(x.Wg_e^T) * (x.Wu_e^T); Y = h.Wd_e^T  (P1, P2)
 *   shared expert S(x) on every token, unweighted       (Q1, Q2)
 *   out    = bf16( sum_j w_j * Y_j + S )                 (stage R's sum,
 *            without residual or norm)
 *
 * Conventions for every entry point
 * - Pointers are device pointers unless marked (host).  bf16 tensors are
 *   passed as uint16_t bit patterns.  All matrices are row-major with the
 *   last index contiguous.  Device pointers must be 16-byte aligned.
 * - Every call is asynchronous on `stream`; nothing synchronises with the
 *   host and no device-side count is read back (Mixture-of-Kittens,
 *   Abstract: no CPU-GPU synchronisation).  Launch errors are reported as
 *   MOE_EHIP; faults inside kernels surface at the caller's next sync.
 * - The caller owns all memory.  The library never allocates.  Calls that
 *   take a workspace need `ws_bytes` >= moe_workspace_size(); the workspace
 *   must be zero-filled once before its first use (torch.zeros is enough):
 *   its first 48 KiB hold the work queues, counters, a launch epoch and
 *   tagged router logits of moe_forward's single-launch path; every call
 *   leaves the queues and counters zero again and advances the epoch.  Calls sharing
 *   one workspace must be ordered on one stream; overlapping calls on one
 *   workspace race.
 * - Status codes: nothing is thrown across the ABI.  Host-side validation
 *   runs before any launch, so a failed check launches nothing.
 *     MOE_EINVAL        null pointer, T < 0, hidden/inter <= 0,
 *                       n_experts % n_groups != 0, topk_groups not in
 *                       [1, n_groups], topk not in [1, candidates], topk >
 *                       16, route_scale not finite, bad format code
 *     MOE_EALIGN        a pointer not 16-byte aligned, or hidden, inter or
 *                       shared_inter not a multiple of 128
 *     MOE_EUNSUPPORTED  n_experts > 256, n_groups > 64, an FP8_B128 format
 *                       with hidden, inter or shared_inter above 8192, or a weight /
 *                       activation format pair that no kernel implements
 *     MOE_EWORKSPACE    ws_bytes below moe_workspace_size()
 *     MOE_EHIP          a HIP launch failed
 *     MOE_EWAIT         (moe_workspace_check only) a bounded wait inside a
 *                       single-launch moe_forward gave up; that call's
 *                       output holds NaN rows
 *   T = 0 is a no-op returning MOE_OK.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,
  MOE_EUNSUPPORTED = 2,
  MOE_EALIGN = 3,
  MOE_EWORKSPACE = 4,
  MOE_EHIP = 5,
  MOE_EWAIT = 6
} moe_status;

/* Weight formats (DSV2-236B-MegaKernel README, "Results": per-128
 * block-scaled FP8; Mixture-of-Kittens, Table 2: MXFP8 routed experts and a
 * BF16 shared expert).  For a weight matrix W[N][K]:
 *   MOE_W_BF16      W bf16 [N][K], no scales
 *   MOE_W_FP8_B128  codes e4m3fn u8 [N][K] and fp32 scales [N/128][K/128];
 *                   W[n][k] = dec(q[n][k]) * S[n/128][k/128]
 *   MOE_W_MXFP8     codes e4m3fn u8 [N][K] and e8m0 u8 scales [N][K/32];
 *                   W[n][k] = dec(q[n][k]) * 2^(E[n][k/32] - 127)          */
typedef enum { MOE_W_BF16 = 0, MOE_W_FP8_B128 = 1, MOE_W_MXFP8 = 2 } moe_wfmt;

/* Activation formats: how the rows entering each FFN matmul (x, then h) are
 * quantised ("From 35 to 873 tokens/s", Rounds 12-15: MXFP8 quantisation of
 * the expert inputs).  Per row:
 *   MOE_A_NONE        bf16 x as given; h kept in fp32 (bf16 for bf16 weights)
 *   MOE_A_FP8_1X128   per 128 columns: s = fl32(amax/448) (1 if amax = 0),
 *                     q = RNE_e4m3(fl32(v/s)) saturating; scales fp32
 *                     [rows][cols/128]
 *   MOE_A_MXFP8_1X32  per 32 columns: X = 2^(floor(log2 amax) - 8) clamped to
 *                     the e8m0 range (1 if amax = 0), q = RNE_e4m3(v/X)
 *                     saturating; scales e8m0 u8 [rows][cols/32]
 * Supported (weight, activation) pairs: (BF16, NONE), (FP8_B128, NONE),
 * (FP8_B128, FP8_1X128), (MXFP8, MXFP8_1X32), (MXFP8, NONE).  Pairs with
 * activation NONE and FP8/MXFP8 weights run on the small-batch GEMV path
 * at any T (slow for large T).                                              */
typedef enum { MOE_A_NONE = 0, MOE_A_FP8_1X128 = 1, MOE_A_MXFP8_1X32 = 2 } moe_afmt;

/* Layer geometry and formats (host struct).  Experts are grouped into
 * n_groups contiguous id ranges of n_experts/n_groups (stage O's
 * "8 groups x 20").  shared_inter = 0 means no shared expert. */
typedef struct {
  int32_t hidden;        /* H */
  int32_t n_experts;     /* E <= 256 */
  int32_t n_groups;      /* G, divides E */
  int32_t topk_groups;   /* TG in [1, G] */
  int32_t topk;          /* K in [1, min(16, TG*E/G)] */
  int32_t inter;         /* I, routed expert intermediate */
  int32_t shared_inter;  /* Is, fused shared intermediate, 0 = none */
  float route_scale;     /* w = route_scale * softmax score */
  int32_t routed_wfmt;   /* moe_wfmt */
  int32_t shared_wfmt;   /* moe_wfmt */
  int32_t routed_afmt;   /* moe_afmt */
  int32_t shared_afmt;   /* moe_afmt */
} moe_config;

/* One set of expert weights (device pointers).  gate, up: [n][I][H];
 * down: [n][H][I]; n = E for routed, 1 for shared.  Scales per moe_wfmt
 * with the same leading [n]; NULL for BF16. */
typedef struct {
  const void* gate;
  const void* up;
  const void* down;
  const void* gate_s;
  const void* up_s;
  const void* down_s;
} moe_ffn_weights;

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(int32_t status);

/* Bytes of workspace that every call below needs for up to max_tokens
 * tokens with this config.  Host-only; no GPU work. */
moe_status moe_workspace_size(const moe_config* cfg /*host*/, int32_t max_tokens,
                              size_t* bytes /*host*/);

/* Stage M of the DSV2-236B-MegaKernel README flowchart (the post-attention
 * RMSNorm with weight gamma4, just before the router GEMV): gamma bf16 [H]
 * (device), eps >= 0.  The layer input becomes
 *   x = bf16( fl32( fl32(h * gamma) * r ) ),  r = fl32( 1 / sqrt(mean(h^2) + eps) )
 * per row, with mean(h^2) in float64 and each rounding to nearest even. */
typedef struct {
  const uint16_t* gamma;
  float eps;
} moe_norm;

/* Stages N + O: router GEMV and group-limited greedy top-k.
 * x bf16 [T][H]; w_router bf16 [E][H]; bias fp32 [E] or NULL (added to the
 * logits before the softmax).  Outputs topk_ids int32 [T][K] in descending
 * score order (ties to the lower id) and topk_w fp32 [T][K] =
 * route_scale * score (no renormalisation over the selected experts).
 * Every id is in [0, E), whatever the logits: -inf logits (a masking bias)
 * tie below every finite logit, lowest id first, with weight 0; a token with
 * a NaN or +inf logit has no defined softmax, takes the lowest ids of the
 * lowest groups and gets NaN weights. */
moe_status moe_route(const moe_config* cfg /*host*/, const uint16_t* x, int32_t T,
                     const uint16_t* w_router, const float* bias, int32_t* topk_ids,
                     float* topk_w, void* ws, size_t ws_bytes, hipStream_t stream);

/* Dispatch (Mixture-of-Kittens, Figure 1: dispatch scheduling on the GPU;
 * "From 35 to 873 tokens/s", Rounds 12-15: the router emits the layout the
 * experts need).  Flat slot p = t*K + j.  Outputs:
 *   expert_offsets int32 [E+1]: exclusive prefix sum of per-expert counts
 *   perm_src int32 [T*K]: slot held by permuted row pos, stable (expert
 *            ascending, then p ascending)
 *   inv_pos int32 [T*K]: permuted row of slot p (-1 if its id is outside
 *            [0, E); such slots are dropped)
 *   x_perm (optional, NULL to skip; needs x): row pos = x[perm_src[pos]/K]
 *            in the routed activation format: bf16 [T*K][H] for NONE, else
 *            e4m3 codes u8 [T*K][H] with scales written to x_perm_scale
 *            (fp32 [T*K][H/128] or e8m0 u8 [T*K][H/32]). */
moe_status moe_permute(const moe_config* cfg /*host*/, const int32_t* topk_ids, int32_t T,
                       const uint16_t* x, int32_t* expert_offsets, int32_t* perm_src,
                       int32_t* inv_pos, void* x_perm, void* x_perm_scale, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/* Stages M (optional) + N + O and the dispatch in one call, the router
 * emitting the layout the experts need ("From 35 to 873 tokens/s", Rounds
 * 12-15; Mixture-of-Kittens, Figure 1): the norm, the router, the top-k, the
 * routed experts' input in their activation format and the per-block expert
 * counts in one launch, then the stable scatter.  Any T >= 1.
 *   h bf16 [T][H]: the pre-norm rows when norm != NULL, else x itself.
 *   Outputs as moe_route and moe_permute (topk_ids, topk_w, expert_offsets,
 *   perm_src, inv_pos), plus, each optional (NULL to skip):
 *   x_out bf16 [T][H]: x (normalised when norm != NULL);
 *   xq u8 [T][H] + xq_scale: x quantised in the routed activation format
 *   (per token, not gathered: row perm_src[pos]/K feeds permuted row pos);
 *   MOE_EINVAL if xq is given and that format is MOE_A_NONE. */
moe_status moe_route_dispatch(const moe_config* cfg /*host*/, const uint16_t* h, int32_t T,
                              const moe_norm* norm /*host struct or NULL*/, const uint16_t* w_router,
                              const float* bias, int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                              int32_t* perm_src, int32_t* inv_pos, uint16_t* x_out, void* xq, void* xq_scale,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/* Stages P1+P2 (which = 0, routed) or Q1+Q2 (which = 1, shared): the SwiGLU
 * FFN y = (SiLU(x.Wg^T) * (x.Wu^T)).Wd^T on `rows` rows.
 *   x: bf16 [rows][H] when x_scale is NULL (quantised here per the afmt),
 *      else e4m3 codes u8 [rows][H] already quantised with x_scale in the
 *      afmt's scale layout.
 *   seg_offsets: routed only, int32 [E+1] device array splitting the rows
 *      into per-expert segments (as written by moe_permute); NULL for shared.
 *   y: fp32 [rows][H], unweighted. */
moe_status moe_expert_ffn(const moe_config* cfg /*host*/, int32_t which, const void* x,
                          const void* x_scale, int32_t rows, const int32_t* seg_offsets,
                          const moe_ffn_weights* weights /*host struct, device ptrs*/,
                          float* y, void* ws, size_t ws_bytes, hipStream_t stream);

/* Stage R's sum, deterministic (a fixed order, no float atomics):
 * out[t] = bf16( sum_{j=0..K-1} topk_w[t][j] * y_perm[inv_pos[t*K+j]]
 *                + y_shared[t] ).
 * y_perm fp32 [T*K][H]; inv_pos int32 [T*K] (-1 entries are skipped);
 * topk_w fp32 [T][K]; y_shared fp32 [T][H] or NULL; out bf16 [T][H]. */
moe_status moe_combine(const moe_config* cfg /*host*/, const float* y_perm, const int32_t* inv_pos,
                       const float* topk_w, const float* y_shared, int32_t T, uint16_t* out,
                       hipStream_t stream);

/* The whole layer: route, dispatch, routed and shared FFNs, combine.
 * out bf16 [T][H].  topk_ids_out int32 [T][K] and topk_w_out fp32 [T][K]
 * may be NULL.  Numerics depend only on cfg: every path honours the same
 * activation format.
 * Paths: T <= 8 with both activation formats MOE_A_NONE, T * H * 2 <= 80 KiB
 * and one weight format for routed and shared experts runs as ONE
 * persistent launch (the DSV2-236B-MegaKernel README's single-launch idea,
 * "What runs inside the single launch"): workgroups take router rows,
 * shared gate/up, routed gate/up and down+combine items in that order (a
 * static round robin when there are at most 16 items per workgroup, else
 * claimed from queues in the workspace), and wait (bounded) only for earlier
 * items.  Waits give up after about 0.2 s: int32 word 0 of the workspace
 * then becomes nonzero (sticky; moe_workspace_check reports and clears it)
 * and the rows of `out` written by the workgroup that gave up are NaN.  With
 * the device to itself a wait lasts microseconds.  Progress needs every
 * workgroup of the launch to become resident (static round robin: each owns
 * a fixed share of the items) or max(E, 32) of them resident at once
 * (claims); the launch asks for the device's resident capacity, so only a
 * kernel on another stream that holds CUs for longer than the wait bound can
 * make a wait give up.  Other T <= 4 cases run in four to six launches
 * (T <= 8 when no grouped-GEMM kernel serves the formats); larger T runs the
 * dispatch + grouped-GEMM path (or the GEMV path for formats it lacks). */
moe_status moe_forward(const moe_config* cfg /*host*/, const uint16_t* x, int32_t T,
                       const uint16_t* w_router, const float* bias,
                       const moe_ffn_weights* routed /*host struct*/,
                       const moe_ffn_weights* shared /*host struct or NULL*/, uint16_t* out,
                       int32_t* topk_ids_out, float* topk_w_out, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* The whole layer from the pre-norm rows h: stage M (norm, required), then
 * exactly moe_forward on the normalised x.  x_out (bf16 [T][H], NULL ok)
 * receives x.  The batched path normalises inside its fused router launch,
 * the single launch stages the normalised rows in LDS itself; the other
 * small-T paths run the norm as a first launch. */
moe_status moe_forward_norm(const moe_config* cfg /*host*/, const uint16_t* h, int32_t T,
                            const moe_norm* norm /*host struct*/, const uint16_t* w_router, const float* bias,
                            const moe_ffn_weights* routed /*host struct*/,
                            const moe_ffn_weights* shared /*host struct or NULL*/, uint16_t* out,
                            int32_t* topk_ids_out, float* topk_w_out, uint16_t* x_out, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* Gradient buffers of one set of experts (device pointers, bf16):
 * gate, up [n][I][H]; down [n][H][I]; n = E for routed, 1 for shared. */
typedef struct {
  void* gate;
  void* up;
  void* down;
} moe_ffn_grads;

/* Bytes of workspace moe_backward needs for up to max_tokens tokens
 * (MOE_EUNSUPPORTED for formats it does not serve). */
moe_status moe_backward_workspace_size(const moe_config* cfg /*host*/, int32_t max_tokens,
                                       size_t* bytes /*host*/);

/* The layer's backward pass (Mixture-of-Kittens, Table 1: the MoE layer's
 * backward beside its forward), for bf16 weights and unquantised
 * activations (MOE_EUNSUPPORTED otherwise).  Given dy bf16 [T][H], the
 * gradient of the layer output out = sum_j w_j Y_j + S of moe_forward on the
 * same x and weights, it writes the gradients of <dy, out>:
 *   dx bf16 [T][H]; d_router bf16 [E][H]; d_bias fp32 [E] (NULL to skip);
 *   d_routed (every expert's gate, up, down; zero for experts no token
 *   chose) and d_shared (NULL when there is no shared expert), bf16.
 * The routing is recomputed (the same ids as the forward: the selection is
 * piecewise constant, so gradients flow only through the routing weights
 * w = route_scale * softmax(logits)[id]); so are the gate/up products and
 * the routed outputs.  Every output is overwritten, none accumulated.
 * Reductions run in a fixed order: repeated calls give identical bits. */
moe_status moe_backward(const moe_config* cfg /*host*/, const uint16_t* x, int32_t T,
                        const uint16_t* w_router, const float* bias,
                        const moe_ffn_weights* routed /*host struct*/,
                        const moe_ffn_weights* shared /*host struct or NULL*/, const uint16_t* dy,
                        uint16_t* dx, uint16_t* d_router, float* d_bias,
                        const moe_ffn_grads* d_routed /*host struct*/,
                        const moe_ffn_grads* d_shared /*host struct or NULL*/, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* moe_forward without a workspace argument, for callers that cannot
 * allocate (code under graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, paths and results as moe_forward; the
 * workspace is a 32 MiB device array inside the library, one per GPU,
 * resolved on the first call on a device (whose 48 KiB counter block that
 * call clears on `stream`) and held until the process ends.  No call allocates
 * memory or creates a stream.  Every call on a GPU uses that GPU's one
 * array: calls that overlap on one GPU (several streams or threads) race,
 * so order them on one stream.  The shared expert always runs in order on
 * `stream`.  MOE_EWORKSPACE when the call needs more than 32 MiB of
 * workspace (moe_workspace_size for T tokens); MOE_EHIP if the array cannot
 * be resolved.  A bounded wait of the single launch that gives up shows as
 * NaN rows of `out` (the array's error word is not exposed). */
moe_status moe_forward_noalloc(const moe_config* cfg /*host*/, const uint16_t* x, int32_t T,
                               const uint16_t* w_router, const float* bias,
                               const moe_ffn_weights* routed /*host struct*/,
                               const moe_ffn_weights* shared /*host struct or NULL*/, uint16_t* out,
                               int32_t* topk_ids_out, float* topk_w_out, hipStream_t stream);

/* Reports the sticky error word of a workspace used by moe_forward's
 * single-launch path: MOE_EWAIT if a bounded wait of an earlier call gave up
 * (its output rows are NaN), else MOE_OK.  clear != 0 resets the word.
 * Host-synchronising: it copies the word to the host after the work queued on
 * `stream` so far and waits for that copy, so it is not for use under graph
 * capture.  MOE_EINVAL for a null ws or ws_bytes below 4. */
moe_status moe_workspace_check(void* ws, size_t ws_bytes, int32_t clear, hipStream_t stream);

/* Diagnostics of the device FP8 codec (the conversions every kernel uses):
 * decode n e4m3 codes to fp32, and encode n fp32 values with the library's
 * round-to-nearest-even saturating rule.  For tests of the codec itself. */
moe_status moe_debug_e4m3_decode(const uint8_t* codes, float* out, int32_t n, hipStream_t stream);
moe_status moe_debug_e4m3_encode(const float* in, uint8_t* codes, int32_t n, hipStream_t stream);

/* Test hooks.  moe_debug_ws_offset: byte offset, inside a workspace planned
 * for max_tokens tokens, of a region that moe_forward's batched path fills:
 * region 0 expert_offsets int32 [E+1], 1 perm_src int32 [T*K], 2 inv_pos
 * int32 [T*K], 3 the grouped-GEMM tile list int32 [2 * n_tiles] (expert,
 * first row of the tile within the expert's segment), 4 n_tiles int32.
 * moe_debug_ffn_tile_rows: rows per tile of the grouped GEMMs that the
 * routed (which = 0) or shared (1) FFN runs on at batched sizes (256: the
 * large-tile kernel, 128: the other), or -1 for an invalid config. */
moe_status moe_debug_ws_offset(const moe_config* cfg /*host*/, int32_t max_tokens, int32_t region,
                               size_t* offset /*host*/);
int32_t moe_debug_ffn_tile_rows(const moe_config* cfg /*host*/, int32_t which);

/* Debug check of the dispatch that moe_forward's batched path (T > 8) or
 * moe_route_dispatch left in a workspace planned for T tokens, against the
 * ids of that call (device, int32 [T][K]): one single-workgroup launch on
 * `stream` that only reads, and ORs into *flags (device int32; the caller
 * zeroes it and reads it after synchronising) bit 0 if expert_offsets[0]
 * != 0 or the offsets decrease, bit 1 if expert_offsets[E] != T*K, bit 2 for
 * an id outside [0, E), bit 3 if perm_src is not a bijection of [0, T*K) or
 * inv_pos not its inverse, bit 4 if a position of an expert's segment holds a
 * slot of another expert or a segment is not in ascending slot order, bit 5
 * if the grouped-GEMM tile list does not cover each segment in order with
 * ceil(count / rows) tiles.  These are the properties the grouped GEMMs and
 * the combine rely on (Mixture-of-Kittens, Figure 1: the dispatch layout the
 * expert GEMMs consume).  MOE_EINVAL / MOE_EWORKSPACE for bad arguments. */
moe_status moe_debug_validate_dispatch(const moe_config* cfg /*host*/, int32_t T, const int32_t* topk_ids,
                                       const void* ws, size_t ws_bytes, int32_t* flags, hipStream_t stream);

/* Measurement hook: arm (events != NULL, n_events >= 2) or disarm (NULL) a
 * launch trace.  While armed, each kernel launch of the entry points records
 * events[2i] before and events[2i+1] after launch i on the call's stream,
 * for the first n_events/2 launches since arming.  The caller creates the
 * events (with timing) and keeps them alive while armed.  Process-global and
 * not thread-safe: one benchmarking thread at a time. */
moe_status moe_debug_trace(hipEvent_t* events /*host array*/, int32_t n_events);
/* Launches recorded since the trace was armed, and the kernel name of one. */
int32_t moe_debug_trace_count(void);
const char* moe_debug_trace_name(int32_t i);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
