"""CPU oracle for one Mixture-of-Experts layer forward (test infrastructure).

This package is test infrastructure only: tests, the smoke check and the
benchmark's CPU-baseline leg call it; the HIP product path never does.  It
is plain, slow, float64 numpy, written from the pages' description of the
layer and sharing no code with the HIP library.

Sources (page title, section):
* DSV2-236B-MegaKernel README, "What runs inside the single launch"
  flowchart, MoE stages N (router GEMV), O (softmax, group-limited greedy:
  max over 8 groups x 20, top-3 groups, top-6 experts, w = score x 16.0),
  P1/Q1 (gate+up, SiLU(g) x u), P2/Q2 (down), R (h += shared_out + routed);
  "Results" (per-128 block-scaled FP8).
  Stage M (post-attention RMSNorm with weight gamma4) precedes the router.
* Mixture-of-Kittens, Abstract and Figure 1 (GPU-side router projection,
  top-k and dispatch scheduling; token dispatch into expert FFNs, token
  combine); Table 2 caption (MXFP8 routed experts, BF16 shared expert).
* "From 35 to 873 tokens/s: the DeepSeek-V4.1 Flash Kernel Journey",
  "Rounds 12-15" (router emits the experts' layout; MXFP8 input
  quantisation of the expert inputs; expert-weighted reduction plus
  shared-expert add).

Parity status of each function is stated in its docstring; every function
here is pinned by a CPU test against something other than itself (library
routines, closed forms, brute force, invariants).
"""
from .fp8 import e4m3_decode, e4m3_encode, e8m0_decode  # noqa: F401
from .moe import (  # noqa: F401
    bf16_to_f64, f32_to_bf16_bits, rmsnorm, dequant_weight, quant_act, route, route_margins, permute,
    expert_ffn, combine, forward, forward_tokens, forward_dense_masked, OracleResult,
)
from .backward import backward, ffn_backward, BackwardResult  # noqa: F401
