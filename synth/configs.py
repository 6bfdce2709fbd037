"""The five layer workloads, with the sizes the pages give.

* DeepSeek-V2 geometry (hidden 5120, 160 routed experts in 8 groups, top-3
  groups, top-6 experts, route scale 16.0, expert intermediate 1536, two
  shared experts fused to 3072): DSV2-236B-MegaKernel README, "What runs
  inside the single launch" flowchart, stages N/O/P1/Q1/P2/Q2, and the
  "Model geometry" paragraph.
* 2,048-token, hidden-7168 shape with uniformly random top-4 routes, MXFP8
  routed experts and a BF16 shared expert: Mixture-of-Kittens, Figure 4
  caption (token width 7,168, 4 random routes), Figure 7 caption (2,048
  tokens per GPU) and Table 2 caption (MXFP8 routed, BF16 shared).

Format names:
  weights      "bf16" | "fp8_b128" (e4m3fn, fp32 scale per 128x128 block)
               | "mxfp8" (e4m3fn, e8m0 scale per 1x32 along K)
  activations  "none" (bf16 rows fed as they are) | "fp8_1x128" (e4m3fn,
               fp32 scale per row per 128 columns) | "mxfp8_1x32" (e4m3fn,
               e8m0 scale per row per 32 columns)
"""
from dataclasses import dataclass, replace

WFMT = {"bf16": 0, "fp8_b128": 1, "mxfp8": 2}
AFMT = {"none": 0, "fp8_1x128": 1, "mxfp8_1x32": 2}


@dataclass(frozen=True)
class LayerConfig:
    name: str
    index: int            # seed component
    tokens: int
    hidden: int
    n_experts: int
    n_groups: int
    topk_groups: int
    topk: int
    route_scale: float
    inter: int
    shared_inter: int     # 0 = no shared expert
    routed_wfmt: str
    shared_wfmt: str
    routed_afmt: str
    shared_afmt: str
    zipf_bias: float = 0.0  # >0: router bias b[e] = -s*ln(rank_e)
    x_sigma: float = 1.0
    w_sigma: float = 0.02
    norm: bool = False      # stage M RMSNorm first: x is then the pre-norm h
    norm_eps: float = 1e-6

    def with_tokens(self, t):
        return replace(self, tokens=t)

    def derive(self, **kw):
        return replace(self, **kw)


CONFIGS = [
    LayerConfig("tiny_8tok", 0, 8, 256, 16, 4, 2, 4, 1.0, 128, 128,
                "bf16", "bf16", "none", "none"),
    LayerConfig("dsv2_b1", 1, 1, 5120, 160, 8, 3, 6, 16.0, 1536, 3072,
                "fp8_b128", "fp8_b128", "none", "none"),
    LayerConfig("dsv2_256tok", 2, 256, 5120, 160, 8, 3, 6, 16.0, 1536, 3072,
                "fp8_b128", "fp8_b128", "fp8_1x128", "fp8_1x128"),
    LayerConfig("h7168_2048tok_mx", 3, 2048, 7168, 32, 1, 1, 4, 1.0, 2048, 2048,
                "mxfp8", "bf16", "mxfp8_1x32", "none"),
    LayerConfig("dsv2_4096tok_zipf", 4, 4096, 5120, 160, 8, 3, 6, 16.0, 1536, 3072,
                "fp8_b128", "fp8_b128", "fp8_1x128", "fp8_1x128", zipf_bias=1.2),
]


def with_norm(cfg, h_sigma=3.0):
    """The same layer preceded by the stage M RMSNorm (DSV2-236B-MegaKernel
    flowchart, stage M: post-attention RMSNorm before the router GEMV): the
    input is the pre-norm h ~ N(0, h_sigma^2), gamma ~ 1 + N(0, 0.1^2)."""
    return replace(cfg, name=cfg.name + "_norm", norm=True, x_sigma=h_sigma)


def get_config(name_or_index):
    for c in CONFIGS:
        if c.name == name_or_index or c.index == name_or_index:
            return c
    raise KeyError(name_or_index)
