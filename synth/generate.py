"""Seeded draws of one MoE layer's inputs.

Every tensor is drawn from torch's generator on the requested device, seeded
from numpy's SeedSequence([42, config, replica, kind, index, attempt]); the
root seed 42 follows the fixed-seed protocol of "From 35 to 873 tokens/s: the
DeepSeek-V4.1 Flash Kernel Journey", section "Benchmarking Honestly".  The
same seed gives the same values on one device type; a test draws once and
hands the very same tensors to both the HIP path and the oracle.

kind: 0 tokens x (the pre-norm h for a layer with the stage M norm), 1
router weight, 2 router-bias ranks, 3/4/5 routed gate/up/down, 6/7/8 shared
gate/up/down, 9 per-token redraws, 10 the norm weight gamma.

Values are fp32 N(0,1)*sigma, then rounded to bf16 (torch RNE) or quantised
to e4m3fn codes with per-format scales.  The weight quantisers below only
prepare inputs: a checkpoint is quantised offline before a forward pass (the
DSV2-236B-MegaKernel README, "Layout", names its block-FP8 quantiser).
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import LayerConfig

ROOT_SEED = 42
FP8_MAX = 448.0


def seed_of(*parts) -> int:
    st = np.random.SeedSequence([ROOT_SEED, *[int(p) for p in parts]]).generate_state(2, np.uint32)
    return int((int(st[0]) << 31) ^ int(st[1])) & ((1 << 63) - 1)


def _randn(shape, seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _quant_b128(w):
    """w fp32 [n][N][K] -> (codes u8 [n][N][K], scales f32 [n][N/128][K/128])."""
    n, N, K = w.shape
    blk = w.view(n, N // 128, 128, K // 128, 128)
    amax = blk.abs().amax(dim=(2, 4))
    s = amax / FP8_MAX
    s = torch.where(amax > 0, s, torch.ones_like(s))
    q = (blk / s[:, :, None, :, None]).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).reshape(n, N, K).contiguous(), s.contiguous()


def _quant_mx(w):
    """w fp32 [n][N][K] -> (codes u8 [n][N][K], e8m0 u8 [n][N][K/32])."""
    n, N, K = w.shape
    blk = w.view(n, N, K // 32, 32)
    amax = blk.abs().amax(dim=3)
    _, ex = torch.frexp(amax)                # amax = m * 2^ex, m in [0.5, 1)
    xe = (ex.to(torch.int32) - 1 - 8).clamp(-127, 127)
    xe = torch.where(amax > 0, xe, torch.zeros_like(xe))
    scale = torch.ldexp(torch.ones_like(amax), xe.to(torch.float32))
    q = (blk / scale[..., None]).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).reshape(n, N, K).contiguous(), (xe + 127).to(torch.uint8).contiguous()


def _quantise(w, fmt):
    if fmt == "bf16":
        return w.to(torch.bfloat16).contiguous(), None
    if fmt == "fp8_b128":
        return _quant_b128(w)
    if fmt == "mxfp8":
        return _quant_mx(w)
    raise ValueError(fmt)


@dataclass
class ExpertWeights:
    """gate/up [n][I][H], down [n][H][I]; codes (u8) or bf16; scales or None."""
    fmt: str
    n: int
    inter: int
    hidden: int
    gate: torch.Tensor
    up: torch.Tensor
    down: torch.Tensor
    gate_s: Optional[torch.Tensor]
    up_s: Optional[torch.Tensor]
    down_s: Optional[torch.Tensor]

    def to(self, device):
        f = lambda t: None if t is None else t.to(device)
        return ExpertWeights(self.fmt, self.n, self.inter, self.hidden, f(self.gate), f(self.up),
                             f(self.down), f(self.gate_s), f(self.up_s), f(self.down_s))

    def expert(self, e):
        """Host numpy arrays of expert e: (gate, up, down, gate_s, up_s, down_s)."""
        def h(t):
            if t is None:
                return None
            t = t[e].cpu()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16)
            return t.numpy()
        return tuple(h(t) for t in (self.gate, self.up, self.down, self.gate_s, self.up_s, self.down_s))

    def nbytes_per_expert(self):
        tot = 0
        for t in (self.gate, self.up, self.down, self.gate_s, self.up_s, self.down_s):
            if t is not None:
                tot += t[0].numel() * t.element_size()
        return tot


def make_experts(cfg: LayerConfig, shared: bool, device, replica=0) -> ExpertWeights:
    n = 1 if shared else cfg.n_experts
    inter = cfg.shared_inter if shared else cfg.inter
    fmt = cfg.shared_wfmt if shared else cfg.routed_wfmt
    H = cfg.hidden
    k0 = 6 if shared else 3
    parts = {"gate": [], "up": [], "down": []}
    scales = {"gate": [], "up": [], "down": []}
    for e in range(n):
        for kk, name in enumerate(("gate", "up", "down")):
            shape = (1, H, inter) if name == "down" else (1, inter, H)
            w = _randn(shape, seed_of(cfg.index, replica, k0 + kk, e), device) * cfg.w_sigma
            q, s = _quantise(w, fmt)
            parts[name].append(q)
            scales[name].append(s)
            del w
    cat = lambda xs: torch.cat(xs, 0).contiguous()
    sc = lambda xs: None if xs[0] is None else cat(xs)
    return ExpertWeights(fmt, n, inter, H, cat(parts["gate"]), cat(parts["up"]), cat(parts["down"]),
                         sc(scales["gate"]), sc(scales["up"]), sc(scales["down"]))


@dataclass
class LayerInputs:
    cfg: LayerConfig
    x: torch.Tensor                 # bf16 [T][H]
    w_router: torch.Tensor          # bf16 [E][H]
    bias: Optional[torch.Tensor]    # f32 [E] or None
    routed: ExpertWeights
    shared: Optional[ExpertWeights]
    replica: int = 0
    gamma: Optional[torch.Tensor] = None   # bf16 [H] norm weight (norm layers)

    @property
    def device(self):
        return self.x.device


def draw_tokens(cfg: LayerConfig, device, replica=0, tokens=None):
    T = cfg.tokens if tokens is None else tokens
    return (_randn((T, cfg.hidden), seed_of(cfg.index, replica, 0, T), device) * cfg.x_sigma).to(torch.bfloat16)


def make_inputs(cfg: LayerConfig, device="cpu", replica=0, with_experts=True) -> LayerInputs:
    device = torch.device(device)
    x = draw_tokens(cfg, device, replica)
    wr = (_randn((cfg.n_experts, cfg.hidden), seed_of(cfg.index, replica, 1, 0), device) * cfg.w_sigma).to(torch.bfloat16)
    bias = None
    if cfg.zipf_bias > 0:
        g = torch.Generator(device="cpu")
        g.manual_seed(seed_of(cfg.index, replica, 2, 0))
        ranks = torch.randperm(cfg.n_experts, generator=g).to(torch.float32) + 1.0
        bias = (-cfg.zipf_bias * torch.log(ranks)).to(device)
    gamma = None
    if cfg.norm:
        gamma = (1.0 + 0.1 * _randn((cfg.hidden,), seed_of(cfg.index, replica, 10, 0), device)).to(torch.bfloat16)
    routed = shared = None
    if with_experts:
        routed = make_experts(cfg, False, device, replica)
        if cfg.shared_inter > 0:
            shared = make_experts(cfg, True, device, replica)
    return LayerInputs(cfg, x.contiguous(), wr.contiguous(), bias, routed, shared, replica, gamma)


def redraw_tokens(inp: LayerInputs, tokens, attempt: int):
    """Redraw rows `tokens` of x in place (deterministic in (token, attempt))."""
    cfg = inp.cfg
    for t in tokens:
        row = _randn((cfg.hidden,), seed_of(cfg.index, inp.replica, 9, int(t), attempt), inp.device) * cfg.x_sigma
        inp.x[int(t)] = row.to(torch.bfloat16)
