"""Stage M (RMSNorm) and the fused routing step on MI355X, through the C ABI,
against the fp64 oracle: moe_route_dispatch (norm + router + top-k + routed
input + dispatch) and moe_forward_norm (the layer from the pre-norm rows).

Bars: ids, offsets, perm_src, inv_pos, the normalised x and the quantised
codes bit-exact; weights within 1e-4; outputs within 2e-2 (as for the layer
without the norm)."""
import sys

import numpy as np
import pytest
import torch

import mixture_experts_layer_router_amd as moe
import oracle
import synth
from helpers import ensure_margin, norm_of, rel_err, small_cfg

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL, WTOL = 2e-2, 1e-4


def say(*a):
    print(*a, flush=True)


ROUTE_CASES = {
    # name: (config, norm)
    "dsv2_256tok": (synth.get_config(2), False),
    "dsv2_256tok_norm": (synth.with_norm(synth.get_config(2)), True),
    "mx_2048tok_norm": (synth.with_norm(synth.get_config(3)), True),
    "zipf_4096tok_norm": (synth.with_norm(synth.get_config(4)), True),
    "bf16_ragged_37tok_norm": (synth.with_norm(small_cfg(0, tokens=37, hidden=384, n_experts=24, n_groups=3,
                                                         topk_groups=2, topk=5)), True),
    "one_token_norm": (synth.with_norm(small_cfg(1, tokens=1, hidden=640, n_experts=32, n_groups=4,
                                                 topk_groups=2, topk=3)), True),
    "e256_k8_100tok": (small_cfg(2, tokens=100, hidden=256, n_experts=256, n_groups=8, topk_groups=4, topk=8), False),
}


@pytest.mark.parametrize("name", list(ROUTE_CASES))
def test_route_dispatch(name):
    cfg, norm = ROUTE_CASES[name]
    say(f"[route_dispatch] {name}")
    inp = ensure_margin(synth.make_inputs(cfg, DEV, with_experts=False))
    T, H, E, K = cfg.tokens, cfg.hidden, cfg.n_experts, cfg.topk
    c = moe.make_config(cfg)
    ws = moe.alloc_workspace(c, T)
    ids = torch.empty(T, K, dtype=torch.int32, device=DEV)
    w = torch.empty(T, K, dtype=torch.float32, device=DEV)
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    perm = torch.empty(T * K, dtype=torch.int32, device=DEV)
    inv = torch.empty(T * K, dtype=torch.int32, device=DEV)
    xo = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    af = cfg.routed_afmt
    xq = xs = None
    if af != "none":
        xq = torch.empty(T, H, dtype=torch.uint8, device=DEV)
        xs = torch.empty(T, H // 128 if af == "fp8_1x128" else H // 32,
                         dtype=torch.float32 if af == "fp8_1x128" else torch.uint8, device=DEV)
    nm = moe.make_norm(inp.gamma, cfg.norm_eps) if norm else None
    moe.route_dispatch(c, inp.x, nm, inp.w_router, inp.bias, ids, w, off, perm, inv, xo, xq, xs, ws)
    torch.cuda.synchronize()
    x = oracle.rmsnorm(inp.x, inp.gamma, cfg.norm_eps)[0] if norm else inp.x.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(xo.view(torch.int16).cpu().numpy().view(np.uint16), x)
    b = None if inp.bias is None else inp.bias.double().cpu().numpy()
    r = oracle.route(oracle.bf16_to_f64(x), oracle.bf16_to_f64(inp.w_router), b, cfg)
    assert np.array_equal(ids.cpu().numpy(), r["ids"])
    assert np.max(np.abs(w.cpu().numpy() - r["w"]) / r["w"]) <= WTOL
    o_off, o_perm, o_inv = oracle.permute(r["ids"], E)
    assert np.array_equal(off.cpu().numpy(), o_off)
    assert np.array_equal(perm.cpu().numpy(), o_perm)
    assert np.array_equal(inv.cpu().numpy(), o_inv)
    if xq is not None:
        _, q, s = oracle.quant_act(oracle.bf16_to_f64(x), af, return_codes=True)
        assert np.array_equal(xq.cpu().numpy(), q)
        assert np.array_equal(xs.cpu().numpy(), s)


NORM_LAYERS = {
    "tiny_8tok_norm": synth.with_norm(synth.get_config(0)),
    "single_launch_4tok_norm": synth.with_norm(small_cfg(1, tokens=4, hidden=1024, n_experts=64, n_groups=8,
                                                         topk_groups=3, topk=6, inter=512, shared_inter=1024)),
    "b128_quant_3tok_norm": synth.with_norm(small_cfg(2, tokens=3, hidden=384, n_experts=16, n_groups=4,
                                                      topk_groups=2, topk=3, inter=256, shared_inter=256)),
    "b128_12exp_97tok_norm": synth.with_norm(small_cfg(2, tokens=97, hidden=512, n_experts=12, n_groups=3,
                                                       topk_groups=2, topk=3, inter=384, shared_inter=256)),
    "mx_4exp_160tok_norm": synth.with_norm(small_cfg(3, tokens=160, hidden=512, n_experts=4, inter=256,
                                                     shared_inter=256)),
    "b128_bf16x_6tok_norm": synth.with_norm(small_cfg(1, tokens=6, hidden=640, n_experts=24, n_groups=4,
                                                      topk_groups=2, topk=5, inter=384, shared_inter=512)),
}


# the format pairs the GEMM path has kernels for
GEMM_PAIRS = {("bf16", "none"), ("fp8_b128", "fp8_1x128"), ("mxfp8", "mxfp8_1x32")}


def served(cfg, path):
    """Whether the library has the forced path for cfg: no GEMM kernel for
    some format pairs, and the staged small-T path serves T <= 8."""
    if path == "gemm":
        return (cfg.routed_wfmt, cfg.routed_afmt) in GEMM_PAIRS and (cfg.shared_wfmt, cfg.shared_afmt) in GEMM_PAIRS
    return path != "staged" or cfg.tokens <= 8


@pytest.mark.parametrize("name,path", [(n, p) for n in NORM_LAYERS for p in ["auto", "staged", "gemv", "gemm"]
                                       if served(NORM_LAYERS[n], p)])
def test_forward_norm_small(name, path, monkeypatch):
    cfg = NORM_LAYERS[name]
    if path != "auto":
        monkeypatch.setenv("MOE_FORCE_PATH", path)
    say(f"[forward_norm] {name} {path}")
    inp = ensure_margin(synth.make_inputs(cfg, DEV))
    _check_layer(cfg, inp)


@pytest.mark.parametrize("base", ["dsv2_b1", "h7168_2048tok_mx", "dsv2_256tok"])
def test_forward_norm_full_size(base):
    """The DeepSeek-V2 B=1 layer (single launch: stage M staged in LDS by every
    workgroup) and the 256- and 2,048-token layers (norm inside the fused
    router launch) at full size: every row against the oracle."""
    cfg = synth.with_norm(synth.get_config(base))
    say(f"[forward_norm full] {cfg.name}")
    inp = ensure_margin(synth.make_inputs(cfg, DEV))
    _check_layer(cfg, inp)


def _check_layer(cfg, inp):
    T, H = cfg.tokens, cfg.hidden
    layer = moe.Layer(cfg, inp)
    xo = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    out = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    ids = torch.empty(T, cfg.topk, dtype=torch.int32, device=DEV)
    w = torch.empty(T, cfg.topk, dtype=torch.float32, device=DEV)
    outs = []
    for _ in range(2):
        moe.forward_norm(layer.cfg, inp.x, moe.make_norm(inp.gamma, cfg.norm_eps), inp.w_router, inp.bias,
                         layer.routed, layer.shared, out, ids, w, xo, layer.ws)
        torch.cuda.synchronize()
        outs.append(out.view(torch.int16).clone())
    moe.workspace_check(layer.ws)
    assert torch.equal(outs[0], outs[1])
    x, _ = oracle.rmsnorm(inp.x, inp.gamma, cfg.norm_eps)
    assert np.array_equal(xo.view(torch.int16).cpu().numpy().view(np.uint16), x)
    r = oracle.forward(cfg, inp.x, inp.w_router, inp.bias, inp.routed, inp.shared, norm=norm_of(inp))
    assert np.array_equal(ids.cpu().numpy(), r.ids)
    assert np.max(np.abs(w.cpu().numpy() - r.w) / r.w) <= WTOL
    assert rel_err(oracle.bf16_to_f64(out), r.out) <= TOL
