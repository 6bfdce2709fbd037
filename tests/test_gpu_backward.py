"""The layer's backward pass on MI355X (moe_backward, through the C ABI)
against the float64 backward oracle: every gradient tensor within
max|err| / max|ref| <= 2e-2 (bf16 inputs, intermediates and outputs; fp32
accumulation), repeated calls bitwise identical, and unsupported formats
refused before any launch."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_router_amd as moe
import oracle
import synth
from helpers import ensure_margin, rel_err, small_cfg

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 2e-2

CASES = {
    "tiny_8tok": small_cfg(0),
    "ragged_97tok": small_cfg(0, tokens=97, hidden=384, n_experts=12, n_groups=3, topk_groups=2, topk=3, inter=256,
                              shared_inter=128),
    "zipf_200tok": small_cfg(4, tokens=200, hidden=256, n_experts=16, n_groups=4, topk_groups=2, topk=4, inter=128,
                             shared_inter=128, routed_wfmt="bf16", shared_wfmt="bf16", routed_afmt="none",
                             shared_afmt="none"),
    "no_shared_k1_64tok": small_cfg(0, tokens=64, n_experts=8, n_groups=1, topk_groups=1, topk=1, shared_inter=0),
    "flat_32exp_300tok": small_cfg(3, tokens=300, hidden=512, n_experts=32, inter=256, shared_inter=256,
                                   routed_wfmt="bf16", shared_wfmt="bf16", routed_afmt="none", shared_afmt="none"),
    "single_token": small_cfg(0, tokens=1, hidden=384, n_experts=16, topk=4, inter=256, shared_inter=128),
    # several 64-row tiles per expert with ragged tails, 128-row forward tiles,
    # grouped routing with a Zipf bias (a reduced DeepSeek-V2 layer)
    "mid_640tok_zipf": small_cfg(4, tokens=640, hidden=1024, n_experts=32, n_groups=8, topk_groups=3, topk=6,
                                 inter=512, shared_inter=1024, routed_wfmt="bf16", shared_wfmt="bf16",
                                 routed_afmt="none", shared_afmt="none"),
}


def _grads_like(cfg):
    E, H, I, Is = cfg.n_experts, cfg.hidden, cfg.inter, cfg.shared_inter
    z = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device=DEV)
    rg = (z(E, I, H), z(E, I, H), z(E, H, I))
    sg = (z(1, Is, H), z(1, Is, H), z(1, H, Is)) if Is else None
    return rg, sg


def _run(cfg, inp, dy):
    T, H, E = cfg.tokens, cfg.hidden, cfg.n_experts
    c = moe.make_config(cfg)
    ws = torch.zeros(moe.backward_workspace_size(c, T), dtype=torch.uint8, device=DEV)
    dx = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    dr = torch.empty(E, H, dtype=torch.bfloat16, device=DEV)
    db = torch.empty(E, dtype=torch.float32, device=DEV) if inp.bias is not None else None
    rg, sg = _grads_like(cfg)
    moe.backward(c, inp.x, inp.w_router, inp.bias, moe.weights_of(inp.routed), moe.weights_of(inp.shared), dy, dx, dr,
                 db, moe.make_grads(*rg), None if sg is None else moe.make_grads(*sg), ws)
    torch.cuda.synchronize()
    return dx, dr, db, rg, sg


@pytest.mark.parametrize("name", list(CASES))
def test_backward_matches_oracle(name):
    cfg = CASES[name]
    print(f"[backward] {name}", flush=True)
    inp = ensure_margin(synth.make_inputs(cfg, DEV))
    g = torch.Generator(device=DEV)
    g.manual_seed(synth.generate.seed_of(cfg.index, 0, 11, cfg.tokens))
    dy = torch.randn(cfg.tokens, cfg.hidden, generator=g, device=DEV).to(torch.bfloat16)
    dx, dr, db, rg, sg = _run(cfg, inp, dy)
    ref = oracle.backward(cfg, inp.x, inp.w_router, inp.bias, inp.routed, inp.shared, dy)
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    errs = {"dx": rel_err(f(dx), ref.dx), "d_router": rel_err(f(dr), ref.d_router)}
    if db is not None:
        errs["d_bias"] = rel_err(f(db), ref.d_bias)
    for k, got, want in zip(("d_gate", "d_up", "d_down"), rg, (ref.d_gate, ref.d_up, ref.d_down)):
        errs[k] = rel_err(f(got), want)
    if sg is not None:
        for k, got, want in zip(("ds_gate", "ds_up", "ds_down"), sg, ref.d_shared):
            errs[k] = rel_err(f(got)[0], want)
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert max(errs.values()) <= TOL, errs
    used = np.zeros(cfg.n_experts, bool)
    used[ref.ids.ravel()] = True
    for t in rg:   # experts no token chose get exact zeros
        assert not t[torch.from_numpy(~used).to(DEV)].float().abs().sum().item()
    # a second call gives the same bits
    dx2, dr2, _, rg2, _ = _run(cfg, inp, dy)
    assert torch.equal(dx.view(torch.int16), dx2.view(torch.int16))
    assert torch.equal(dr.view(torch.int16), dr2.view(torch.int16))
    for a, b in zip(rg, rg2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_backward_refuses_quantised_formats():
    c = moe.make_config(synth.get_config("dsv2_256tok"))
    with pytest.raises(moe.MoEError) as e:
        moe.backward_workspace_size(c, 256)
    assert e.value.status == 2
