"""The device-side dispatch check (moe_debug_validate_dispatch) passes on the
dispatch every batched forward leaves in its workspace, and reports each
planted inconsistency (planted from the host into a copy of the workspace
or the ids; the check only reads) with its own bit."""
import pytest
import torch

import mixture_experts_layer_router_amd as moe
import synth
from helpers import ensure_margin, small_cfg

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = {
    "b128_12exp_97tok": small_cfg(2, tokens=97, hidden=256, n_experts=12, n_groups=3, topk_groups=2, topk=3,
                                  inter=256, shared_inter=128),
    "zipf_16exp_200tok": small_cfg(4, tokens=200, hidden=256, n_experts=16, n_groups=4, topk_groups=2, topk=4,
                                   inter=128, shared_inter=128),
    "mx_mid_600tok": small_cfg(3, tokens=600, hidden=1024, n_experts=8, inter=512, shared_inter=512),
    "bf16_32exp_300tok": small_cfg(0, tokens=300, hidden=512, n_experts=32, n_groups=1, topk_groups=1, topk=4,
                                   inter=256, shared_inter=256),
}


def _run(cfg):
    inp = ensure_margin(synth.make_inputs(cfg, DEV))
    layer = moe.Layer(cfg, inp)
    _, ids, _ = layer.forward()
    torch.cuda.synchronize()
    return layer, ids


@pytest.mark.parametrize("name", list(CASES))
def test_dispatch_checks_hold(name):
    cfg = CASES[name]
    print(f"[validate] {name}", flush=True)
    layer, ids = _run(cfg)
    assert moe.validate_dispatch(layer.cfg, cfg.tokens, ids, layer.ws) == 0


def test_planted_inconsistencies_are_reported():
    cfg = CASES["zipf_16exp_200tok"]
    print("[validate] planted", flush=True)
    layer, ids = _run(cfg)
    c, T, E = layer.cfg, cfg.tokens, cfg.n_experts
    base = layer.ws.clone()

    def check(ws, ids_=ids):
        return moe.validate_dispatch(c, T, ids_, ws)

    ws = base.clone()
    moe.ws_region(c, T, ws, "offsets", E + 1)[E] += 1
    assert check(ws) & 2
    ws = base.clone()
    perm = moe.ws_region(c, T, ws, "perm_src", T * cfg.topk)
    a, b = perm[0].item(), perm[1].item()
    perm[0], perm[1] = b, a
    assert check(ws) & 8
    bad_ids = ids.clone()
    bad_ids.view(-1)[0] = E
    assert check(base.clone(), bad_ids) & 4
    ws = base.clone()
    moe.ws_region(c, T, ws, "tiles", 2)[1] += 1
    assert check(ws) & 32
    ws = base.clone()
    moe.ws_region(c, T, ws, "ntiles", 1)[0] = 1 << 30
    assert check(ws) & 32
    assert check(base.clone()) == 0
