"""moe_forward_noalloc (no workspace argument: the library's own per-GPU
device array) against moe_forward on the same inputs, through the C ABI.
Two calls in a row on each case, the second with fewer tokens; ids and
weights equal, outputs bitwise equal (the same kernels run) and within the
oracle's bar.  Calls needing more than the array's 32 MiB are refused."""
import sys

import numpy as np
import pytest
import torch

import mixture_experts_layer_router_amd as moe
import oracle
import synth
from helpers import ensure_margin, rel_err, small_cfg

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = {
    # single launch (T <= 4, bf16 x)
    "single_launch_64exp": (small_cfg(1, tokens=4, hidden=1024, n_experts=64, n_groups=8, topk_groups=3, topk=6,
                                      inter=512, shared_inter=1024), (4, 2)),
    "dsv2_b1_dims": (synth.get_config(1).derive(tokens=4), (4, 1)),
    # staged small-T launches with quantised activations
    "b128_quant_3tok": (small_cfg(2, tokens=3, hidden=384, n_experts=16, n_groups=4, topk_groups=2, topk=3,
                                  inter=256, shared_inter=256), (3, 2)),
    # batched: dispatch + grouped GEMMs; moe_forward puts this shared expert on its side stream
    "batched_b128": (small_cfg(2, tokens=97, hidden=512, n_experts=12, n_groups=3, topk_groups=2, topk=3, inter=384,
                               shared_inter=256), (97, 40)),
    "batched_mx": (small_cfg(3, tokens=160, hidden=512, n_experts=4, inter=256, shared_inter=256), (160, 33)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_matches_forward(name):
    cfg, sizes = CASES[name]
    print(f"[noalloc] {name} T={sizes}", flush=True)
    inp = ensure_margin(synth.make_inputs(cfg, DEV))
    layer = moe.Layer(cfg, inp)
    r = oracle.forward(cfg, inp.x, inp.w_router, inp.bias, inp.routed, inp.shared)
    for T in sizes:
        x = inp.x[:T].contiguous()
        out_ref, ids_ref, w_ref = layer.forward(x)
        out = torch.full_like(out_ref, float("nan"))
        ids = torch.full_like(ids_ref, -1)
        w = torch.full_like(w_ref, float("nan"))
        moe.forward_noalloc(layer.cfg, x, inp.w_router, inp.bias, layer.routed, layer.shared, out, ids, w)
        torch.cuda.synchronize()
        assert torch.equal(ids, ids_ref)
        assert np.array_equal(ids.cpu().numpy(), r.ids[:T])
        assert torch.equal(w, w_ref)
        assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16))
        assert rel_err(oracle.bf16_to_f64(out), r.out[:T]) <= 2e-2


def test_noalloc_refuses_calls_beyond_its_array():
    cfg = synth.get_config("dsv2_256tok")          # 256 tokens need about 70 MiB of workspace
    c = moe.make_config(cfg)
    assert moe.workspace_size(c, cfg.tokens) > (32 << 20)
    inp = synth.make_inputs(cfg, DEV, with_experts=False)
    dummy = torch.zeros(16, dtype=torch.uint8, device=DEV)
    w = moe.make_weights(dummy, dummy, dummy, dummy, dummy, dummy)
    out = torch.zeros(cfg.tokens, cfg.hidden, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moe.MoEError) as e:
        moe.forward_noalloc(c, inp.x, inp.w_router, None, w, w, out, None, None)
    assert e.value.status == 4                      # MOE_EWORKSPACE, before any launch
    torch.cuda.synchronize()
    assert not out.any()
