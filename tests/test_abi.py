"""The C-ABI library loads, exports every entry point the header declares, and
its host-side validation rejects bad calls before any launch (no GPU needed)."""
import ctypes
import os
import re

import pytest

import mixture_experts_layer_router_amd as moe
import synth

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")
pytestmark = pytest.mark.skipif(not os.path.exists(moe.LIB_PATH), reason="libmoe.so not built")

OK, EINVAL, EUNSUP, EALIGN, EWS = 0, 1, 2, 3, 4


def declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:moe_status|const char\*|int32_t)\s+(moe_\w+)\s*\(", src, re.M)))


def test_exports_every_declared_symbol():
    names = declared()
    assert len(names) >= 9
    lib = ctypes.CDLL(moe.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(moe.EXPORTS)


def test_workspace_check_rejects_bad_arguments():
    lib = moe._lib()
    assert lib.moe_workspace_check(None, 1 << 20, 1, None) == EINVAL


def cfg(**kw):
    c = moe.make_config(synth.get_config(1))
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def ws_size(c, T=1):
    n = ctypes.c_size_t(0)
    st = moe._lib().moe_workspace_size(ctypes.byref(c), T, ctypes.byref(n))
    return st, n.value


def test_status_strings():
    lib = moe._lib()
    for s in range(7):
        assert lib.moe_status_string(s).decode().startswith("MOE_")
    assert b"unknown" in lib.moe_status_string(99)


@pytest.mark.parametrize("field,value,want", [
    ("n_groups", 7, EINVAL),            # 160 % 7 != 0
    ("topk_groups", 0, EINVAL),
    ("topk_groups", 9, EINVAL),
    ("topk", 61, EINVAL),               # more than 3 groups x 20 candidates
    ("topk", 17, EINVAL),
    ("topk", 0, EINVAL),
    ("hidden", 5000, EALIGN),
    ("inter", 1500, EALIGN),
    ("shared_inter", 100, EALIGN),
    ("routed_wfmt", 3, EINVAL),
    ("routed_afmt", -1, EINVAL),
    ("route_scale", float("inf"), EINVAL),
    ("route_scale", float("nan"), EINVAL),
])
def test_config_validation(field, value, want):
    assert ws_size(cfg(**{field: value}))[0] == want


def test_unsupported_pairs_and_sizes():
    assert ws_size(cfg(routed_wfmt=0, routed_afmt=1))[0] == EUNSUP     # bf16 weights, fp8 activations
    assert ws_size(cfg(n_experts=512, n_groups=8))[0] == EUNSUP
    assert ws_size(cfg())[0] == OK


def test_workspace_grows_with_tokens():
    c = cfg()
    a, b = ws_size(c, 1)[1], ws_size(c, 256)[1]
    assert 0 < a < b
    n = ctypes.c_size_t(0)
    assert moe._lib().moe_workspace_size(ctypes.byref(c), -1, ctypes.byref(n)) == EINVAL
    assert moe._lib().moe_workspace_size(ctypes.byref(c), 1, None) == EINVAL


FAKE = 0x10000  # an aligned address that is never dereferenced: validation fails first


def fwd(c, x=FAKE, T=1, wr=FAKE, routed=True, shared=True, out=FAKE, ws=FAKE, ws_bytes=1 << 40, wfake=FAKE):
    W = moe.FfnWeights(wfake, wfake, wfake, wfake, wfake, wfake)
    return moe._lib().moe_forward(ctypes.byref(c), x, T, wr, None, ctypes.byref(W) if routed else None,
                                  ctypes.byref(W) if shared else None, out, None, None, ws, ws_bytes, None)


def test_forward_error_paths():
    c = cfg()
    assert fwd(c, T=0) == OK                 # no-op
    assert fwd(c, T=-1) == EINVAL
    assert fwd(c, x=None) == EINVAL
    assert fwd(c, out=None) == EINVAL
    assert fwd(c, routed=False) == EINVAL
    assert fwd(c, shared=False) == EINVAL
    assert fwd(c, x=FAKE + 8) == EALIGN
    assert fwd(c, wfake=FAKE + 4) == EALIGN
    assert fwd(c, ws_bytes=16) == EWS
    bad = cfg(topk_groups=0)
    assert fwd(bad) == EINVAL


def test_other_entry_points_error_paths():
    lib = moe._lib()
    c = cfg()
    assert lib.moe_route(ctypes.byref(c), FAKE, 0, FAKE, None, FAKE, FAKE, FAKE, 1 << 40, None) == OK
    assert lib.moe_route(ctypes.byref(c), None, 1, FAKE, None, FAKE, FAKE, FAKE, 1 << 40, None) == EINVAL
    assert lib.moe_route(ctypes.byref(c), FAKE, 1, FAKE, None, FAKE, FAKE, FAKE, 8, None) == EWS
    assert lib.moe_permute(ctypes.byref(c), None, 4, None, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 40, None) == EINVAL
    assert lib.moe_permute(ctypes.byref(c), FAKE, 4, None, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None) == EINVAL
    W = moe.FfnWeights(FAKE, FAKE, FAKE, None, None, None)           # FP8 weights without scales
    assert lib.moe_expert_ffn(ctypes.byref(c), 0, FAKE, None, 4, FAKE, ctypes.byref(W), FAKE, FAKE, 1 << 40, None) == EINVAL
    W2 = moe.FfnWeights(*[FAKE] * 6)
    assert lib.moe_expert_ffn(ctypes.byref(c), 2, FAKE, None, 4, FAKE, ctypes.byref(W2), FAKE, FAKE, 1 << 40, None) == EINVAL
    assert lib.moe_expert_ffn(ctypes.byref(c), 0, FAKE, None, 4, None, ctypes.byref(W2), FAKE, FAKE, 1 << 40, None) == EINVAL
    assert lib.moe_expert_ffn(ctypes.byref(c), 0, FAKE, FAKE, 4, FAKE, ctypes.byref(W2), FAKE, FAKE, 1 << 40, None) == EINVAL  # scales with afmt none
    assert lib.moe_combine(ctypes.byref(c), FAKE, FAKE, FAKE, None, 0, FAKE, None) == OK
    assert lib.moe_combine(ctypes.byref(c), FAKE, None, FAKE, None, 3, FAKE, None) == EINVAL
    assert lib.moe_combine(ctypes.byref(c), FAKE + 4, FAKE, FAKE, None, 3, FAKE, None) == EALIGN
    assert lib.moe_debug_e4m3_decode(None, None, 0, None) == OK
    assert lib.moe_debug_e4m3_decode(None, FAKE, 5, None) == EINVAL
