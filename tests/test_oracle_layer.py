"""Pins of the oracle's quantisers, dispatch, FFN and whole-layer forward."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import ensure_margin, small_cfg
from oracle import e4m3_decode


# ------------------------------------------------------------ quantisers

def _grid_rows(rng, rows, K, blk, exp_fn):
    codes = rng.integers(0, 0x7E, size=(rows, K), dtype=np.uint8)
    codes |= rng.integers(0, 2, size=(rows, K), dtype=np.uint8) << 7
    scale = exp_fn(rng, rows, K // blk)
    v = e4m3_decode(codes).reshape(rows, K // blk, blk) * scale[:, :, None]
    return codes, v, scale


def test_quant_1x128_identity_on_grid():
    rng = np.random.default_rng(3)
    codes, v, s = _grid_rows(rng, 8, 512, 128, lambda r, a, b: np.ldexp(1.0, r.integers(-12, 4, size=(a, b))))
    v[:, :, 0] = 448.0 * s                  # amax exactly 448 * s -> recovered scale s
    codes = codes.reshape(8, 4, 128)
    codes[:, :, 0] = 0x7E
    out, q, sc = oracle.quant_act(v.reshape(8, 512), "fp8_1x128", return_codes=True)
    assert np.array_equal(out, v.reshape(8, 512))
    assert np.array_equal(sc, s.astype(np.float32))
    assert np.array_equal(e4m3_decode(q), e4m3_decode(codes.reshape(8, 512)))


def test_quant_mx_identity_on_grid():
    rng = np.random.default_rng(4)
    codes, v, X = _grid_rows(rng, 8, 256, 32, lambda r, a, b: np.ldexp(1.0, r.integers(-20, 10, size=(a, b))))
    v[:, :, 0] = 256.0 * X                  # floor(log2 amax) - 8 = log2 X
    out, q, e8 = oracle.quant_act(v.reshape(8, 256), "mxfp8_1x32", return_codes=True)
    assert np.array_equal(out, v.reshape(8, 256))
    assert np.array_equal(oracle.e8m0_decode(e8), X)


@pytest.mark.parametrize("afmt,blk", [("fp8_1x128", 128), ("mxfp8_1x32", 32)])
def test_quant_error_bound_and_zero_block(afmt, blk):
    rng = np.random.default_rng(5)
    v = rng.standard_normal((16, 512)).astype(np.float32).astype(np.float64) * 3.0
    v[0, :blk] = 0.0
    out = oracle.quant_act(v, afmt)
    assert np.all(out[0, :blk] == 0.0)
    # 3 mantissa bits: relative error <= 2^-4 for normals, plus the subnormal step
    amax = np.abs(v.reshape(16, -1, blk)).max(axis=2, keepdims=True)
    step = np.repeat(amax * 2.0 ** -9 / 448.0 * (1 if blk == 128 else 2), blk, axis=2).reshape(16, 512)
    sat = 0.0
    if blk == 32:   # X = 2^(floor(log2 amax) - 8) puts amax/X in [256, 512): the top saturates at 448
        X = np.ldexp(1.0, np.frexp(amax)[1] - 1 - 8)
        sat = np.maximum(np.abs(v) - 448.0 * np.repeat(X, blk, axis=2).reshape(16, 512), 0.0)
    assert np.all(np.abs(out - v) <= np.abs(v) * 2.0 ** -4 + step + sat + 1e-300)


def test_quant_codes_match_torch_cast():
    """The 1x128 codes equal torch's e4m3fn cast of the fp32 quotient."""
    rng = np.random.default_rng(6)
    x = torch.from_numpy(rng.standard_normal((4, 256)).astype(np.float32)).to(torch.bfloat16)
    xf = oracle.bf16_to_f64(x)
    _, q, s = oracle.quant_act(xf, "fp8_1x128", return_codes=True)
    x32 = x.float().view(4, 2, 128)
    amax = x32.abs().amax(dim=2)
    ts = amax / 448.0
    assert np.array_equal(ts.numpy(), s)
    ref = (x32 / ts[:, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).reshape(4, 256)
    assert np.array_equal(ref.numpy(), q)


def test_dequant_b128_and_mx_exact_products():
    q = np.array([[0x38, 0x7E], [0x01, 0xB8]], dtype=np.uint8).repeat(64, 0).repeat(64, 1)  # [128][128]
    s = np.array([[0.5]], dtype=np.float32)
    w = oracle.dequant_weight(q, s, "fp8_b128")
    assert w[0, 0] == 0.5 and w[0, 127] == 224.0 and w[127, 0] == 2.0 ** -10 and w[127, 127] == -0.5
    e8 = np.full((128, 4), 130, dtype=np.uint8)
    w2 = oracle.dequant_weight(q, e8, "mxfp8")
    assert w2[0, 0] == 8.0 and w2[0, 127] == 448.0 * 8


# --------------------------------------------------------------- dispatch

def test_permute_matches_library_and_is_a_bijection():
    rng = np.random.default_rng(7)
    ids = np.stack([rng.choice(40, size=6, replace=False) for _ in range(300)]).astype(np.int32)
    off, perm, inv = oracle.permute(ids, 40)
    flat = ids.ravel()
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=40))]))
    assert np.array_equal(np.sort(perm), np.arange(flat.size))
    assert np.array_equal(perm[inv], np.arange(flat.size))
    assert np.array_equal(inv[perm], np.arange(flat.size))
    for e in range(40):
        seg = perm[off[e]:off[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)   # stable
    # unpermute(permute(v)) = v
    v = rng.standard_normal(flat.size)
    assert np.array_equal(v[perm][inv], v)


def test_permute_empty_experts():
    ids = np.array([[3, 1], [3, 0]], dtype=np.int32)
    off, perm, inv = oracle.permute(ids, 6)
    assert list(off) == [0, 1, 2, 2, 4, 4, 4]
    assert list(perm) == [3, 1, 0, 2]


# ---------------------------------------------------------------------- FFN

def test_ffn_is_textbook_swiglu():
    rng = np.random.default_rng(8)
    H, I = 6, 4
    X = rng.standard_normal((3, H))
    wg, wu, wd = rng.standard_normal((I, H)), rng.standard_normal((I, H)), rng.standard_normal((H, I))
    y = oracle.expert_ffn(X, wg, wu, wd, "none")
    for r in range(3):
        for n in range(H):
            acc = 0.0
            for i in range(I):
                g = sum(X[r, k] * wg[i, k] for k in range(H))
                u = sum(X[r, k] * wu[i, k] for k in range(H))
                acc += wd[n, i] * (g / (1.0 + np.exp(-g))) * u
            assert abs(y[r, n] - acc) < 1e-12 * max(1.0, abs(acc))
    assert np.all(oracle.expert_ffn(X, np.zeros((I, H)), wu, wd, "none") == 0.0)   # SiLU(0) = 0


class _Split:
    """One half of a shared expert (rows/cols [a, b) of the intermediate)."""

    def __init__(self, w, a, b, fmt):
        self.w, self.a, self.b, self.fmt = w, a, b, fmt

    def expert(self, e):
        g, u, d, gs, us, ds = self.w.expert(0)
        a, b = self.a, self.b
        if self.fmt == "fp8_b128":
            return g[a:b], u[a:b], d[:, a:b], gs[a // 128:b // 128], us[a // 128:b // 128], ds[:, a // 128:b // 128]
        return g[a:b], u[a:b], d[:, a:b], None, None, None


@pytest.mark.parametrize("fmt,afmt", [("bf16", "none"), ("fp8_b128", "none"), ("fp8_b128", "fp8_1x128")])
def test_fused_shared_equals_sum_of_split_experts(fmt, afmt):
    cfg = small_cfg(2, tokens=5, hidden=256, n_experts=8, n_groups=4, topk_groups=2, topk=2,
                    inter=128, shared_inter=256, routed_wfmt=fmt, shared_wfmt=fmt,
                    routed_afmt=afmt, shared_afmt=afmt)
    inp = synth.make_inputs(cfg)
    x = oracle.bf16_to_f64(inp.x)
    full = oracle.expert_ffn(x, *oracle.moe._Dequant(inp.shared, fmt)(0), afmt)
    parts = sum(oracle.expert_ffn(x, *oracle.moe._Dequant(_Split(inp.shared, a, a + 128, fmt), fmt)(0), afmt)
                for a in (0, 128))
    assert np.allclose(full, parts, rtol=1e-12, atol=1e-14)


# -------------------------------------------------------------------- layer

LAYER_CASES = [
    ("tiny_8tok", dict()),
    ("dsv2_b1", dict(tokens=6, hidden=256, n_experts=16, n_groups=4, topk_groups=2, topk=3, inter=256, shared_inter=256)),
    ("dsv2_256tok", dict(tokens=9, hidden=384, n_experts=12, n_groups=3, topk_groups=2, topk=3, inter=128, shared_inter=256)),
    ("h7168_2048tok_mx", dict(tokens=7, hidden=256, n_experts=8, inter=128, shared_inter=128)),
    ("dsv2_4096tok_zipf", dict(tokens=10, hidden=256, n_experts=16, n_groups=4, topk_groups=2, topk=4, inter=128, shared_inter=128)),
]


@pytest.mark.parametrize("name,kw", LAYER_CASES)
def test_sparse_layer_equals_dense_masked(name, kw):
    cfg = small_cfg(name, **kw)
    inp = ensure_margin(synth.make_inputs(cfg))
    r = oracle.forward(cfg, inp.x, inp.w_router, inp.bias, inp.routed, inp.shared)
    dense = oracle.forward_dense_masked(cfg, inp.x, inp.w_router, inp.bias, inp.routed, inp.shared)
    assert np.allclose(r.out, dense, rtol=1e-12, atol=1e-13)
    ids, w, rows = oracle.forward_tokens(cfg, inp.x, inp.w_router, inp.bias, inp.routed, inp.shared, [0, cfg.tokens - 1])
    assert np.array_equal(ids, r.ids[[0, -1]])
    assert np.allclose(rows, r.out[[0, -1]], rtol=1e-12, atol=1e-13)


def test_single_expert_layer_is_a_dense_ffn():
    cfg = small_cfg(0, tokens=4, n_experts=1, n_groups=1, topk_groups=1, topk=1, shared_inter=0)
    inp = synth.make_inputs(cfg)
    r = oracle.forward(cfg, inp.x, inp.w_router, None, inp.routed, None)
    assert np.allclose(r.w, 1.0)
    x = oracle.bf16_to_f64(inp.x)
    wg, wu, wd = (oracle.bf16_to_f64(t[0]) for t in (inp.routed.gate, inp.routed.up, inp.routed.down))
    g, u = x @ wg.T, x @ wu.T
    assert np.allclose(r.out, (g * (1 / (1 + np.exp(-g))) * u) @ wd.T, rtol=1e-12, atol=1e-14)
