"""Pins of the oracle's stage M RMSNorm (DSV2-236B-MegaKernel README,
flowchart stage M: the post-attention RMSNorm before the router GEMV)."""
import numpy as np
import pytest
import torch

import oracle


def bf16_bits(t):
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(100000) * s for s in (1e-3, 1.0, 1e3)]).astype(np.float32)
    # exact midpoints between neighbouring bf16 values (ties to even)
    mids = (v.view(np.uint32) & 0xFFFF0000) | 0x8000
    v = np.concatenate([v, mids.astype(np.uint32).view(np.float32)])
    assert np.array_equal(oracle.f32_to_bf16_bits(v), bf16_bits(torch.from_numpy(v)))


@pytest.mark.parametrize("eps", [0.0, 1e-6])
def test_matches_library_rms_norm(eps):
    """Against torch.nn.functional.rms_norm in float64: the oracle's bf16 x is
    the library's value up to the float32 / bf16 roundings (2 bf16 ulps)."""
    g = torch.Generator().manual_seed(1)
    h = (torch.randn(32, 640, generator=g) * 3.0).to(torch.bfloat16)
    gamma = (1.0 + 0.2 * torch.randn(640, generator=g)).to(torch.bfloat16)
    x, r = oracle.rmsnorm(bf16_bits(h), bf16_bits(gamma), eps)
    ref = torch.nn.functional.rms_norm(h.double(), (640,), gamma.double(), eps=eps).numpy()
    got = oracle.bf16_to_f64(x)
    assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-30)
    ms = (h.double() ** 2).mean(dim=1).numpy()
    assert np.allclose(r, 1.0 / np.sqrt(ms + eps), rtol=2.0 ** -23)


def test_constant_row_normalises_to_unit():
    for c in (0.375, -3.0, 1024.0, 2.0 ** -10):
        h = torch.full((1, 256), c).to(torch.bfloat16)
        x, _ = oracle.rmsnorm(bf16_bits(h), bf16_bits(torch.ones(256)), 0.0)
        assert np.all(oracle.bf16_to_f64(x) == np.sign(c))


def test_power_of_two_scale_invariance():
    """eps = 0: scaling h by 2^k changes nothing (every step commutes with 2^k)."""
    g = torch.Generator().manual_seed(2)
    h = torch.randn(8, 384, generator=g).to(torch.bfloat16)
    gamma = (1.0 + 0.1 * torch.randn(384, generator=g)).to(torch.bfloat16)
    x0, _ = oracle.rmsnorm(bf16_bits(h), bf16_bits(gamma), 0.0)
    for k in (-6, 3, 9):
        xk, _ = oracle.rmsnorm(bf16_bits(h * 2.0 ** k), bf16_bits(gamma), 0.0)
        assert np.array_equal(xk, x0)


def test_unit_gamma_gives_unit_mean_square():
    g = torch.Generator().manual_seed(3)
    h = (torch.randn(16, 512, generator=g) * 7.0).to(torch.bfloat16)
    x, _ = oracle.rmsnorm(bf16_bits(h), bf16_bits(torch.ones(512)), 0.0)
    ms = (oracle.bf16_to_f64(x) ** 2).mean(axis=1)
    assert np.all(np.abs(ms - 1.0) < 2.0 ** -7)
