"""Pins of the oracle's FP8 codecs against torch's float8_e4m3fn and the OCP definitions."""
import json
import os

import numpy as np
import torch

from oracle import e4m3_decode, e4m3_encode, e8m0_decode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_encode_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(e4m3_encode(e4m3_decode(codes)), codes)


def test_encode_midpoints_round_to_even():
    pos = np.arange(0, 0x7E, dtype=np.uint8)
    lo, hi = e4m3_decode(pos), e4m3_decode(pos + 1)
    mid = (lo + hi) / 2
    got = e4m3_encode(mid)
    want = np.where(pos % 2 == 0, pos, pos + 1).astype(np.uint8)
    assert np.array_equal(got, want)
    ref = torch.from_numpy(mid).to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)
    assert np.array_equal(e4m3_encode(-mid), want | 0x80)


def test_encode_random_fp32_matches_torch_with_clamp():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1, 30, 300)]).astype(np.float32)
    ref = torch.from_numpy(v).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(v.astype(np.float64)), ref)


def test_saturation_and_zero():
    got = e4m3_encode(np.array([448.0, 449.0, 463.9, 500.0, 1e30, -1e30, 0.0, 2.0 ** -11]))
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x00, 0x00]


def test_golden_codes_from_ocp_definition():
    with open(os.path.join(GOLDEN, "e4m3_e8m0_values.json")) as f:
        g = json.load(f)
    for code, val in g["e4m3"]:
        assert e4m3_decode(np.uint8(code)) == val, code
    for code, val in g["e8m0"]:
        assert e8m0_decode(np.uint8(code)) == val, code
