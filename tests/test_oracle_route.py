"""Pins of the oracle's router + group-limited top-k (DSV2-236B-MegaKernel README, stage O)."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from helpers import ensure_margin, small_cfg

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


class _Cfg:
    def __init__(self, E, G, TG, K, scale=1.0):
        self.n_experts, self.n_groups, self.topk_groups, self.topk, self.route_scale = E, G, TG, K, scale


def test_hand_example():
    with open(os.path.join(GOLDEN, "route_hand_example.json")) as f:
        g = json.load(f)
    l = np.array(g["logits"])
    cfg = _Cfg(8, g["n_groups"], g["topk_groups"], g["topk"], g["route_scale"])
    r = oracle.route(l[None, :], np.eye(8), None, cfg)
    assert list(r["ids"][0]) == g["ids"]
    flat = oracle.route(l[None, :], np.eye(8), None, _Cfg(8, 1, 1, 3, 2.0))
    assert list(flat["ids"][0]) == g["ids_without_group_limit"]
    tot = sum(math.exp(v) for v in g["logits"])
    for j, e in enumerate(g["ids"]):
        assert abs(r["w"][0, j] - 2.0 * math.exp(g["logits"][e]) / tot) < 1e-15


def test_softmax_normalised_and_shift_invariant():
    rng = np.random.default_rng(1)
    x, wr = rng.standard_normal((20, 64)), rng.standard_normal((16, 64)) * 0.1
    cfg = _Cfg(16, 4, 2, 4, 3.0)
    r0 = oracle.route(x, wr, None, cfg)
    assert np.allclose(r0["scores"].sum(axis=1), 1.0, atol=1e-14)
    r1 = oracle.route(x, wr, np.full(16, 7.5), cfg)
    assert np.array_equal(r0["ids"], r1["ids"])
    assert np.allclose(r0["w"], r1["w"], rtol=1e-12)


@pytest.mark.parametrize("E,G,TG,K", [(16, 1, 1, 4), (16, 4, 4, 3), (32, 8, 8, 6)])
def test_reduces_to_plain_topk(E, G, TG, K):
    rng = np.random.default_rng(E + K)
    x, wr = rng.standard_normal((50, 32)), rng.standard_normal((E, 32))
    r = oracle.route(x, wr, None, _Cfg(E, G, TG, K))
    ref = np.argsort(-r["logits"], axis=1, kind="stable")[:, :K]
    assert np.array_equal(r["ids"], ref)


@pytest.mark.parametrize("E,G,TG,K", [(16, 4, 2, 4), (12, 4, 3, 2), (20, 5, 2, 5), (16, 4, 1, 3)])
def test_matches_bruteforce_enumeration(E, G, TG, K):
    rng = np.random.default_rng(100 + E + G + TG + K)
    cfg = _Cfg(E, G, TG, K)
    x, wr = rng.standard_normal((60, 16)), rng.standard_normal((E, 16))
    r = oracle.route(x, wr, None, cfg)
    for t in range(x.shape[0]):
        assert np.array_equal(r["ids"][t], oracle.moe.route_bruteforce(r["scores"][t], cfg))


def test_weight_ratios_and_sum():
    rng = np.random.default_rng(2)
    cfg = _Cfg(160, 8, 3, 6, 16.0)
    x, wr = rng.standard_normal((10, 128)), rng.standard_normal((160, 128)) * 0.1
    r = oracle.route(x, wr, None, cfg)
    l = r["logits"]
    for t in range(10):
        ids, w = r["ids"][t], r["w"][t]
        assert np.all(np.diff(w) < 0)                        # descending score order
        assert w.sum() <= 16.0
        for j in range(1, 6):
            assert abs(w[0] / w[j] - math.exp(l[t, ids[0]] - l[t, ids[j]])) < 1e-9 * w[0] / w[j]
        assert len(set(ids)) == 6
        groups = set(int(e) // 20 for e in ids)
        assert len(groups) <= 3


def test_generator_margin_guarantee():
    cfg = small_cfg(0, tokens=64)
    inp = ensure_margin(synth.make_inputs(cfg, with_experts=False))
    l = oracle.bf16_to_f64(inp.x) @ oracle.bf16_to_f64(inp.w_router).T
    assert oracle.route_margins(l, cfg).min() >= 1e-3


def test_margin_detects_a_near_tie():
    cfg = _Cfg(8, 4, 2, 3)
    l = np.array([[0.1, 2.0, 1.5, -1.0, 0.3, 1.9, 3.0, 2.0005]])
    assert oracle.route_margins(l, cfg)[0] < 1e-3
    l2 = np.array([[0.1, 2.0, 1.5, -1.0, 0.3, 1.9, 3.0, -2.0]])
    assert abs(oracle.route_margins(l2, cfg)[0] - 0.1) < 1e-12   # group gap 2.0 vs 1.9
