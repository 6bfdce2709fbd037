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


def test_neg_inf_logits_tie_below_finite_ones():
    """-inf logits (a masking bias) are candidates that tie with each other
    below every finite logit; they get weight 0.  Hand-worked: groups of 4,
    keep 1 group, top 3.  g0 holds one finite logit (1.0 at e2), g1 one (2.0
    at e5), so g1 is kept; e5 first, then the -inf members e4, e6 by id."""
    b = np.array([-np.inf, -np.inf, 1.0, -np.inf, -np.inf, 2.0, -np.inf, -np.inf])
    r = oracle.route(np.zeros((1, 8)), np.eye(8), b, _Cfg(8, 2, 1, 3, 2.0))   # logits = bias
    assert list(r["ids"][0]) == [5, 4, 6]
    assert abs(r["w"][0, 0] - 2.0 * math.exp(2.0) / (math.exp(1.0) + math.exp(2.0))) < 1e-15
    assert r["w"][0, 1] == 0.0 and r["w"][0, 2] == 0.0


@pytest.mark.parametrize("bad", [np.nan, np.inf])
def test_undefined_softmax_routes_to_lowest_ids(bad):
    """A NaN or +inf logit leaves the softmax undefined: every candidate ties,
    so the token takes the lowest ids of the lowest kept groups (g0, g1 of 4
    groups of 2 with 2 kept; 3 slots: e0, e1, e2) and NaN weights."""
    l = np.array([0.1, 2.0, 1.5, -1.0, 0.3, 1.9, 3.0, -2.0])
    r = oracle.route(np.eye(8)[[5]] * 0, np.eye(8), l + np.where(np.arange(8) == 5, bad, 0.0), _Cfg(8, 4, 2, 3, 2.0))
    assert list(r["ids"][0]) == [0, 1, 2]
    assert np.isnan(r["w"][0]).all()
    r = oracle.route(np.zeros((1, 8)), np.eye(8), l, _Cfg(8, 4, 2, 3, 2.0))
    assert list(r["ids"][0]) == [6, 1, 0]   # without the bad logit: the hand example


def test_all_neg_inf_token():
    r = oracle.route(np.zeros((1, 8)), np.eye(8), np.full(8, -np.inf), _Cfg(8, 4, 2, 3))
    assert list(r["ids"][0]) == [0, 1, 2]
    assert np.isnan(r["w"][0]).all()


def test_zipf_workload_skew_in_band():
    """The skewed 4,096-token workload: a router bias b[e] = -1.2 ln(rank_e)
    stands in for trained-router popularity (Zipf, s = 1.2).  Its realised
    load, routed by the oracle, has max/mean in [15, 160/6]: the hottest
    expert near 20x the mean, capped by each token taking 6 distinct experts."""
    cfg = synth.get_config("dsv2_4096tok_zipf")
    inp = ensure_margin(synth.make_inputs(cfg, with_experts=False))
    r = oracle.route(oracle.bf16_to_f64(inp.x), oracle.bf16_to_f64(inp.w_router),
                     inp.bias.double().numpy(), cfg)
    cnt = np.bincount(r["ids"].ravel(), minlength=cfg.n_experts)
    ratio = cnt.max() / cnt.mean()
    assert 15.0 <= ratio <= 160 / 6, ratio
    # groups still bind: every token's experts come from at most 3 groups
    assert max(len(set(int(e) // 20 for e in row)) for row in r["ids"]) <= 3
