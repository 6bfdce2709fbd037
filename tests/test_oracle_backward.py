"""Pins of the backward oracle (Mixture-of-Kittens, Table 1: the MoE layer's
backward pass), against what does not depend on its hand-derived formulas:
central finite differences of the forward oracle, and torch autograd of an
independently written dense forward."""
import numpy as np
import pytest
import torch

import oracle


class _Cfg:
    def __init__(self, **kw):
        self.__dict__.update(kw)


class F64Experts:
    """Float64 expert weights in the oracle's weight-set interface."""
    fmt = "f64"

    def __init__(self, g, u, d):
        self.g, self.u, self.d = g, u, d

    def expert(self, e):
        return self.g[e], self.u[e], self.d[e], None, None, None


def tiny(seed=0, T=3, H=24, E=6, G=3, TG=2, K=3, I=16, Is=8, scale=2.5, bias=True):
    rng = np.random.default_rng(seed)
    cfg = _Cfg(n_experts=E, n_groups=G, topk_groups=TG, topk=K, route_scale=scale, hidden=H, inter=I,
               shared_inter=Is, routed_afmt="none", shared_afmt="none")
    x = rng.standard_normal((T, H))
    wr = rng.standard_normal((E, H)) * 0.5
    b = rng.standard_normal(E) * 0.3 if bias else None
    rw = [rng.standard_normal((E, I, H)) * 0.3, rng.standard_normal((E, I, H)) * 0.3,
          rng.standard_normal((E, H, I)) * 0.3]
    sw = [rng.standard_normal((1, Is, H)) * 0.3, rng.standard_normal((1, Is, H)) * 0.3,
          rng.standard_normal((1, H, Is)) * 0.3] if Is else None
    dy = rng.standard_normal((T, H))
    return cfg, x, wr, b, rw, sw, dy


def loss(cfg, x, wr, b, rw, sw, dy):
    r = oracle.forward(cfg, x, wr, b, F64Experts(*rw), None if sw is None else F64Experts(*sw))
    return float((dy * r.out).sum()), r.ids


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_central_finite_differences(seed):
    cfg, x, wr, b, rw, sw, dy = tiny(seed)
    g = oracle.backward(cfg, x, wr, b, F64Experts(*rw), F64Experts(*sw), dy)
    _, ids0 = loss(cfg, x, wr, b, rw, sw, dy)
    rng = np.random.default_rng(100 + seed)
    eps = 1e-6

    def fd(arr, idx, rebuild):
        a0 = arr[idx]
        arr[idx] = a0 + eps
        lp, ids = loss(*rebuild())
        arr[idx] = a0 - eps
        lm, ids2 = loss(*rebuild())
        arr[idx] = a0
        assert np.array_equal(ids, ids0) and np.array_equal(ids2, ids0)   # the selection did not move
        return (lp - lm) / (2 * eps)

    rebuild = lambda: (cfg, x, wr, b, rw, sw, dy)
    checks = []
    for _ in range(6):
        i = tuple(rng.integers(0, s) for s in x.shape)
        checks.append((fd(x, i, rebuild), g.dx[i]))
        i = tuple(rng.integers(0, s) for s in wr.shape)
        checks.append((fd(wr, i, rebuild), g.d_router[i]))
        i = (rng.integers(0, b.size),)
        checks.append((fd(b, i, rebuild), g.d_bias[i]))
    # expert weights: pick entries of experts that some token selected
    used = sorted(set(g.ids.ravel().tolist()))
    for _ in range(6):
        e = used[rng.integers(0, len(used))]
        for k, d in enumerate((g.d_gate, g.d_up, g.d_down)):
            i = (e,) + tuple(rng.integers(0, s) for s in rw[k].shape[1:])
            checks.append((fd(rw[k], i, rebuild), d[i]))
        for k in range(3):
            i = (0,) + tuple(rng.integers(0, s) for s in sw[k].shape[1:])
            checks.append((fd(sw[k], i, rebuild), g.d_shared[k][i[1:]]))
    num = np.array([c[0] for c in checks])
    ana = np.array([c[1] for c in checks])
    assert np.max(np.abs(num - ana)) <= 1e-6 * max(1.0, np.abs(ana).max())


def test_unused_experts_get_zero_gradients():
    cfg, x, wr, b, rw, sw, dy = tiny(3, T=2, E=6, K=2)
    g = oracle.backward(cfg, x, wr, b, F64Experts(*rw), F64Experts(*sw), dy)
    unused = sorted(set(range(6)) - set(g.ids.ravel().tolist()))
    assert unused
    for e in unused:
        assert not g.d_gate[e].any() and not g.d_up[e].any() and not g.d_down[e].any()


@pytest.mark.parametrize("seed", [4, 5])
def test_matches_torch_autograd_of_a_dense_forward(seed):
    """Every token through its selected experts written densely in torch
    (float64), differentiated by autograd; the ids are held fixed."""
    cfg, x, wr, b, rw, sw, dy = tiny(seed, T=5, H=32, E=8, G=4, TG=2, K=3, I=24, Is=16)
    g = oracle.backward(cfg, x, wr, b, F64Experts(*rw), F64Experts(*sw), dy)
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    X, WR, B = t(x), t(wr), t(b)
    RW = [t(a) for a in rw]
    SW = [t(a) for a in sw]
    ids = torch.tensor(g.ids, dtype=torch.long)

    def ffn(xr, wg, wu, wd):
        return (torch.nn.functional.silu(xr @ wg.T) * (xr @ wu.T)) @ wd.T

    s = torch.softmax(X @ WR.T + B, dim=1)
    out = ffn(X, SW[0][0], SW[1][0], SW[2][0])
    rows = []
    for tt in range(x.shape[0]):
        acc = torch.zeros(x.shape[1], dtype=torch.float64)
        for j in range(cfg.topk):
            e = int(ids[tt, j])
            acc = acc + cfg.route_scale * s[tt, e] * ffn(X[tt:tt + 1], RW[0][e], RW[1][e], RW[2][e])[0]
        rows.append(acc)
    out = out + torch.stack(rows)
    (out * torch.tensor(dy)).sum().backward()
    close = lambda a, ref: np.max(np.abs(a - ref.detach().numpy())) <= 1e-10 * max(1.0, np.abs(a).max())
    assert close(g.dx, X.grad)
    assert close(g.d_router, WR.grad) and close(g.d_bias, B.grad)
    for k, d in enumerate((g.d_gate, g.d_up, g.d_down)):
        assert close(d, RW[k].grad)
        assert close(g.d_shared[k], SW[k].grad[0])
