"""Float64 CPU oracle of one MoE layer's backward pass (test infrastructure only).

Mixture-of-Kittens (Table 1) reports the MoE layer's backward beside its
forward; this is the single-GPU half of it: given the gradient dy of the
layer output out = sum_j w_j * Y_j + S (the forward of oracle.moe), the
gradients of the input x, the router weight and bias, and every expert's
gate, up and down weights.  Activations are unquantised (activation format
"none"); weights of any format are used dequantised, and their gradients
are dense float64.  The expert selection is piecewise constant, so no
gradient flows through the choice of ids, only through the routing weights
w = route_scale * softmax(logits)[id].

Derivation (chain rule, written out):
  combine    dY_slot[p] = w[t,j] dy[t],  dw[t,j] = <dy[t], Y_slot[p]>,  dS = dy
  SwiGLU     g = X Wg^T, u = X Wu^T, a = silu(g), h = a u, Y = h Wd^T:
             dh = dY Wd,  dWd = dY^T h,  du = dh a,  dg = dh u silu'(g),
             silu'(g) = sigma(g) (1 + g (1 - sigma(g))),
             dX = dg Wg + du Wu,  dWg = dg^T X,  dWu = du^T X
  routing    ds[t,e] = route_scale dw[t,j] for e = ids[t,j] (0 elsewhere),
             dl[t,e] = s[t,e] (ds[t,e] - sum_f s[t,f] ds[t,f])   (softmax),
             dWr = dl^T x,  dbias = sum_t dl[t],  dx += dl Wr
  dx[t] = sum_j dX_slot[t*K+j] + dX_shared[t] + (dl Wr)[t]

Parity status: pinned by central finite differences of the forward on tiny
layers and by torch autograd of an independently written dense forward.
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .moe import _Dequant, as_f64, expert_ffn, permute, route, _f64


def _sigmoid(g):
    return 1.0 / (1.0 + np.exp(-g))


def ffn_backward(X, wg, wu, wd, dY):
    """Backward of one SwiGLU FFN on rows X (float64, activation format
    none): returns (Y, dX, dWg, dWu, dWd)."""
    g = X @ wg.T
    u = X @ wu.T
    sg = _sigmoid(g)
    a = g * sg
    h = a * u
    Y = h @ wd.T
    dh = dY @ wd
    dWd = dY.T @ h
    du = dh * a
    dg = dh * u * (sg * (1.0 + g * (1.0 - sg)))
    dX = dg @ wg + du @ wu
    return Y, dX, dg.T @ X, du.T @ X, dWd


@dataclass
class BackwardResult:
    dx: np.ndarray                 # [T][H]
    d_router: np.ndarray           # [E][H]
    d_bias: Optional[np.ndarray]   # [E] (None without a bias)
    d_gate: np.ndarray             # [E][I][H]
    d_up: np.ndarray               # [E][I][H]
    d_down: np.ndarray             # [E][H][I]
    d_shared: Optional[tuple]      # (d_gate [Is][H], d_up [Is][H], d_down [H][Is]) or None
    dw: np.ndarray                 # [T][K] gradient of the routing weights
    ids: np.ndarray


def backward(cfg, x, w_router, bias, routed, shared, dy):
    """Gradients of <dy, out> for the layer forward(cfg, x, ...) of oracle.moe
    (activation formats "none").  dy: float64 or bf16 [T][H]."""
    assert cfg.routed_afmt == "none" and (shared is None or cfg.shared_afmt == "none")
    xf = as_f64(x)
    wr = as_f64(w_router)
    dyf = _f64(dy)
    b = None if bias is None else _f64(bias)
    r = route(xf, wr, b, cfg)
    T, K = r["ids"].shape
    E, H, I = cfg.n_experts, cfg.hidden, cfg.inter
    offsets, perm_src, inv_pos = permute(r["ids"], E)
    deq = _Dequant(routed, routed.fmt)
    wflat = r["w"].reshape(-1)
    dx = np.zeros((T, H))
    d_gate = np.zeros((E, I, H))
    d_up = np.zeros((E, I, H))
    d_down = np.zeros((E, H, I))
    dw_flat = np.zeros(T * K)
    for e in range(E):
        a, z = offsets[e], offsets[e + 1]
        if a == z:
            continue
        slots = perm_src[a:z]
        tok = slots // K
        wg, wu, wd = deq(e)
        X = xf[tok]
        # Y of each slot first (for dw), then the FFN backward with dY = w dy
        Y = expert_ffn(X, wg, wu, wd, "none")
        dw_flat[slots] = np.einsum("rh,rh->r", dyf[tok], Y)
        dY = wflat[slots][:, None] * dyf[tok]
        _, dX, dWg, dWu, dWd = ffn_backward(X, wg, wu, wd, dY)
        d_gate[e], d_up[e], d_down[e] = dWg, dWu, dWd
        np.add.at(dx, tok, dX)
    d_shared = None
    if shared is not None:
        wg, wu, wd = _Dequant(shared, shared.fmt)(0)
        _, dX, dWg, dWu, dWd = ffn_backward(xf, wg, wu, wd, dyf)
        dx += dX
        d_shared = (dWg, dWu, dWd)
    dw = dw_flat.reshape(T, K)
    s = r["scores"]
    ds = np.zeros((T, E))
    for t in range(T):
        ds[t, r["ids"][t]] = cfg.route_scale * dw[t]
    dl = s * (ds - (s * ds).sum(axis=1, keepdims=True))
    dx += dl @ wr
    return BackwardResult(dx, dl.T @ xf, None if b is None else dl.sum(axis=0), d_gate, d_up, d_down, d_shared, dw,
                          r["ids"])
