"""Float64 CPU oracle of one MoE layer forward (test infrastructure only).

Steps, in the order the DSV2-236B-MegaKernel README's flowchart runs the
MoE block ("What runs inside the single launch", stages N, O, P1/Q1, P2/Q2,
R), generalised from one token to T tokens with the dispatch/combine of
Mixture-of-Kittens (Abstract, Figure 1):

  N   logits = x . Wr^T (+ bias)
  O   scores = softmax(logits) over all experts; group score = max of its
      members' scores; keep the top-TG groups; take the top-K experts of the
      kept groups; w = route_scale * score
  --  dispatch: stable sort of the T*K (token, slot) pairs by expert
  P1  per expert: g = X.Wg^T, u = X.Wu^T, h = SiLU(g) * u
  P2  Y = h.Wd^T
  Q   shared expert: the same FFN on every token, unweighted
  R   out = sum_j w_j * Y_j + S   (no residual, no norm)

Readings of open points (each is listed in the design notes):
* softmax runs over all E logits before selection; weights are not
  renormalised over the selected experts (stage O: w = score x 16.0);
* groups are contiguous id ranges; a group's score is its max member score;
* the selected slots are ordered by descending score, ties to the lower id;
* quantised-activation modes quantise the FFN inputs (x rows and h) per row:
  1x128 blocks with an fp32 scale amax/448, or 1x32 blocks with an e8m0
  scale 2^(floor(log2 amax) - 8).  The code an element gets is decided in
  fp32 (scale = fl32(amax/448), code = RNE_e4m3(fl32(v/scale))), the same
  precision the HIP kernels use, so the codes of x match bit for bit;
* h is rounded to fp32 before it is quantised (the kernels hold h in fp32).

Parity status: every function below is pinned by CPU tests (brute-force
top-k, library argsort/bincount, SwiGLU closed form, dense-masked layer,
split-vs-fused shared expert, on-grid quantiser identity).
"""
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from itertools import combinations
from typing import Optional

import numpy as np

from .fp8 import e4m3_decode, e4m3_encode, e8m0_decode, E4M3_MAX


# ---------------------------------------------------------------- decoding

def bf16_to_f64(a):
    """bf16 given as uint16 bit patterns (numpy) or a torch bfloat16 tensor -> float64."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    except ImportError:  # pragma: no cover
        pass
    u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def as_f64(a):
    """bf16 (uint16 bits or torch bf16) -> float64; float64 arrays pass through
    (the finite-difference pins perturb float64 parameters)."""
    if isinstance(a, np.ndarray) and a.dtype == np.float64:
        return a
    return bf16_to_f64(a)


def dequant_weight(codes, scales, fmt):
    """Weight matrix [N][K] -> float64.

    fp8_b128: W[n,k] = dec(q[n,k]) * S[n//128, k//128]   (per-128 block FP8,
              DSV2-236B-MegaKernel README, "Results")
    mxfp8:    W[n,k] = dec(q[n,k]) * 2^(E[n, k//32] - 127)  (Mixture-of-Kittens,
              Table 2 caption: MXFP8 routed experts)
    bf16:     exact widening.
    The products are exact in float64 (4 significant bits times 24 bits).
    """
    if fmt == "bf16":
        return bf16_to_f64(codes)
    if fmt == "f64":   # float64 weights as given (finite-difference pins)
        return np.asarray(codes, dtype=np.float64)
    codes = np.asarray(codes, dtype=np.uint8)
    N, K = codes.shape
    out = np.empty((N, K))
    if fmt == "fp8_b128":
        s = np.asarray(scales, dtype=np.float32).astype(np.float64)

        def rows(a, b):   # 128-row blocks a..b
            q = _E4M3_TABLE[codes[a * 128:b * 128]]
            out[a * 128:b * 128] = (q.reshape(b - a, 128, K // 128, 128) * s[a:b, None, :, None]).reshape(-1, K)
        nblk = N // 128
    elif fmt == "mxfp8":
        s = e8m0_decode(scales)

        def rows(a, b):   # rows a..b
            q = _E4M3_TABLE[codes[a:b]]
            out[a:b] = (q.reshape(b - a, K // 32, 32) * s[a:b, :, None]).reshape(-1, K)
        nblk = N
    else:
        raise ValueError(fmt)
    # independent row ranges, on a few threads (numpy releases the interpreter lock)
    nt = os.cpu_count() or 1
    step = max(1, -(-nblk // nt))
    with ThreadPoolExecutor(max_workers=nt) as ex:
        list(ex.map(lambda a: rows(a, min(a + step, nblk)), range(0, nblk, step)))
    return out


_E4M3_TABLE = e4m3_decode(np.arange(256, dtype=np.uint8))


def _encode_rows(v):
    """e4m3_encode over the rows of a 3-D block array, in row chunks on a few
    threads (rows are independent; numpy releases the interpreter lock)."""
    n = v.shape[0]
    if n < 256:
        return e4m3_encode(v)
    out = np.empty(v.shape, dtype=np.uint8)
    step = max(64, -(-n // (4 * (os.cpu_count() or 1))))

    def work(a):
        out[a:a + step] = e4m3_encode(v[a:a + step])

    with ThreadPoolExecutor(max_workers=os.cpu_count() or 1) as ex:
        list(ex.map(work, range(0, n, step)))
    return out


# ------------------------------------------------- activation quantisation

def quant_act(v, afmt, return_codes=False):
    """Quantise rows of activations and return their dequantised float64 values.

    afmt "none": identity.
    afmt "fp8_1x128": per row, per 128 columns: s = fl32(amax / 448) (1 when
      amax = 0), code = RNE_e4m3(fl32(v / s)) saturating at +-448.
    afmt "mxfp8_1x32": per row, per 32 columns: X = 2^(floor(log2 amax) - 8)
      clamped to the e8m0 range (1 when amax = 0), code = RNE_e4m3(v / X).
    Input values are first rounded to fp32 (bf16 inputs are exact).
    With return_codes, also returns (codes uint8, scales) in the HIP layout:
    fp32 [rows][K/128] or e8m0 uint8 [rows][K/32].
    """
    v = np.asarray(v, dtype=np.float64)
    if afmt == "none":
        return (v, None, None) if return_codes else v
    v32 = v.astype(np.float32)
    rows, K = v32.shape
    if afmt == "fp8_1x128":
        blk = v32.reshape(rows, K // 128, 128)
        amax = np.abs(blk).max(axis=2)
        s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        t = (blk / s[:, :, None]).astype(np.float32)          # IEEE fp32 division
        codes = _encode_rows(t.astype(np.float64))
        deq = _E4M3_TABLE[codes] * s[:, :, None].astype(np.float64)
        out = deq.reshape(rows, K)
        if return_codes:
            return out, codes.reshape(rows, K), s
        return out
    if afmt == "mxfp8_1x32":
        blk = v32.reshape(rows, K // 32, 32)
        amax = np.abs(blk).max(axis=2).astype(np.float64)
        _, ex = np.frexp(np.where(amax > 0, amax, 1.0))       # amax = f * 2^ex, f in [0.5, 1)
        xe = np.clip(ex - 1 - 8, -127, 127)
        xe = np.where(amax > 0, xe, 0)
        X = np.ldexp(1.0, xe)
        codes = _encode_rows(blk.astype(np.float64) / X[:, :, None])
        deq = _E4M3_TABLE[codes] * X[:, :, None]
        out = deq.reshape(rows, K)
        if return_codes:
            return out, codes.reshape(rows, K), (xe + 127).astype(np.uint8)
        return out
    raise ValueError(afmt)


# ------------------------------------------------------------- stage M norm

def rmsnorm(h, gamma, eps):
    """Stage M of the DSV2-236B-MegaKernel flowchart (post-attention RMSNorm
    with weight gamma), producing the layer's bf16 input x.

    h, gamma: bf16 (uint16 bits or torch bf16) [T][H] and [H]; eps: float.
    ms = mean(h^2) over the row (float64; the squares of bf16 values are
    exact); r = fl32(1 / sqrt(ms + eps)); x = bf16(fl32(fl32(h * gamma) * r))
    with round-to-nearest-even at each step.  The pages do not fix the
    precision of the norm: the rounding points are those of a float32 norm
    whose output is the bf16 activation the router and the experts read.
    Returns x as uint16 bf16 bits [T][H] and r float32 [T].
    """
    hf = bf16_to_f64(h)
    g32 = bf16_to_f64(gamma).astype(np.float32)
    ms = np.sum(hf * hf, axis=1) / hf.shape[1]
    r = (1.0 / np.sqrt(ms + np.float64(np.float32(eps)))).astype(np.float32)
    p = hf.astype(np.float32) * g32[None, :]                    # exact: 8 x 8 significant bits
    xn = (p * r[:, None]).astype(np.float32)                    # one fp32 rounding
    return f32_to_bf16_bits(xn), r


def f32_to_bf16_bits(v):
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return np.where(nan, 0x7FC0, rounded).astype(np.uint16)


# ------------------------------------------------------------------ routing

def _group_view(cfg):
    E, G = cfg.n_experts, cfg.n_groups
    assert E % G == 0
    return E // G


def route(x, w_router, bias, cfg):
    """Router GEMV + softmax + group-limited greedy top-k (stages N and O).

    x: float64 [T][H]; w_router: float64 [E][H]; bias: float64 [E] or None.
    Returns dict(logits [T][E], scores [T][E], ids int32 [T][K] in descending
    score order, w float64 [T][K] = route_scale * score).

    The selection compares logits: softmax is monotone, so the logit order is
    the score order (and stays strict where a float64 score would underflow
    to 0).  Group score = max member logit; keep the TG best groups (ties to
    the lower group); take the K best experts of the kept groups (ties to the
    lower id).  -inf logits are candidates like any other: they tie with each
    other below every finite logit and get weight 0.  A token whose softmax is
    undefined (a NaN or +inf logit) has all its candidates tie, so it takes
    the lowest ids of the lowest groups; its weights are NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    logits = x @ np.asarray(w_router, dtype=np.float64).T
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)[None, :]
    with np.errstate(invalid="ignore"):
        m = logits.max(axis=1, keepdims=True)
        ex = np.exp(logits - m)
        scores = ex / ex.sum(axis=1, keepdims=True)
    T, E = scores.shape
    gsz = _group_view(cfg)
    G, TG, K = cfg.n_groups, cfg.topk_groups, cfg.topk
    ids = np.zeros((T, K), dtype=np.int32)
    w = np.zeros((T, K), dtype=np.float64)
    for t in range(T):
        l = logits[t]
        undefined = np.isnan(l).any() or np.isposinf(l).any()
        key = np.full(E, -np.inf) if undefined else l
        gs = key.reshape(G, gsz).max(axis=1)
        kept = np.argsort(-gs, kind="stable")[:TG]           # ties: lower group first
        cand = np.concatenate([np.arange(g * gsz, (g + 1) * gsz) for g in sorted(kept)])
        order = np.lexsort((cand, -key[cand]))                # by logit desc, then id asc
        sel = cand[order[:K]]
        ids[t] = sel
        w[t] = cfg.route_scale * scores[t, sel]
    return {"logits": logits, "scores": scores, "ids": ids, "w": w}


def route_bruteforce(scores_row, cfg):
    """Selection by enumeration, for tiny configs: the kept group set maximises
    the sum of group scores over all TG-subsets, and the expert set maximises
    the sum of scores over all K-subsets of the kept groups' experts.  Returns
    the ids in descending score order.  Unique when there are no ties."""
    G, TG, K = cfg.n_groups, cfg.topk_groups, cfg.topk
    gsz = _group_view(cfg)
    gs = scores_row.reshape(G, gsz).max(axis=1)
    best_g = max(combinations(range(G), TG), key=lambda c: sum(gs[list(c)]))
    cand = [e for g in best_g for e in range(g * gsz, (g + 1) * gsz)]
    best_e = max(combinations(cand, K), key=lambda c: sum(scores_row[list(c)]))
    return np.array(sorted(best_e, key=lambda e: -scores_row[e]), dtype=np.int32)


def route_margins(logits, cfg):
    """Smallest selection gap per token, in float64 logit space (after bias).

    Gaps: between the TG-th and (TG+1)-th group maxima (if TG < G), and
    between consecutive entries among the top K+1 logits of the kept groups'
    experts.  The generator redraws tokens whose gap is below 1e-3 so that the
    selection is unique and fp32 evaluation cannot reorder it.
    """
    T, E = logits.shape
    G, TG, K = cfg.n_groups, cfg.topk_groups, cfg.topk
    gsz = _group_view(cfg)
    out = np.full(T, np.inf)
    for t in range(T):
        l = logits[t]
        gm = l.reshape(G, gsz).max(axis=1)
        go = np.sort(gm)[::-1]
        gaps = []
        if TG < G:
            gaps.append(go[TG - 1] - go[TG])
        kept = np.argsort(-gm, kind="stable")[:TG]
        cand = np.sort(np.concatenate([l[g * gsz:(g + 1) * gsz] for g in kept]))[::-1]
        n = min(K + 1, cand.size)
        gaps.extend(cand[:n - 1] - cand[1:n])
        out[t] = min(gaps) if gaps else np.inf
    return out


# ----------------------------------------------------------------- dispatch

def permute(ids, n_experts):
    """Dispatch of the T*K (token, slot) pairs into per-expert segments.

    Flat slot p = t*K + j.  offsets = [0, cumsum(bincount)], perm_src[pos] = p
    for the stable order (expert asc, then p asc), inv_pos[p] = pos.
    """
    flat = np.asarray(ids, dtype=np.int64).ravel()
    perm_src = np.argsort(flat, kind="stable").astype(np.int32)
    counts = np.bincount(flat, minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    inv_pos = np.empty_like(perm_src)
    inv_pos[perm_src] = np.arange(flat.size, dtype=np.int32)
    return offsets, perm_src, inv_pos


# ---------------------------------------------------------------------- FFN

def silu(g):
    return g / (1.0 + np.exp(-g))


def expert_ffn(X, wg, wu, wd, afmt):
    """One expert on rows X (float64): stages P1 and P2 of the flowchart.

    wg, wu: float64 [I][H]; wd: float64 [H][I] (dequantised).
    X and h go through quant_act(afmt) before their matmuls.
    """
    Xq = quant_act(X, afmt)
    g = Xq @ wg.T
    u = Xq @ wu.T
    h = silu(g) * u
    hq = quant_act(h, afmt)
    return hq @ wd.T


def combine(y_perm, inv_pos, w, shared=None):
    """Stage R's sum: out[t] = sum_j w[t,j] * y_perm[inv_pos[t*K+j]] (+ shared[t]);
    slots with inv_pos < 0 contribute nothing."""
    w = np.asarray(w, dtype=np.float64)
    T, K = w.shape
    inv = np.asarray(inv_pos).reshape(T, K)
    y = np.asarray(y_perm, dtype=np.float64)
    out = np.zeros((T, y.shape[1]))
    for t in range(T):
        for j in range(K):
            if inv[t, j] >= 0:
                out[t] += w[t, j] * y[inv[t, j]]
    if shared is not None:
        out += np.asarray(shared, dtype=np.float64)
    return out


class _Dequant:
    """Per-expert dequantisation with a small cache."""

    def __init__(self, weights, fmt):
        self.w, self.fmt, self.cache = weights, fmt, {}

    def __call__(self, e):
        if e not in self.cache:
            if len(self.cache) > 48:
                self.cache.clear()
            g, u, d, gs, us, ds = self.w.expert(e)
            self.cache[e] = (dequant_weight(g, gs, self.fmt), dequant_weight(u, us, self.fmt),
                             dequant_weight(d, ds, self.fmt))
        return self.cache[e]


@dataclass
class OracleResult:
    logits: np.ndarray
    ids: np.ndarray
    w: np.ndarray
    offsets: np.ndarray
    perm_src: np.ndarray
    inv_pos: np.ndarray
    y_perm: np.ndarray
    shared: Optional[np.ndarray]
    out: np.ndarray


def forward(cfg, x, w_router, bias, routed, shared, norm=None):
    """Whole layer.  x, w_router: bf16 (uint16 bits or torch bf16); bias f32 or
    None; routed/shared: objects with .fmt and .expert(e) -> (gate, up, down,
    gate_s, up_s, down_s) host arrays.  Output out is the unrounded float64
    sum_j w_j * Y_j + S (stage R without the residual).
    norm: None, or (gamma, eps): x is then the pre-norm h and the layer runs
    on rmsnorm(h, gamma, eps) (stage M before stage N)."""
    if norm is not None:
        x, _ = rmsnorm(x, norm[0], norm[1])
    xf = as_f64(x)
    wr = as_f64(w_router)
    b = None if bias is None else _f64(bias)
    r = route(xf, wr, b, cfg)
    T, K = r["ids"].shape
    offsets, perm_src, inv_pos = permute(r["ids"], cfg.n_experts)
    deq = _Dequant(routed, routed.fmt)
    y_perm = np.zeros((T * K, cfg.hidden))
    for e in range(cfg.n_experts):
        a, z = offsets[e], offsets[e + 1]
        if a == z:
            continue
        wg, wu, wd = deq(e)
        y_perm[a:z] = expert_ffn(xf[perm_src[a:z] // K], wg, wu, wd, cfg.routed_afmt)
    S = None
    if shared is not None:
        wg, wu, wd = _Dequant(shared, shared.fmt)(0)
        S = expert_ffn(xf, wg, wu, wd, cfg.shared_afmt)
    out = combine(y_perm, inv_pos, r["w"], S)
    return OracleResult(r["logits"], r["ids"], r["w"], offsets, perm_src, inv_pos, y_perm, S, out)


def forward_tokens(cfg, x, w_router, bias, routed, shared, tokens, deq_cache=None):
    """Output rows of the listed tokens only (each token's path is independent
    of the others: routing, per-row quantisation and FFN act row by row).
    Returns (ids [n][K], w [n][K], out [n][H])."""
    tokens = np.asarray(tokens, dtype=np.int64)
    xf = bf16_to_f64(x)[tokens] if not _is_f64(x) else np.asarray(x)[tokens]
    r = route(xf, bf16_to_f64(w_router), None if bias is None else _f64(bias), cfg)
    deq = deq_cache if deq_cache is not None else _Dequant(routed, routed.fmt)
    out = np.zeros((tokens.size, cfg.hidden))
    for i in range(tokens.size):
        for j in range(cfg.topk):
            wg, wu, wd = deq(int(r["ids"][i, j]))
            out[i] += r["w"][i, j] * expert_ffn(xf[i:i + 1], wg, wu, wd, cfg.routed_afmt)[0]
    if shared is not None:
        wg, wu, wd = _Dequant(shared, shared.fmt)(0)
        out += expert_ffn(xf, wg, wu, wd, cfg.shared_afmt)
    return r["ids"], r["w"], out


def forward_dense_masked(cfg, x, w_router, bias, routed, shared):
    """Brute-force layer: every token through every expert, gated by its
    routing weight or 0; no permutation.  Must equal forward().out."""
    xf = bf16_to_f64(x)
    r = route(xf, bf16_to_f64(w_router), None if bias is None else _f64(bias), cfg)
    T = xf.shape[0]
    gate = np.zeros((T, cfg.n_experts))
    for t in range(T):
        gate[t, r["ids"][t]] = r["w"][t]
    deq = _Dequant(routed, routed.fmt)
    out = np.zeros((T, cfg.hidden))
    for e in range(cfg.n_experts):
        wg, wu, wd = deq(e)
        for t in range(T):
            out[t] += gate[t, e] * expert_ffn(xf[t:t + 1], wg, wu, wd, cfg.routed_afmt)[0]
    if shared is not None:
        wg, wu, wd = _Dequant(shared, shared.fmt)(0)
        out += expert_ffn(xf, wg, wu, wd, cfg.shared_afmt)
    return out


def _is_f64(a):
    return isinstance(a, np.ndarray) and a.dtype == np.float64


def _f64(a):
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return a.detach().cpu().double().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(a, dtype=np.float64)
