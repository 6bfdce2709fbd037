"""Test helpers: margin-checked input draws and the parity metric."""
import numpy as np
import torch

import oracle
import synth

MARGIN = 1e-3


def ensure_margin(inp, max_attempts=100):
    """Redraw tokens whose routing gap (float64 logit space, after bias) is
    below 1e-3, so expert ids are unique and robust to fp32 evaluation."""
    cfg = inp.cfg
    wr = oracle.bf16_to_f64(inp.w_router)
    bias = None if inp.bias is None else inp.bias.detach().cpu().double().numpy()
    todo = np.arange(cfg.tokens)
    for attempt in range(max_attempts):
        rows = inp.x[torch.as_tensor(todo, device=inp.x.device)]
        if cfg.norm:   # the router reads the normalised x
            rows, _ = oracle.rmsnorm(rows, inp.gamma, cfg.norm_eps)
        x = oracle.bf16_to_f64(rows)
        logits = x @ wr.T
        if bias is not None:
            logits = logits + bias
        m = oracle.route_margins(logits, cfg)
        bad = todo[m < MARGIN]
        if bad.size == 0:
            return inp
        synth.redraw_tokens(inp, bad, attempt)
        todo = bad
    raise RuntimeError("could not meet the routing margin")


def norm_of(inp):
    """The oracle's norm argument for a layer's inputs (None without a norm)."""
    return (inp.gamma, inp.cfg.norm_eps) if inp.cfg.norm else None


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def small_cfg(base, **kw):
    """A reduced layer with the base config's formats and routing rule."""
    return synth.get_config(base).derive(**kw)
