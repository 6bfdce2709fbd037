"""Python binding of libmoe.so, the MI355X (gfx950) MoE layer forward.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Tensors are torch CUDA (HIP) tensors; their device pointers and the
current HIP stream are handed to the C ABI declared in include/moe.h.  The
library must be built (python -m mixture_experts_layer_router_amd.build);
importing works without it, but every call raises if it is missing.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libmoe.so")

WFMT = {"bf16": 0, "fp8_b128": 1, "mxfp8": 2}
AFMT = {"none": 0, "fp8_1x128": 1, "mxfp8_1x32": 2}

STATUS = {0: "MOE_OK", 1: "MOE_EINVAL", 2: "MOE_EUNSUPPORTED", 3: "MOE_EALIGN", 4: "MOE_EWORKSPACE", 5: "MOE_EHIP",
          6: "MOE_EWAIT"}


class MoEError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {_lib().moe_status_string(status).decode()} ({status})")


class Config(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("n_groups", ctypes.c_int32),
        ("topk_groups", ctypes.c_int32), ("topk", ctypes.c_int32), ("inter", ctypes.c_int32),
        ("shared_inter", ctypes.c_int32), ("route_scale", ctypes.c_float),
        ("routed_wfmt", ctypes.c_int32), ("shared_wfmt", ctypes.c_int32),
        ("routed_afmt", ctypes.c_int32), ("shared_afmt", ctypes.c_int32),
    ]


class Norm(ctypes.Structure):
    _fields_ = [("gamma", ctypes.c_void_p), ("eps", ctypes.c_float)]


class FfnGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("gate", "up", "down")]


class FfnWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("gate", "up", "down", "gate_s", "up_s", "down_s")]


_LIB = None
_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mixture_experts_layer_router_amd.build` (no CPU fallback exists)")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        sig = {
            "moe_status_string": (ctypes.c_char_p, [_i32]),
            "moe_workspace_size": (_i32, [P(Config), _i32, P(_sz)]),
            "moe_route": (_i32, [P(Config), _vp, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
            "moe_permute": (_i32, [P(Config), _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
            "moe_expert_ffn": (_i32, [P(Config), _i32, _vp, _vp, _i32, _vp, P(FfnWeights), _vp, _vp, _sz, _vp]),
            "moe_combine": (_i32, [P(Config), _vp, _vp, _vp, _vp, _i32, _vp, _vp]),
            "moe_forward": (_i32, [P(Config), _vp, _i32, _vp, _vp, P(FfnWeights), P(FfnWeights), _vp, _vp, _vp,
                                   _vp, _sz, _vp]),
            "moe_workspace_check": (_i32, [_vp, _sz, _i32, _vp]),
            "moe_backward_workspace_size": (_i32, [P(Config), _i32, P(_sz)]),
            "moe_backward": (_i32, [P(Config), _vp, _i32, _vp, _vp, P(FfnWeights), P(FfnWeights), _vp, _vp, _vp, _vp,
                                    P(FfnGrads), P(FfnGrads), _vp, _sz, _vp]),
            "moe_route_dispatch": (_i32, [P(Config), _vp, _i32, P(Norm), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                          _vp, _vp, _sz, _vp]),
            "moe_forward_norm": (_i32, [P(Config), _vp, _i32, P(Norm), _vp, _vp, P(FfnWeights), P(FfnWeights), _vp,
                                        _vp, _vp, _vp, _vp, _sz, _vp]),
            "moe_forward_noalloc": (_i32, [P(Config), _vp, _i32, _vp, _vp, P(FfnWeights), P(FfnWeights), _vp, _vp,
                                           _vp, _vp]),
            "moe_debug_ws_offset": (_i32, [P(Config), _i32, _i32, P(_sz)]),
            "moe_debug_validate_dispatch": (_i32, [P(Config), _i32, _vp, _vp, _sz, _vp, _vp]),
            "moe_debug_ffn_tile_rows": (_i32, [P(Config), _i32]),
            "moe_debug_e4m3_decode": (_i32, [_vp, _vp, _i32, _vp]),
            "moe_debug_e4m3_encode": (_i32, [_vp, _vp, _i32, _vp]),
            "moe_debug_trace": (_i32, [_vp, _i32]),
            "moe_debug_trace_count": (_i32, []),
            "moe_debug_trace_name": (ctypes.c_char_p, [_i32]),
        }
        for name, (res, args) in sig.items():
            f = getattr(lib, name)
            f.restype, f.argtypes = res, args
        _LIB = lib
    return _LIB


EXPORTS = ("moe_status_string", "moe_workspace_size", "moe_route", "moe_permute", "moe_expert_ffn",
           "moe_combine", "moe_forward", "moe_backward", "moe_backward_workspace_size", "moe_forward_norm", "moe_route_dispatch", "moe_forward_noalloc", "moe_workspace_check", "moe_debug_ws_offset",
           "moe_debug_validate_dispatch",
           "moe_debug_ffn_tile_rows", "moe_debug_e4m3_decode", "moe_debug_e4m3_encode", "moe_debug_trace",
           "moe_debug_trace_count", "moe_debug_trace_name")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(st, where):
    if st != 0:
        raise MoEError(st, where)


def make_config(layer):
    """Config from any object with the layer fields (hidden, n_experts, ...,
    routed_wfmt as a format name)."""
    return Config(layer.hidden, layer.n_experts, layer.n_groups, layer.topk_groups, layer.topk, layer.inter,
                  layer.shared_inter, float(layer.route_scale), WFMT[layer.routed_wfmt], WFMT[layer.shared_wfmt],
                  AFMT[layer.routed_afmt], AFMT[layer.shared_afmt])


def make_weights(gate, up, down, gate_s=None, up_s=None, down_s=None):
    w = FfnWeights(*[None if t is None else t.data_ptr() for t in (gate, up, down, gate_s, up_s, down_s)])
    w._keep = (gate, up, down, gate_s, up_s, down_s)
    return w


def weights_of(ew):
    """FfnWeights from an object with gate/up/down(+_s) tensors."""
    return None if ew is None else make_weights(ew.gate, ew.up, ew.down, ew.gate_s, ew.up_s, ew.down_s)


def workspace_size(cfg, max_tokens):
    n = ctypes.c_size_t(0)
    _check(_lib().moe_workspace_size(ctypes.byref(cfg), int(max_tokens), ctypes.byref(n)), "moe_workspace_size")
    return n.value


def alloc_workspace(cfg, max_tokens, device="cuda"):
    return torch.zeros(workspace_size(cfg, max_tokens), dtype=torch.uint8, device=device)


def _u16(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def route(cfg, x, w_router, bias, ids, w, ws, stream=None):
    _check(_lib().moe_route(ctypes.byref(cfg), _ptr(x), x.shape[0], _ptr(w_router), _ptr(bias), _ptr(ids), _ptr(w),
                            _ptr(ws), ws.numel(), _stream(stream)), "moe_route")


def permute(cfg, ids, T, x, offsets, perm_src, inv_pos, x_perm, x_perm_scale, ws, stream=None):
    _check(_lib().moe_permute(ctypes.byref(cfg), _ptr(ids), int(T), _ptr(x), _ptr(offsets), _ptr(perm_src),
                              _ptr(inv_pos), _ptr(x_perm), _ptr(x_perm_scale), _ptr(ws), ws.numel(),
                              _stream(stream)), "moe_permute")


def expert_ffn(cfg, which, x, x_scale, rows, seg_offsets, weights, y, ws, stream=None):
    _check(_lib().moe_expert_ffn(ctypes.byref(cfg), int(which), _ptr(x), _ptr(x_scale), int(rows), _ptr(seg_offsets),
                                 ctypes.byref(weights), _ptr(y), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_expert_ffn")


def combine(cfg, y_perm, inv_pos, topk_w, y_shared, T, out, stream=None):
    _check(_lib().moe_combine(ctypes.byref(cfg), _ptr(y_perm), _ptr(inv_pos), _ptr(topk_w), _ptr(y_shared), int(T),
                              _ptr(out), _stream(stream)), "moe_combine")


def forward(cfg, x, w_router, bias, routed, shared, out, ids, w, ws, stream=None):
    """routed/shared: FfnWeights (shared may be None)."""
    _check(_lib().moe_forward(ctypes.byref(cfg), _ptr(x), x.shape[0], _ptr(w_router), _ptr(bias),
                              ctypes.byref(routed), None if shared is None else ctypes.byref(shared), _ptr(out),
                              _ptr(ids), _ptr(w), _ptr(ws), ws.numel(), _stream(stream)), "moe_forward")


def workspace_check(ws, clear=True, stream=None):
    """Raise MoEError(MOE_EWAIT) if a bounded wait of the single-launch path
    gave up in an earlier call on this workspace (synchronises the stream)."""
    _check(_lib().moe_workspace_check(_ptr(ws), ws.numel(), int(bool(clear)), _stream(stream)), "moe_workspace_check")


WS_REGIONS = {"offsets": 0, "perm_src": 1, "inv_pos": 2, "tiles": 3, "ntiles": 4}


def ws_region(cfg, max_tokens, ws, name, count):
    """int32 view of `count` entries of a dispatch region of a workspace (test hook)."""
    off = ctypes.c_size_t(0)
    _check(_lib().moe_debug_ws_offset(ctypes.byref(cfg), int(max_tokens), WS_REGIONS[name], ctypes.byref(off)),
           "moe_debug_ws_offset")
    return ws[off.value:off.value + 4 * count].view(torch.int32)


def validate_dispatch(cfg, T, ids, ws, stream=None):
    """Bit mask of the dispatch checks that fail on the arrays a batched call
    left in `ws` for the ids `ids` (0: all hold; synchronises the stream)."""
    flags = torch.zeros(1, dtype=torch.int32, device=ws.device)
    _check(_lib().moe_debug_validate_dispatch(ctypes.byref(cfg), int(T), _ptr(ids), _ptr(ws), ws.numel(), _ptr(flags),
                                              _stream(stream)), "moe_debug_validate_dispatch")
    torch.cuda.synchronize(ws.device)
    return int(flags.item())


def ffn_tile_rows(cfg, which):
    return _lib().moe_debug_ffn_tile_rows(ctypes.byref(cfg), int(which))


def make_norm(gamma, eps):
    n = Norm(gamma.data_ptr(), float(eps))
    n._keep = gamma
    return n


def route_dispatch(cfg, h, norm, w_router, bias, ids, w, offsets, perm_src, inv_pos, x_out, xq, xq_scale, ws,
                   stream=None):
    """norm: Norm or None."""
    _check(_lib().moe_route_dispatch(ctypes.byref(cfg), _ptr(h), h.shape[0], None if norm is None else ctypes.byref(norm),
                                     _ptr(w_router), _ptr(bias), _ptr(ids), _ptr(w), _ptr(offsets), _ptr(perm_src),
                                     _ptr(inv_pos), _ptr(x_out), _ptr(xq), _ptr(xq_scale), _ptr(ws), ws.numel(),
                                     _stream(stream)), "moe_route_dispatch")


def forward_norm(cfg, h, norm, w_router, bias, routed, shared, out, ids, w, x_out, ws, stream=None):
    _check(_lib().moe_forward_norm(ctypes.byref(cfg), _ptr(h), h.shape[0], ctypes.byref(norm), _ptr(w_router),
                                   _ptr(bias), ctypes.byref(routed), None if shared is None else ctypes.byref(shared),
                                   _ptr(out), _ptr(ids), _ptr(w), _ptr(x_out), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_forward_norm")


def make_grads(gate, up, down):
    g = FfnGrads(gate.data_ptr(), up.data_ptr(), down.data_ptr())
    g._keep = (gate, up, down)
    return g


def backward_workspace_size(cfg, max_tokens):
    n = ctypes.c_size_t(0)
    _check(_lib().moe_backward_workspace_size(ctypes.byref(cfg), int(max_tokens), ctypes.byref(n)),
           "moe_backward_workspace_size")
    return n.value


def backward(cfg, x, w_router, bias, routed, shared, dy, dx, d_router, d_bias, d_routed, d_shared, ws, stream=None):
    """routed/shared: FfnWeights; d_routed/d_shared: FfnGrads (d_shared None without a shared expert)."""
    _check(_lib().moe_backward(ctypes.byref(cfg), _ptr(x), x.shape[0], _ptr(w_router), _ptr(bias), ctypes.byref(routed),
                               None if shared is None else ctypes.byref(shared), _ptr(dy), _ptr(dx), _ptr(d_router),
                               _ptr(d_bias), ctypes.byref(d_routed), None if d_shared is None else ctypes.byref(d_shared),
                               _ptr(ws), ws.numel(), _stream(stream)), "moe_backward")


def forward_noalloc(cfg, x, w_router, bias, routed, shared, out, ids, w, stream=None):
    """moe_forward on the library's own per-GPU device array (no workspace)."""
    _check(_lib().moe_forward_noalloc(ctypes.byref(cfg), _ptr(x), x.shape[0], _ptr(w_router), _ptr(bias),
                                      ctypes.byref(routed), None if shared is None else ctypes.byref(shared),
                                      _ptr(out), _ptr(ids), _ptr(w), _stream(stream)), "moe_forward_noalloc")


def e4m3_decode(codes, out, stream=None):
    _check(_lib().moe_debug_e4m3_decode(_ptr(codes), _ptr(out), codes.numel(), _stream(stream)), "e4m3_decode")


def e4m3_encode(vals, codes, stream=None):
    _check(_lib().moe_debug_e4m3_encode(_ptr(vals), _ptr(codes), vals.numel(), _stream(stream)), "e4m3_encode")


class LaunchTrace:
    """Bracket every kernel launch of the library with HIP events (measurement only).

    with LaunchTrace(max_launches) as tr:
        ...calls...
    tr.kernels() -> [(name, ms), ...] after a synchronize.
    """

    def __init__(self, max_launches=4096):
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * max_launches)]

    def __enter__(self):
        for e in self.events:   # torch creates the HIP event on first record
            e.record()
        torch.cuda.synchronize()
        handles = [e.cuda_event for e in self.events]
        if not all(handles):
            raise RuntimeError("torch did not create the HIP events")
        self._arr = (ctypes.c_void_p * len(self.events))(*handles)
        _check(_lib().moe_debug_trace(self._arr, len(self.events)), "moe_debug_trace")
        return self

    def __exit__(self, *exc):
        self.n = _lib().moe_debug_trace_count()
        self.names = [_lib().moe_debug_trace_name(i).decode() for i in range(self.n)]
        _lib().moe_debug_trace(None, 0)

    def kernels(self):
        torch.cuda.synchronize()
        return [(self.names[i], self.events[2 * i].elapsed_time(self.events[2 * i + 1])) for i in range(self.n)]


class Layer:
    """Convenience holder: one layer's config, device weights and workspace."""

    def __init__(self, layer_cfg, inputs, max_tokens=None):
        self.lc = layer_cfg
        self.cfg = make_config(layer_cfg)
        self.inp = inputs
        self.routed = weights_of(inputs.routed)
        self.shared = weights_of(inputs.shared)
        T = max_tokens or layer_cfg.tokens
        self.ws = alloc_workspace(self.cfg, T, inputs.x.device)

    def forward(self, x=None, out=None, ids=None, w=None, stream=None):
        x = self.inp.x if x is None else x
        T = x.shape[0]
        dev = x.device
        out = torch.empty(T, self.lc.hidden, dtype=torch.bfloat16, device=dev) if out is None else out
        ids = torch.empty(T, self.lc.topk, dtype=torch.int32, device=dev) if ids is None else ids
        w = torch.empty(T, self.lc.topk, dtype=torch.float32, device=dev) if w is None else w
        if getattr(self.lc, "norm", False):
            if not hasattr(self, "_norm"):
                self._norm = make_norm(self.inp.gamma, self.lc.norm_eps)
            forward_norm(self.cfg, x, self._norm, self.inp.w_router, self.inp.bias, self.routed, self.shared, out, ids,
                         w, None, self.ws, stream)
        else:
            forward(self.cfg, x, self.inp.w_router, self.inp.bias, self.routed, self.shared, out, ids, w, self.ws,
                    stream)
        return out, ids, w
