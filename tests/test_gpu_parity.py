"""Parity of the HIP path (through the C ABI) with the fp64 oracle on MI355X.

Bars: expert ids, dispatch offsets / permutation / inverse and quantised codes
of x bit-exact; routing weights within 1e-4 relative (fp32 logits carry
~1e-5 absolute error, and w moves with exp of it); layer output within
max|err| / max|ref| <= 2e-2 of the unrounded fp64 oracle.
"""
import os
import sys

import numpy as np
import pytest
import torch

import mixture_experts_layer_router_amd as moe
import oracle
import synth
from helpers import ensure_margin, rel_err, small_cfg

pytestmark = pytest.mark.gpu
TOL = 2e-2
WTOL = 1e-4
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


SMALL = {
    "tiny_8tok": small_cfg(0),
    "gemv_dsv2_3tok": small_cfg(1, tokens=3, hidden=384, n_experts=16, n_groups=4, topk_groups=2, topk=3,
                                inter=256, shared_inter=256),
    "b128_4exp_150tok": small_cfg(2, tokens=150, hidden=384, n_experts=4, n_groups=2, topk_groups=1, topk=2,
                                  inter=256, shared_inter=384),
    "b128_12exp_97tok": small_cfg(2, tokens=97, hidden=512, n_experts=12, n_groups=3, topk_groups=2, topk=3,
                                  inter=384, shared_inter=256),
    "mx_4exp_160tok": small_cfg(3, tokens=160, hidden=512, n_experts=4, inter=256, shared_inter=256),
    "zipf_16exp_200tok": small_cfg(4, tokens=200, hidden=256, n_experts=16, n_groups=4, topk_groups=2, topk=4,
                                   inter=128, shared_inter=128),
    "flat_k1_64tok": small_cfg(0, tokens=64, n_experts=8, n_groups=1, topk_groups=1, topk=1, shared_inter=0),
    "one_group_32tok": small_cfg(2, tokens=32, hidden=256, n_experts=16, n_groups=4, topk_groups=1, topk=2,
                                 inter=128, shared_inter=128),
    # small T: the decode path (router || shared gate/up, top-k || shared down)
    "b128_quant_2tok": small_cfg(2, tokens=2, hidden=384, n_experts=16, n_groups=4, topk_groups=2, topk=3,
                                 inter=256, shared_inter=256),
    "mx_3tok": small_cfg(3, tokens=3, hidden=512, n_experts=8, inter=256, shared_inter=256),
    "bf16_1tok": small_cfg(0, tokens=1),
    "b128_4tok_noshared": small_cfg(1, tokens=4, hidden=256, n_experts=12, n_groups=3, topk_groups=2, topk=2,
                                    inter=128, shared_inter=0),
    # small T with bf16 activations: the single-launch path
    "mx_none_2tok": small_cfg(3, tokens=2, hidden=512, n_experts=8, inter=256, shared_inter=256,
                              routed_afmt="none"),
    "dsv2_like_4tok": small_cfg(1, tokens=4, hidden=1024, n_experts=64, n_groups=8, topk_groups=3, topk=6,
                                inter=512, shared_inter=1024),
    "mx_both_3tok": small_cfg(3, tokens=3, hidden=512, n_experts=8, inter=256, shared_inter=384,
                              routed_afmt="none", shared_wfmt="mxfp8"),
    "bf16_long_k_2tok": small_cfg(0, tokens=2, hidden=512, n_experts=16, topk=4, inter=1536, shared_inter=2048),
}


def gpu_inputs(cfg, with_experts=True):
    say(f"[inputs] {cfg.name} T={cfg.tokens} H={cfg.hidden} E={cfg.n_experts}")
    return ensure_margin(synth.make_inputs(cfg, DEV, with_experts=with_experts))


def pairs_ok(cfg):
    ok = {("bf16", "none"), ("fp8_b128", "fp8_1x128"), ("mxfp8", "mxfp8_1x32")}
    return (cfg.routed_wfmt, cfg.routed_afmt) in ok and (cfg.shared_inter == 0 or
                                                         (cfg.shared_wfmt, cfg.shared_afmt) in ok)


# ---------------------------------------------------------------- codec

def test_device_e4m3_codec_matches_oracle():
    codes = torch.arange(256, dtype=torch.uint8, device=DEV)
    out = torch.empty(256, dtype=torch.float32, device=DEV)
    moe.e4m3_decode(codes, out)
    torch.cuda.synchronize()
    ref = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    got = out.cpu().double().numpy()
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    rng = np.random.default_rng(11)
    pos = np.arange(0, 0x7E, dtype=np.uint8)
    mids = (oracle.e4m3_decode(pos) + oracle.e4m3_decode(pos + 1)) / 2
    vals = np.concatenate([rng.standard_normal(50000) * s for s in (1e-3, 0.1, 1, 50, 400)] +
                          [mids, -mids, [448.0, 460.0, 1e6, -1e6, 0.0, -0.0, 2.0 ** -10, 2.0 ** -11]]).astype(np.float32)
    vt = torch.from_numpy(vals).to(DEV)
    qc = torch.empty(vals.size, dtype=torch.uint8, device=DEV)
    moe.e4m3_encode(vt, qc)
    torch.cuda.synchronize()
    want = oracle.e4m3_encode(vals.astype(np.float64))
    got = qc.cpu().numpy()
    # -0.0 and +0.0 both encode to a zero code; compare values for zeros
    nz = vals != 0
    assert np.array_equal(got[nz], want[nz])
    assert np.all((got[~nz] & 0x7F) == 0)


# ---------------------------------------------------------------- routing

def _route(cfg, inp):
    c = moe.make_config(cfg)
    ws = moe.alloc_workspace(c, cfg.tokens)
    ids = torch.empty(cfg.tokens, cfg.topk, dtype=torch.int32, device=DEV)
    w = torch.empty(cfg.tokens, cfg.topk, dtype=torch.float32, device=DEV)
    moe.route(c, inp.x, inp.w_router, inp.bias, ids, w, ws)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def _oracle_route(cfg, inp):
    b = None if inp.bias is None else inp.bias.double().cpu().numpy()
    return oracle.route(oracle.bf16_to_f64(inp.x), oracle.bf16_to_f64(inp.w_router), b, cfg)


@pytest.mark.parametrize("name", list(SMALL) + ["full:" + c.name for c in synth.CONFIGS])
def test_route(name):
    cfg = SMALL[name] if name in SMALL else synth.get_config(name[5:])
    inp = gpu_inputs(cfg, with_experts=False)
    say(f"[route] {name}")
    ids, w = _route(cfg, inp)
    r = _oracle_route(cfg, inp)
    assert np.array_equal(ids, r["ids"])
    assert np.max(np.abs(w - r["w"]) / np.abs(r["w"])) <= WTOL


# ---------------------------------------------------------------- dispatch

@pytest.mark.parametrize("afmt", ["none", "fp8_1x128", "mxfp8_1x32"])
# slots T*K: 6; 3,000 (3 chunks of 1,024); 999; 512; exactly 1,024 (one full chunk); 2,049 (a
# 1-slot tail chunk); 24,576 (24 chunks, skewed like the 4,096-token workload)
@pytest.mark.parametrize("T,E,K", [(1, 160, 6), (500, 160, 6), (333, 7, 3), (64, 256, 8), (512, 16, 2),
                                   (683, 12, 3), (4096, 160, 6)])
def test_permute(T, E, K, afmt):
    rng = np.random.default_rng(T * 7 + E + K)
    if E == 160 and T > 1:   # skewed popularity, leaves some experts empty
        p = 1.0 / np.arange(1, E + 1) ** 1.2
        ids = np.stack([rng.choice(E, K, replace=False, p=p / p.sum()) for _ in range(T)])
    else:
        ids = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
    ids = ids.astype(np.int32)
    cfg = small_cfg(2, tokens=T, hidden=256, n_experts=E, n_groups=1, topk_groups=1, topk=K, inter=128,
                    shared_inter=0, routed_afmt=afmt, routed_wfmt={"none": "bf16", "fp8_1x128": "fp8_b128",
                                                                   "mxfp8_1x32": "mxfp8"}[afmt])
    say(f"[permute] T={T} E={E} K={K} {afmt}")
    c = moe.make_config(cfg)
    ws = moe.alloc_workspace(c, T)
    x = synth.draw_tokens(cfg, DEV)
    idt = torch.from_numpy(ids).to(DEV)
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    perm = torch.empty(T * K, dtype=torch.int32, device=DEV)
    inv = torch.empty(T * K, dtype=torch.int32, device=DEV)
    if afmt == "none":
        xp = torch.empty(T * K, 256, dtype=torch.bfloat16, device=DEV)
        xs = None
    else:
        xp = torch.empty(T * K, 256, dtype=torch.uint8, device=DEV)
        xs = torch.empty(T * K, 2 if afmt == "fp8_1x128" else 8, dtype=torch.float32 if afmt == "fp8_1x128" else torch.uint8,
                         device=DEV)
    moe.permute(c, idt, T, x, off, perm, inv, xp, xs, ws)
    torch.cuda.synchronize()
    o_off, o_perm, o_inv = oracle.permute(ids, E)
    assert np.array_equal(off.cpu().numpy(), o_off)
    assert np.array_equal(perm.cpu().numpy(), o_perm)
    assert np.array_equal(inv.cpu().numpy(), o_inv)
    rows = oracle.bf16_to_f64(x)[o_perm // K]
    if afmt == "none":
        assert np.array_equal(oracle.bf16_to_f64(xp), rows)
    else:
        _, q, s = oracle.quant_act(rows, afmt, return_codes=True)
        assert np.array_equal(xp.cpu().numpy(), q)
        assert np.array_equal(xs.cpu().numpy(), s)


# ---------------------------------------------------------------- expert FFN

# only the (config, path) pairs the library serves: the GEMM path has no
# kernel for some weight / activation format pairs
@pytest.mark.parametrize("name,path", [(n, p) for n in ["tiny_8tok", "b128_4exp_150tok", "mx_4exp_160tok",
                                                         "gemv_dsv2_3tok"]
                                       for p in ["gemv", "gemm"] if p != "gemm" or pairs_ok(SMALL[n])])
def test_expert_ffn(name, path, monkeypatch):
    cfg = SMALL[name]
    monkeypatch.setenv("MOE_FORCE_PATH", path)
    inp = gpu_inputs(cfg)
    r = oracle.forward(cfg, inp.x, inp.w_router, inp.bias, inp.routed, inp.shared)
    T, K, H = cfg.tokens, cfg.topk, cfg.hidden
    c = moe.make_config(cfg)
    ws = moe.alloc_workspace(c, T)
    xperm = inp.x[torch.from_numpy(r.perm_src // K).long().to(DEV)].contiguous()
    off = torch.from_numpy(r.offsets).to(DEV)
    y = torch.empty(T * K, H, dtype=torch.float32, device=DEV)
    say(f"[expert_ffn routed] {name} {path}")
    moe.expert_ffn(c, 0, xperm, None, T * K, off, moe.weights_of(inp.routed), y, ws)
    torch.cuda.synchronize()
    assert rel_err(y.cpu().numpy(), r.y_perm) <= TOL
    if cfg.shared_inter:
        ys = torch.empty(T, H, dtype=torch.float32, device=DEV)
        say(f"[expert_ffn shared] {name} {path}")
        moe.expert_ffn(c, 1, inp.x, None, T, None, moe.weights_of(inp.shared), ys, ws)
        torch.cuda.synchronize()
        assert rel_err(ys.cpu().numpy(), r.shared) <= TOL


def test_expert_ffn_prequantised_rows(monkeypatch):
    cfg = SMALL["b128_4exp_150tok"]
    inp = gpu_inputs(cfg)
    r = oracle.forward(cfg, inp.x, inp.w_router, inp.bias, inp.routed, inp.shared)
    T, K, H = cfg.tokens, cfg.topk, cfg.hidden
    c = moe.make_config(cfg)
    ws = moe.alloc_workspace(c, T)
    _, q, s = oracle.quant_act(oracle.bf16_to_f64(inp.x)[r.perm_src // K], "fp8_1x128", return_codes=True)
    qt, st = torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV)
    off = torch.from_numpy(r.offsets).to(DEV)
    for path in ("gemv", "gemm"):
        monkeypatch.setenv("MOE_FORCE_PATH", path)
        y = torch.empty(T * K, H, dtype=torch.float32, device=DEV)
        say(f"[expert_ffn prequantised] {path}")
        moe.expert_ffn(c, 0, qt, st, T * K, off, moe.weights_of(inp.routed), y, ws)
        torch.cuda.synchronize()
        assert rel_err(y.cpu().numpy(), r.y_perm) <= TOL


# ---------------------------------------------------------------- combine

def test_combine():
    rng = np.random.default_rng(5)
    T, K, H, E = 37, 3, 384, 9
    ids = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    _, perm, inv = oracle.permute(ids, E)
    yp = rng.standard_normal((T * K, H)).astype(np.float32)
    ys = rng.standard_normal((T, H)).astype(np.float32)
    w = rng.random((T, K)).astype(np.float32)
    cfg = small_cfg(0, tokens=T, hidden=H, n_experts=E, n_groups=1, topk_groups=1, topk=K)
    c = moe.make_config(cfg)
    out = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    t = lambda a: torch.from_numpy(a).to(DEV)
    for shared in (ys, None):
        moe.combine(c, t(yp), t(inv), t(w), None if shared is None else t(shared), T, out)
        torch.cuda.synchronize()
        ref = oracle.combine(yp, inv, w, shared)
        assert rel_err(oracle.bf16_to_f64(out), ref) <= 2.0 ** -8


# ---------------------------------------------------------------- whole layer

def _forward(cfg, inp, x=None, layer=None):
    layer = moe.Layer(cfg, inp) if layer is None else layer
    out, ids, w = layer.forward(x)
    torch.cuda.synchronize()
    return out, ids, w


# only the (config, path) pairs the library serves: no GEMM kernel for some
# format pairs, and the staged small-T path serves T <= 8
@pytest.mark.parametrize("name,path", [(n, p) for n in SMALL for p in ["auto", "gemv", "gemm", "staged"]
                                       if (p != "gemm" or pairs_ok(SMALL[n])) and (p != "staged" or SMALL[n].tokens <= 8)])
def test_forward_small(name, path, monkeypatch):
    cfg = SMALL[name]
    if path != "auto":
        monkeypatch.setenv("MOE_FORCE_PATH", path)
    inp = gpu_inputs(cfg)
    say(f"[forward] {name} {path}")
    out, ids, w = _forward(cfg, inp)
    r = oracle.forward(cfg, inp.x, inp.w_router, inp.bias, inp.routed, inp.shared)
    assert np.array_equal(ids.cpu().numpy(), r.ids)
    assert np.max(np.abs(w.cpu().numpy() - r.w) / r.w) <= WTOL
    assert rel_err(oracle.bf16_to_f64(out), r.out) <= TOL


def _check_dispatch(cfg, layer, r):
    """The forward's own dispatch arrays (read from its workspace) equal the
    oracle's, and its grouped-GEMM tile list covers every expert's segment
    exactly once in tiles of the kernel's row count."""
    T, K, E = cfg.tokens, cfg.topk, cfg.n_experts
    c = layer.cfg
    off = moe.ws_region(c, T, layer.ws, "offsets", E + 1).cpu().numpy()
    perm = moe.ws_region(c, T, layer.ws, "perm_src", T * K).cpu().numpy()
    inv = moe.ws_region(c, T, layer.ws, "inv_pos", T * K).cpu().numpy()
    assert np.array_equal(off, r.offsets)
    assert np.array_equal(perm, r.perm_src)
    assert np.array_equal(inv, r.inv_pos)
    bm = moe.ffn_tile_rows(c, 0)
    n = int(moe.ws_region(c, T, layer.ws, "ntiles", 1).cpu().numpy()[0])
    tiles = moe.ws_region(c, T, layer.ws, "tiles", 2 * n).cpu().numpy().reshape(n, 2)
    cnt = np.diff(r.offsets)
    want = []
    for e in range(E):
        n, step = _tile_split(int(cnt[e]), bm)
        want += [(e, i * step) for i in range(n)]
    want.sort()
    assert sorted(map(tuple, tiles.tolist())) == want
    # every row of every segment in exactly one tile
    for e in range(E):
        starts = sorted(m for (ee, m) in tiles.tolist() if ee == e)
        ends = starts[1:] + [int(cnt[e])]
        assert all(0 <= a < b <= int(cnt[e]) for a, b in zip(starts, ends)) and (not starts or starts[0] == 0)


def _tile_split(cnt, bm):
    """(tiles, row step) of one expert's grouped-GEMM tiles.  128-row kernel:
    ceil(cnt/bm) tiles of bm rows.  Large-tile kernel (256 main rows + one
    extra 32-row block): up to 288 rows in one tile; more rows in
    ceil(cnt/288) tiles sharing them evenly in multiples of 32, each tile
    non-empty (else 256-row steps)."""
    if cnt <= 0:
        return 0, bm
    if bm != 256:
        return -(-cnt // bm), bm
    n = -(-cnt // 288)
    if n == 1:
        return 1, 288
    h = (-(-cnt // n) + 31) // 32 * 32
    if (n - 1) * h < cnt:
        return n, h
    return -(-cnt // 256), 256


@pytest.mark.parametrize("cfgname", [c.name for c in synth.CONFIGS])
def test_forward_full_size(cfgname):
    """Full workload sizes, default path selection (the configuration the
    benchmark times): every token's ids, every output row, the dispatch
    arrays of the batched path, and three calls bitwise identical."""
    cfg = synth.get_config(cfgname)
    inp = gpu_inputs(cfg)
    say(f"[forward full] {cfgname}")
    layer = moe.Layer(cfg, inp)
    outs = []
    for _ in range(3):
        out, ids, w = layer.forward()
        torch.cuda.synchronize()
        outs.append((out.view(torch.int16).cpu().numpy().copy(), ids.cpu().numpy().copy(), w.cpu().numpy().copy()))
    moe.workspace_check(layer.ws)
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b), "repeated calls differ"
    say(f"[oracle full] {cfgname}")
    r = oracle.forward(cfg, inp.x, inp.w_router, inp.bias, inp.routed, inp.shared)
    assert np.array_equal(outs[0][1], r.ids)
    assert np.max(np.abs(outs[0][2] - r.w) / r.w) <= WTOL
    assert rel_err(oracle.bf16_to_f64(outs[0][0].view(np.uint16)), r.out) <= TOL
    if cfg.tokens > 8:   # the batched path (T <= 8 runs the single launch here)
        _check_dispatch(cfg, layer, r)


# Mid-size layers whose routed FFN runs on the large-tile kernel (MXFP8 with
# H and I multiples of 512, or bf16): about 300 rows per expert (most experts
# split over two tiles), and 256-280 rows per expert (experts that use the
# tile's extra 32-row block beside experts of at most 256 rows or experts split
# over two tiles).
MID = {
    "mx_8exp_600tok": small_cfg(3, tokens=600, hidden=1024, n_experts=8, inter=512, shared_inter=512),
    "mx_8exp_512tok": small_cfg(3, tokens=512, hidden=1024, n_experts=8, inter=512, shared_inter=512),
    "mx_8exp_560tok": small_cfg(3, tokens=560, hidden=1024, n_experts=8, inter=512, shared_inter=512),
    "bf16_8exp_512tok": small_cfg(0, tokens=512, hidden=512, n_experts=8, n_groups=1, topk_groups=1, topk=4,
                                  inter=256, shared_inter=256),
    "bf16_8exp_560tok": small_cfg(0, tokens=560, hidden=512, n_experts=8, n_groups=1, topk_groups=1, topk=4,
                                  inter=256, shared_inter=256),
}


@pytest.mark.parametrize("name", list(MID))
def test_forward_mid_size_large_tiles(name):
    cfg = MID[name]
    inp = gpu_inputs(cfg)
    layer = moe.Layer(cfg, inp)
    assert moe.ffn_tile_rows(layer.cfg, 0) == 256 and moe.ffn_tile_rows(layer.cfg, 1) == 256
    say(f"[forward mid] {name}")
    out, ids, w = _forward(cfg, inp, layer=layer)
    r = oracle.forward(cfg, inp.x, inp.w_router, inp.bias, inp.routed, inp.shared)
    cnt = np.diff(r.offsets)
    if name == "mx_8exp_600tok":
        assert (cnt > 288).sum() >= 4, cnt   # experts split over two tiles
    else:
        assert ((cnt > 256) & (cnt <= 288)).sum() >= 2, cnt   # the extra 32-row block
        assert ((cnt <= 256) | (cnt > 288)).sum() >= 1, cnt    # next to plain or split experts
    assert np.array_equal(ids.cpu().numpy(), r.ids)
    assert rel_err(oracle.bf16_to_f64(out), r.out) <= TOL
    _check_dispatch(cfg, layer, r)
    out2, _, _ = _forward(cfg, inp, layer=layer)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("rows", [2000, 1793])
def test_shared_ffn_dense_large_tiles(rows):
    """The dense bf16 large-tile GEMM (no tile list: 8 x 28 tiles of 256 rows
    in the down GEMM at H = 7168) with a ragged last row tile, fp32 output."""
    cfg = synth.get_config(3).derive(tokens=rows)
    inp = synth.make_inputs(cfg, DEV, with_experts=False)
    shared = synth.make_experts(cfg, True, DEV)
    c = moe.make_config(cfg)
    ws = moe.alloc_workspace(c, rows)
    y = torch.empty(rows, cfg.hidden, dtype=torch.float32, device=DEV)
    say(f"[shared dense] rows={rows}")
    moe.expert_ffn(c, 1, inp.x, None, rows, None, moe.weights_of(shared), y, ws)
    torch.cuda.synchronize()
    wg, wu, wd = [oracle.dequant_weight(a, None, "bf16") for a in shared.expert(0)[:3]]
    ref = oracle.expert_ffn(oracle.bf16_to_f64(inp.x), wg, wu, wd, "none")
    assert rel_err(y.cpu().numpy(), ref) <= TOL


# The DeepSeek-V2 layer at verify-sized batches, all in the single launch
# (x in LDS: 80 KB at T = 8).
@pytest.mark.parametrize("T", [2, 4, 5, 8])
def test_forward_dsv2_small_m(T):
    cfg = synth.get_config(1).derive(tokens=T)
    inp = gpu_inputs(cfg)
    say(f"[forward dsv2 small-M] T={T}")
    layer = moe.Layer(cfg, inp)
    out, ids, w = _forward(cfg, inp, layer=layer)
    moe.workspace_check(layer.ws)
    r = oracle.forward(cfg, inp.x, inp.w_router, inp.bias, inp.routed, inp.shared)
    assert np.array_equal(ids.cpu().numpy(), r.ids)
    assert np.max(np.abs(w.cpu().numpy() - r.w) / r.w) <= WTOL
    assert rel_err(oracle.bf16_to_f64(out), r.out) <= TOL
    out2, _, _ = _forward(cfg, inp, layer=layer)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("T,path", [(5, "auto"), (8, "auto"), (5, "staged"), (7, "staged"), (8, "gemv"),
                                    (12, "auto"), (21, "auto")])
def test_forward_b128_bf16x_small_t(T, path, monkeypatch):
    """FP8 block-scaled weights with bf16 activations: T <= 8 in the single
    launch (auto) or the staged launches; above that the GEMV launches
    (routed + shared gate/up in one launch, down + combine in another)."""
    cfg = small_cfg(1, tokens=T, hidden=640, n_experts=24, n_groups=4, topk_groups=2, topk=5, inter=384,
                    shared_inter=512)
    if path != "auto":
        monkeypatch.setenv("MOE_FORCE_PATH", path)
    inp = gpu_inputs(cfg)
    say(f"[forward b128 bf16-x] T={T} {path}")
    out, ids, w = _forward(cfg, inp)
    r = oracle.forward(cfg, inp.x, inp.w_router, inp.bias, inp.routed, inp.shared)
    assert np.array_equal(ids.cpu().numpy(), r.ids)
    assert np.max(np.abs(w.cpu().numpy() - r.w) / r.w) <= WTOL
    assert rel_err(oracle.bf16_to_f64(out), r.out) <= TOL


@pytest.mark.parametrize("T,hidden,forced", [(3, 640, 5), (5, 640, 3), (8, 640, 5), (8, 4608, 5), (8, 4608, 3)])
def test_single_launch_repeated_experts(T, hidden, forced):
    """From 3 tokens on, the single launch runs one routed gate/up item per
    distinct expert, for every slot that chose it.  A bias every token
    follows puts `forced` of the 5 slots on the same experts for all tokens
    (the other slots free), so a distinct expert serves up to T slots; at
    hidden 4608 the 8 tokens' x is read from global memory instead of LDS.
    Ids, weights and output match the oracle; a second call is bitwise equal."""
    cfg = small_cfg(1, tokens=T, hidden=hidden, n_experts=24, n_groups=4, topk_groups=2, topk=5, inter=384,
                    shared_inter=512)
    inp = synth.make_inputs(cfg, DEV)
    bias = torch.zeros(cfg.n_experts, device=DEV)
    chosen = [0, 1, 2, 6, 7][:forced]  # in groups 0 and 1 (6 experts per group)
    bias[chosen] = 30.0
    inp.bias = bias
    inp = ensure_margin(inp)
    say(f"[repeated experts] T={T} H={hidden} forced={forced}")
    layer = moe.Layer(cfg, inp)
    out, ids, w = _forward(cfg, inp, layer=layer)
    moe.workspace_check(layer.ws)
    ids_np = ids.cpu().numpy()
    for e in chosen:
        assert (ids_np == e).any(axis=1).all()  # every token holds every forced expert
    r = oracle.forward(cfg, inp.x, inp.w_router, inp.bias, inp.routed, inp.shared)
    assert np.array_equal(ids_np, r.ids)
    assert np.max(np.abs(w.cpu().numpy() - r.w) / r.w) <= WTOL
    assert rel_err(oracle.bf16_to_f64(out), r.out) <= TOL
    out2, _, _ = _forward(cfg, inp, layer=layer)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("name,path", [("dsv2_like_4tok", "auto"), ("dsv2_like_4tok", "staged"),
                                       ("b128_12exp_97tok", "auto"), ("zipf_16exp_200tok", "auto"),
                                       ("tiny_8tok", "auto"), ("mx_4exp_160tok", "auto")])
def test_forward_degenerate_routing(name, path, monkeypatch):
    """A masking bias leaves fewer finite logits than slots (-inf experts fill
    the rest, lowest id first, weight 0), and token 0 holds a NaN (no defined
    softmax: the lowest ids, NaN weights, a NaN output row).  Every id stays
    in range, so no kernel reads outside the weights; the other rows match."""
    cfg = SMALL[name]
    if path != "auto":
        monkeypatch.setenv("MOE_FORCE_PATH", path)
    inp = synth.make_inputs(cfg, DEV)
    gsz = cfg.n_experts // cfg.n_groups
    bias = torch.full((cfg.n_experts,), float("-inf"), device=DEV)
    bias[::gsz] = 0.0                       # one finite expert per group
    inp.bias = bias
    inp = ensure_margin(inp)
    inp.x[0, 5] = float("nan")
    say(f"[degenerate] {name} {path}")
    layer = moe.Layer(cfg, inp)
    out, ids, w = _forward(cfg, inp, layer=layer)
    moe.workspace_check(layer.ws)
    r = oracle.forward(cfg, inp.x, inp.w_router, inp.bias, inp.routed, inp.shared)
    ids, w = ids.cpu().numpy(), w.cpu().numpy()
    assert np.array_equal(ids, r.ids)
    assert list(ids[0]) == list(range(cfg.topk))   # lowest ids of the lowest groups (groups >= slots here)
    assert np.isnan(w[0]).all() and np.isnan(r.w[0]).all()
    assert (w[1:, cfg.topk_groups:] == 0).all()
    o = oracle.bf16_to_f64(out)
    assert np.isnan(o[0]).all()
    assert rel_err(o[1:], r.out[1:]) <= TOL


def test_single_launch_epoch_wrap():
    """The launch tag comes from an epoch word advanced modulo 0xffffffff, so
    consecutive launches never share a tag, also across the wrap: from epoch
    0xfffffffe, three calls with the tokens rotated must each route their own
    tokens (a repeated tag would hand the previous call's logits over)."""
    cfg = SMALL["dsv2_like_4tok"]
    inp = gpu_inputs(cfg)
    r = oracle.forward(cfg, inp.x, inp.w_router, inp.bias, inp.routed, inp.shared)
    layer = moe.Layer(cfg, inp)
    layer.ws[4:8].view(torch.int32).fill_(-2)    # epoch word = 0xfffffffe
    for k, want_epoch in enumerate((0, 1, 2)):
        order = [(k + i) % 4 for i in range(4)]
        out, ids, w = _forward(cfg, inp, inp.x[order].contiguous(), layer=layer)
        assert np.array_equal(ids.cpu().numpy(), r.ids[order])
        assert rel_err(oracle.bf16_to_f64(out), r.out[order]) <= TOL
        q = _queue_words(layer)
        assert q[0] == 0 and q[1] == want_epoch


def test_forward_is_bitwise_deterministic():
    cfg = SMALL["zipf_16exp_200tok"]
    inp = gpu_inputs(cfg)
    layer = moe.Layer(cfg, inp)
    outs = []
    for _ in range(3):
        out, ids, w = layer.forward()
        torch.cuda.synchronize()
        outs.append((out.view(torch.int16).cpu().numpy().copy(), ids.cpu().numpy().copy(), w.cpu().numpy().copy()))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)


def test_forward_zero_tokens_is_noop():
    cfg = SMALL["tiny_8tok"]
    inp = synth.make_inputs(cfg, DEV)
    layer = moe.Layer(cfg, inp)
    out = torch.full((0, cfg.hidden), 7, dtype=torch.bfloat16, device=DEV)
    layer.forward(inp.x[:0], out=out, ids=torch.empty(0, cfg.topk, dtype=torch.int32, device=DEV),
                  w=torch.empty(0, cfg.topk, dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()


def _queue_words(layer):
    """Error word, epoch word and counter lines of the single-launch path (the
    tagged router logits follow them in the first 32 KiB)."""
    return layer.ws[:24576].view(torch.int32).cpu().numpy()


def test_single_launch_queue_across_calls():
    """The single-launch small-T path over many calls on one workspace, with
    T changing between 1 and 8 and two layers interleaved on one stream:
    every output matches the oracle and the queue state is zero after each
    call (no bounded wait gave up, every counter reset) but for the epoch
    word, which each call advances by one."""
    layers = []
    for name in ("dsv2_like_4tok", "bf16_1tok"):
        cfg = SMALL[name].derive(tokens=8)
        inp = gpu_inputs(cfg)
        r = oracle.forward(cfg, inp.x, inp.w_router, inp.bias, inp.routed, inp.shared)
        layers.append((name, moe.Layer(cfg, inp), inp, r))
    for it in range(12):
        for name, layer, inp, r in layers:
            T = 1 + (it * 3 + len(name)) % 8
            say(f"[single-launch] {name} call {it} T={T}")
            out, ids, w = layer.forward(inp.x[:T].contiguous())
            torch.cuda.synchronize()
            assert np.array_equal(ids.cpu().numpy(), r.ids[:T])
            assert np.max(np.abs(w.cpu().numpy() - r.w[:T]) / r.w[:T]) <= WTOL
            assert rel_err(oracle.bf16_to_f64(out), r.out[:T]) <= TOL
            q = _queue_words(layer)
            assert q[0] == 0 and q[1] == it + 1
            q[1] = 0
            assert not q.any()


def test_forward_reuses_workspace_across_sizes():
    """One workspace, calls with decreasing T (the route counter is left at 0)."""
    cfg = SMALL["b128_12exp_97tok"]
    inp = gpu_inputs(cfg)
    layer = moe.Layer(cfg, inp)
    r = oracle.forward(cfg, inp.x, inp.w_router, inp.bias, inp.routed, inp.shared)
    for T in (97, 40, 3, 1, 2, 97):
        out, ids, _ = layer.forward(inp.x[:T].contiguous())
        torch.cuda.synchronize()
        assert np.array_equal(ids.cpu().numpy(), r.ids[:T])
        # the per-token output does not depend on the other tokens
        assert rel_err(oracle.bf16_to_f64(out), r.out[:T]) <= TOL
