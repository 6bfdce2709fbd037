"""Benchmark of one MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline workload: the DeepSeek-V2 MoE layer at B=1 (hidden 5120, 160 routed
experts in 8 groups of 20, top-3 groups, top-6 experts, route scale 16,
intermediate 1536, shared experts fused to 3072, FP8 e4m3 weights with fp32
per-128x128 block scales).  One step is one full layer forward (router,
top-k, routed + shared FFNs, combine) on one token.  Steps cycle through 24
replicas of the layer's inputs and weights (about 4.5 GB touched per cycle),
so the 256 MB Infinity Cache cannot hold the working set and the weights
stream from HBM, as they would across the layers of a model.

Secondary: the 2,048-token layer (hidden 7168, 32 experts, top-4 flat
routing, intermediate 2048, MXFP8 routed experts, bf16 shared expert), as
effective TFLOP/s.

Prints one JSON line.  Inputs are resident in HBM before the timed region.
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer µs @B=1 (HBM GB/s, %peak); TFLOP/s @2048 tok (%FP8 MFMA peak)"
HBM_PEAK_GBPS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=24)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-secondary", action="store_true", help="skip the 2048-token workload")
    ap.add_argument("--no-small-m", action="store_true", help="skip the 2-8 token DeepSeek-V2 layers")
    ap.add_argument("--no-batched", action="store_true", help="skip the 256- and 4096-token DeepSeek-V2 layers")
    ap.add_argument("--no-backward", action="store_true", help="skip the bf16 backward of the 2048-token layer")
    ap.add_argument("--backward-only", action="store_true", help="only run the backward (for profiling its kernels)")
    ap.add_argument("--secondary-steps", type=int, default=20)
    ap.add_argument("--secondary-only", action="store_true",
                    help="only run the 2048-token workload (for profiling its kernels)")
    ap.add_argument("--batched-only", metavar="NAME", choices=("dsv2_256tok", "dsv2_4096tok_zipf"),
                    help="only run one batched workload (for profiling its kernels)")
    ap.add_argument("--sources-hash", metavar="KERNEL", help="print the sources hash recorded with KERNEL's counters")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (a known-size reference for HBM counters)")
    return ap.parse_args()


def wbytes(ew, experts):
    """Bytes of weights + scales of the listed experts of an ExpertWeights set."""
    tot = 0
    for t in (ew.gate, ew.up, ew.down, ew.gate_s, ew.up_s, ew.down_s):
        if t is not None:
            tot += t[0].numel() * t.element_size() * len(experts)
    return tot


def gate_up_bytes(ew, experts):
    tot = 0
    for t in (ew.gate, ew.up, ew.gate_s, ew.up_s):
        if t is not None:
            tot += t[0].numel() * t.element_size() * len(experts)
    return tot


class HostExperts:
    """Host copies of a few experts, shaped like the generator's weight sets."""

    def __init__(self, ew, experts):
        self.fmt = ew.fmt
        self.data = {int(e): ew.expert(int(e)) for e in experts}

    def expert(self, e):
        return self.data[int(e)]


def time_layers(layers, xs, steps, warmup, torch):
    """Mean ms per step over `steps` back-to-back steps (events on the launch
    stream around the loop), and the wall-clock ms per step."""
    n = len(layers)
    for i in range(warmup):
        layers[i % n].forward(xs[i % n])
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        layers[i % n].forward(xs[i % n])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(stop) / steps, wall / steps * 1e3


def block_stats(layers, xs, blocks, per_block, torch):
    """Median, p10 and p90 (us per step) over `blocks` runs of `per_block`
    back-to-back steps, each run between its own two events (the median over
    runs of "Benchmarking Honestly"; runs of several steps keep the events'
    own gaps out of the per-step figure)."""
    n = len(layers)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * blocks)]
    i = 0
    for b in range(blocks):
        ev[2 * b].record()
        for _ in range(per_block):
            layers[i % n].forward(xs[i % n])
            i += 1
        ev[2 * b + 1].record()
    torch.cuda.synchronize()
    us = sorted(ev[2 * b].elapsed_time(ev[2 * b + 1]) * 1e3 / per_block for b in range(blocks))
    q = lambda f: us[min(len(us) - 1, int(round(f * (len(us) - 1))))]
    return {"median": round(statistics.median(us), 3), "p10": round(q(0.1), 3), "p90": round(q(0.9), 3),
            "runs": blocks, "steps_per_run": per_block}


def check_workspaces(layers, moe):
    """Every single-launch call's bounded waits completed (raises otherwise)."""
    for lay in layers:
        moe.workspace_check(lay.ws)


def trace_kernels(layers, xs, steps, moe, torch):
    n = len(layers)
    per = {}
    with moe.LaunchTrace(64 * steps) as tr:
        for i in range(steps):
            layers[i % n].forward(xs[i % n])
    for name, ms in tr.kernels():
        per.setdefault(name, []).append(ms)
    return {k: (statistics.mean(v), len(v) // steps) for k, v in per.items()}


def main():
    args = parse()
    if args.sources_hash:
        print(csrc_hash(args.sources_hash))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import numpy as np
    import mixture_experts_layer_router_amd as moe
    import synth

    dev = "cuda:0"
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel(), "copies": 5}))
        return
    if args.secondary_only:
        print(json.dumps({"secondary": secondary(args, moe, synth, torch)}), flush=True)
        return
    if args.backward_only:
        print(json.dumps({"backward": backward(moe, synth, torch)}), flush=True)
        return
    if args.batched_only:
        print(json.dumps({"batched": batched(moe, synth, torch, names=(args.batched_only,))}), flush=True)
        return
    cfg = synth.get_config("dsv2_b1")
    reps = [synth.make_inputs(cfg, dev, replica=r) for r in range(args.replicas)]
    layers = [moe.Layer(cfg, inp) for inp in reps]
    xs = [inp.x for inp in reps]
    torch.cuda.synchronize()

    ms_step, wall_ms = time_layers(layers, xs, args.steps, args.warmup, torch)
    us = ms_step * 1e3
    stats = block_stats(layers, xs, 20, 10, torch)
    check_workspaces(layers, moe)

    # algorithmic bytes per step, from each replica's actual routing
    step_bytes, gu_bytes = [], []
    for lay, inp in zip(layers, reps):
        _, ids, _ = lay.forward()
        torch.cuda.synchronize()
        touched = sorted(set(ids.flatten().tolist()))
        io = inp.x.numel() * 2 * 2
        router = inp.w_router.numel() * 2
        step_bytes.append(wbytes(inp.routed, touched) + wbytes(inp.shared, [0]) + router + io)
        gu_bytes.append(gate_up_bytes(inp.routed, touched) + inp.x.numel() * 2)  # routed gate/up launch
    bytes_step = statistics.mean(step_bytes)
    gbps = bytes_step / (us * 1e-6) / 1e9

    kern = trace_kernels(layers, xs, min(args.steps, 100), moe, torch)
    if list(kern) == ["decode_fused"]:
        # the whole layer is one launch: its bytes are the step's, and the
        # timed loop (back-to-back launches, events around the loop on the
        # launch stream) gives its average duration without per-launch events
        dom, dom_bytes, dom_us = "decode_fused", bytes_step, us
    else:  # staged launches: the routed gate/up is the largest single stream (94 MB)
        dom, dom_bytes = "gemv_gate_up", statistics.mean(gu_bytes)
        dom_us = kern[dom][0] * 1e3
    dom_gbps = dom_bytes / (dom_us * 1e-6) / 1e9
    traffic = measured_traffic(dom)

    out = {
        "metric": METRIC,
        "value": round(us, 3),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3-weights/bf16-x/fp32",
        "data": "synthetic",
        "config": {
            "workload": "DeepSeek-V2 MoE layer, B=1 decode: H=5120, 160 experts (8 groups x 20, top-3 groups, top-6), "
                        "route scale 16, I=1536, fused shared 3072, FP8 e4m3 + fp32 128x128 block scales",
            "tokens": 1,
            "replicas": args.replicas,
        },
        "tokens_per_s": round(1e6 / us, 1),
        "hbm_GBps": round(gbps, 1),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": int(bytes_step),
        "wall_ms_per_step": round(wall_ms, 6),
        "step_us_stats": stats,
        "kernels_us": {k: round(v[0] * 1e3, 3) for k, v in kern.items()},
        "roofline": {
            "kernel": dom,
            "bound": "hbm",
            "achieved": round(dom_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "bytes_per_launch": int(dom_bytes),
            "launch_us": round(dom_us, 3),
        },
    }

    out["tiny"] = tiny(moe, synth, torch)
    if not args.no_secondary:
        out["secondary"] = secondary(args, moe, synth, torch)
    if not args.no_small_m:
        out["small_m"] = small_m(moe, synth, torch)
    if not args.no_batched:
        out["batched"] = batched(moe, synth, torch)
    if not args.no_backward:
        out["backward"] = backward(moe, synth, torch)

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(cfg, reps[0], layers[0], torch)

    print(json.dumps(out), flush=True)


# sources each measured kernel is built from: its counter summary stays valid
# while these files are unchanged
KERNEL_SOURCES = {
    "decode_fused": ("decode.hip", "gemv_dev.h", "route_dev.h", "common.h", "kernels.h"),
    "gemm_gate_up_routed": ("gemm.hip", "gemm2.hip", "gemm_dev.h", "common.h", "kernels.h"),
    "gemm_down_routed": ("gemm.hip", "gemm2.hip", "gemm_dev.h", "common.h", "kernels.h"),
}


def csrc_hash(kernel):
    import hashlib
    csrc = os.path.join(ROOT, "mixture_experts_layer_router_amd", "csrc")
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, sorted(os.listdir(csrc))):
        h.update(f.encode())
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload="dsv2_b1"):
    """HBM bytes per launch from the committed counter summary of `kernel` on
    `workload`, or None when the kernel sources changed since the counters
    were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("sources sha256 at measurement") != csrc_hash(kernel) or "traffic_bytes" not in fields:
        return None
    return int(fields["traffic_bytes"])


def gemm_roofline(workload, kern, rows, H, I, kernel):
    """Roofline of a grouped FFN GEMM launch: flops over the real rows
    (gate/up: 2 * rows * 2I * H; down: 2 * rows * H * I) over the launch's
    average duration (events on the launch stream), against the dense FP8
    matrix peak; traffic from the committed counter summary, if current."""
    flops = 2.0 * rows * (2 * I if "gate_up" in kernel else I) * H
    us = kern[kernel][0] * 1e3
    achieved = flops / (us * 1e-6) / 1e12
    return {"kernel": kernel, "bound": "mfma", "achieved": round(achieved, 1), "peak": FP8_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / FP8_PEAK_TFLOPS, 4),
            "traffic": measured_traffic(kernel, workload), "flops_per_launch": flops, "launch_us": round(us, 2)}


def batched(moe, synth, torch, steps=20, names=("dsv2_256tok", "dsv2_4096tok_zipf")):
    """The DeepSeek-V2 FP8 layer at 256 tokens (near-uniform routing) and at
    4,096 tokens (Zipf-skewed routing): us/layer, the HBM rate of the bytes
    the routing touches (weights of the touched experts, shared expert,
    router, x and out) and the matrix rate of the flops over real rows.
    Both working sets exceed the 256 MB memory-side cache."""
    import numpy as np
    res = []
    for name in names:
        cfg = synth.get_config(name)
        inp = synth.make_inputs(cfg, "cuda:0")
        lay = moe.Layer(cfg, inp)
        ms, _ = time_layers([lay], [inp.x], steps, 3, torch)
        stats = block_stats([lay], [inp.x], 10, 2, torch)
        _, ids, _ = lay.forward()
        torch.cuda.synchronize()
        touched = sorted(set(ids.flatten().tolist()))
        T, H, K, I, Is, E = cfg.tokens, cfg.hidden, cfg.topk, cfg.inter, cfg.shared_inter, cfg.n_experts
        nbytes = (wbytes(inp.routed, touched) + wbytes(inp.shared, [0]) + inp.w_router.numel() * 2 +
                  inp.x.numel() * 2 * 2)
        flops = 2.0 * T * K * 3 * H * I + 2.0 * T * 3 * H * Is + 2.0 * T * H * E
        kern = trace_kernels([lay], [inp.x], 3, moe, torch)
        cnt = np.bincount(ids.flatten().cpu().numpy(), minlength=E)
        res.append({"workload": name, "tokens": T, "us_per_layer": round(ms * 1e3, 2), "step_us_stats": stats,
                    "max_mean_load": round(float(cnt.max() / cnt.mean()), 2), "empty_experts": int((cnt == 0).sum()),
                    "roofline": gemm_roofline(name, kern, T * K, H, I, "gemm_gate_up_routed"),
                    "touched_experts": len(touched), "algorithmic_bytes": int(nbytes),
                    "hbm_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                    "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                    "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                    "frac_fp8_peak": round(flops / (ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
                    "kernels_us": {k: round(v[0] * 1e3, 2) for k, v in kern.items()}})
        del lay, inp
        torch.cuda.empty_cache()
    return res


def small_m(moe, synth, torch, tokens=(2, 4, 8), replicas=8):
    """The DeepSeek-V2 layer at a few tokens (verify-sized batches): us/layer
    and the HBM rate of the bytes the routing touches, 8 replicas cycled."""
    base = synth.get_config("dsv2_b1")
    res = []
    for T in tokens:
        cfg = base.derive(tokens=T)
        reps = [synth.make_inputs(cfg, "cuda:0", replica=r) for r in range(replicas)]
        layers = [moe.Layer(cfg, inp) for inp in reps]
        ms, _ = time_layers(layers, [inp.x for inp in reps], 100, 10, torch)
        check_workspaces(layers, moe)
        nbytes = []
        for lay, inp in zip(layers, reps):
            _, ids, _ = lay.forward()
            torch.cuda.synchronize()
            touched = sorted(set(ids.flatten().tolist()))
            nbytes.append(wbytes(inp.routed, touched) + wbytes(inp.shared, [0]) + inp.w_router.numel() * 2 +
                          inp.x.numel() * 2 * 2)
        b = statistics.mean(nbytes)
        res.append({"tokens": T, "us_per_layer": round(ms * 1e3, 2), "algorithmic_bytes": int(b),
                    "hbm_GBps": round(b / (ms * 1e-3) / 1e9, 1),
                    "path": "single launch" if T <= 8 else "GEMV launches"})
        del layers, reps
        torch.cuda.empty_cache()
    return res


def tiny(moe, synth, torch, replicas=8):
    """The tiny 8-token bf16 layer (hidden 256, 16 experts): launch-latency
    bound; us per layer over 8 replicas cycled."""
    cfg = synth.get_config("tiny_8tok")
    reps = [synth.make_inputs(cfg, "cuda:0", replica=r) for r in range(replicas)]
    layers = [moe.Layer(cfg, inp) for inp in reps]
    ms, _ = time_layers(layers, [inp.x for inp in reps], 200, 20, torch)
    return {"workload": "tiny_8tok: 8 tokens, H=256, 16 experts (4 groups, top-2 groups, top-4), I=128, bf16",
            "us_per_layer": round(ms * 1e3, 2), "step_us_stats": block_stats(layers, [inp.x for inp in reps], 20, 10,
                                                                              torch),
            "kernels_us": {k: round(v[0] * 1e3, 2) for k, v in trace_kernels(layers, [i.x for i in reps], 8, moe,
                                                                               torch).items()}}


def secondary(args, moe, synth, torch):
    cfg = synth.get_config("h7168_2048tok_mx")
    inp = synth.make_inputs(cfg, "cuda:0")
    lay = moe.Layer(cfg, inp)
    ms, _ = time_layers([lay], [inp.x], args.secondary_steps, 3, torch)
    T, H, K, I, Is, E = cfg.tokens, cfg.hidden, cfg.topk, cfg.inter, cfg.shared_inter, cfg.n_experts
    flops = 2.0 * T * K * 3 * H * I + 2.0 * T * 3 * H * Is + 2.0 * T * H * E
    tflops = flops / (ms * 1e-3) / 1e12
    kern = trace_kernels([lay], [inp.x], 5, moe, torch)
    stats = block_stats([lay], [inp.x], 10, 5, torch)
    del lay, inp
    torch.cuda.empty_cache()
    return {
        "workload": "2,048 tokens, H=7168, 32 experts flat top-4, I=2048, MXFP8 routed (e8m0 1x32) + bf16 shared 2048",
        "us_per_layer": round(ms * 1e3, 2),
        "step_us_stats": stats,
        "roofline": gemm_roofline("h7168_2048tok_mx", kern, T * K, H, I, "gemm_gate_up_routed"),
        "tflops": round(tflops, 1),
        "frac_fp8_peak": round(tflops / FP8_PEAK_TFLOPS, 4),
        "flops_per_layer": flops,
        "kernels_us": {k: round(v[0] * 1e3, 2) for k, v in kern.items()},
    }


def backward_config(synth):
    """The 2,048-token H=7168 layer with bf16 weights and unquantised
    activations: the shape the backward is measured on."""
    return synth.get_config("h7168_2048tok_mx").derive(name="h7168_2048tok_bf16", routed_wfmt="bf16",
                                                        shared_wfmt="bf16", routed_afmt="none", shared_afmt="none")


def backward(moe, synth, torch, steps=5):
    """The layer's backward (Mixture-of-Kittens, Table 1) on the 2,048-token
    H=7168 layer in bf16: us per call, and the matrix rate of the flops it
    executes (routed: the recomputed gate/up/down and six backward GEMM
    passes, 9 x 2 TK H I; shared: the recomputed gate/up and six passes,
    8 x 2 T H Is; router: logits, dWr and dl Wr, 3 x 2 T E H) against the
    dense bf16 matrix peak."""
    cfg = backward_config(synth)
    inp = synth.make_inputs(cfg, "cuda:0")
    T, H, K, I, Is, E = cfg.tokens, cfg.hidden, cfg.topk, cfg.inter, cfg.shared_inter, cfg.n_experts
    c = moe.make_config(cfg)
    g = torch.Generator(device="cuda:0")
    g.manual_seed(synth.generate.seed_of(cfg.index, 0, 11, T))
    dy = torch.randn(T, H, generator=g, device="cuda:0").to(torch.bfloat16)
    ws = torch.empty(moe.backward_workspace_size(c, T), dtype=torch.uint8, device="cuda:0")
    bf = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device="cuda:0")
    dx, dr, db = bf(T, H), bf(E, H), torch.empty(E, dtype=torch.float32, device="cuda:0")
    rg = moe.make_grads(bf(E, I, H), bf(E, I, H), bf(E, H, I))
    sg = moe.make_grads(bf(1, Is, H), bf(1, Is, H), bf(1, H, Is))
    rw, sw = moe.weights_of(inp.routed), moe.weights_of(inp.shared)
    call = lambda: moe.backward(c, inp.x, inp.w_router, inp.bias, rw, sw, dy, dx, dr, db, rg, sg, ws)
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    for i in range(steps):
        ev[2 * i].record()
        call()
        ev[2 * i + 1].record()
    torch.cuda.synchronize()
    us = sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e3 for i in range(steps))
    with moe.LaunchTrace(256) as tr:
        call()
    kern = {}
    for name, ms in tr.kernels():
        kern[name] = round(kern.get(name, 0.0) + ms * 1e3, 2)
    flops = 2.0 * T * K * H * I * 9 + 2.0 * T * H * Is * 8 + 2.0 * T * E * H * 3
    med = statistics.median(us)
    del inp, ws, dy, dx, dr, db, rg, sg
    torch.cuda.empty_cache()
    return {"workload": "h7168_2048tok_bf16: 2,048 tokens, H=7168, 32 experts flat top-4, I=2048, bf16 routed + "
                        "bf16 shared 2048, unquantised activations",
            "us_per_call": {"median": round(med, 1), "min": round(us[0], 1), "max": round(us[-1], 1),
                            "calls": steps},
            "flops_per_call": flops, "tflops": round(flops / (med * 1e-6) / 1e12, 1),
            "frac_bf16_peak": round(flops / (med * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "kernels_us": kern}


def cpu_baseline(cfg, inp, lay, torch):
    """The fp64 oracle on the host cores, on the same B=1 layer (replica 0)."""
    import oracle
    from threadpoolctl import threadpool_limits
    _, ids, _ = lay.forward()
    torch.cuda.synchronize()
    touched = sorted(set(ids.flatten().tolist()))
    routed = HostExperts(inp.routed, touched)
    shared = HostExperts(inp.shared, [0])
    x, wr = inp.x.cpu(), inp.w_router.cpu()
    cores = len(os.sched_getaffinity(0))
    times = []
    with threadpool_limits(limits=cores):
        deadline = time.perf_counter() + 20.0
        while len(times) < 3 and (not times or time.perf_counter() < deadline):
            t0 = time.perf_counter()
            oracle.forward(cfg, x, wr, None, routed, shared)
            times.append(time.perf_counter() - t0)
    s = statistics.median(times)
    return {"value": round(s * 1e6, 1), "unit": "us/layer", "cores": cores, "kind": "oracle",
            "sample": f"the whole B=1 layer forward (replica 0: router, top-k, the 6 routed and the shared "
                      f"expert, combine), median of {len(times)} runs, float64 numpy with BLAS on {cores} threads"}


if __name__ == "__main__":
    main()
