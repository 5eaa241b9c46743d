#!/usr/bin/env python3
"""Benchmark of the multi-LoRA hot path on one MI355X.

A step is one pass of the whole path over one batch: the segment build, then
for every LoRA layer of the workload its shrink and (where timed) its expand.
By default each layer with a timed expand is one shrink_expand call, and the
first one is given the batch's idx so that it builds the segment record
itself (inside its single launch for 16-bit batches of at most 4096 tokens
and 256 slots); the later layers read that record.  --separate-build runs
lora_build_segments first instead.  The segment build is timed on its own as
the `segments` call either way.
Inputs are resident in HBM before timing starts.  Steps rotate over several
device copies of the inputs, enough that the working set exceeds the 256 MB
last-level cache, so the byte rates below are HBM rates, not cache rates.
Steps are replayed from a captured HIP graph, as a serving engine replays its
decode step; the eager (host-launched) time is reported alongside.

Prints ONE JSON line on stdout.  `value` is tokens per second (batch tokens T
per step).  `roofline` is for the call that takes the most GPU time per step:
its algorithmic bytes (active rows, distinct slots at their real ranks, the
fp32 intermediate's write and read) divided by its average duration, measured
here with HIP events around graph replays of that call alone.  `cpu_baseline`
is the fp64 oracle timed on a bounded sample of the same workload on the
host cores.  For an all-base batch (zipf_many_noop) a `noop` object times the
layer's base projection with and without the (no-op) LoRA call.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "shrink+expand tokens/s and achieved HBM GB/s (% roofline), Llama-8B shapes"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, public datasheet
MFMA_PEAK_TFLOPS_16 = 2500.0   # dense fp16/bf16 MFMA
MALL_BYTES = 256 << 20
DEFAULT_WORKLOAD = "decode_qproj"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1280)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--mode", default="auto", choices=["auto", "bgmv", "sgmv"])
    ap.add_argument("--separate-build", action="store_true",
                    help="build the segment record with lora_build_segments before the first layer "
                         "instead of inside the first layer's shrink_expand call")
    ap.add_argument("--eager", action="store_true", help="time host launches instead of graph replay")
    ap.add_argument("--path", default="fused", choices=["fused", "split"],
                    help="fused: each layer with a timed expand is one shrink_expand call (one "
                         "launch for 16-bit batches up to lora_fused_max_tokens(), else two); "
                         "split: a shrink call then an expand call")
    ap.add_argument("--no-calls", action="store_true",
                    help="skip the per-call timing (counter runs: kernels then run in step order only)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of the oracle's CPU timing (0 disables it)")
    ap.add_argument("--json-out", default=None, help="also append the JSON line to this file")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="run one device-to-device copy of this many MiB before timing, as the "
                         "known-size reference kernel for FETCH_SIZE/WRITE_SIZE counter runs")
    return ap.parse_args()


# --------------------------------------------------------------------------
# measured HBM traffic, from a committed counter summary of these very sources
# --------------------------------------------------------------------------

def kernel_source_hash():
    """Short hash of the HIP sources; a traffic figure is only valid for it."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gemm_lora_shrink_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, call):
    """Bytes per launch of `call` from profiles/traffic.md, or None.

    A row reads: | workload | call | kernel | source hash | fetch KiB | write KiB |
    fetch factor | write factor | bytes per launch |.  It is used only when its
    source hash equals the hash of the sources being benchmarked.
    """
    path = os.path.join(ROOT, "profiles", "traffic.md")
    if not os.path.exists(path):
        return None
    want = kernel_source_hash()
    for line in open(path):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 9 and cells[0] == workload and cells[1] == call and cells[3] == want:
            try:
                return float(cells[8])
            except ValueError:
                return None
    return None


# --------------------------------------------------------------------------
# algorithmic work (active rows, distinct slots at their real ranks)
# --------------------------------------------------------------------------

def algorithmic(p):
    import numpy as np
    e = p.elem_bytes
    valid = (p.idx >= 0) & (p.idx < p.S)
    n_active = int(valid.sum())
    slots = np.unique(p.idx[valid])
    rk = (lambda s: p.r_max) if p.ranks is None else (lambda s: int(p.ranks[s]))
    sum_r_distinct = sum(rk(s) for s in slots)
    sum_r_active = sum(rk(int(s)) for s in p.idx[valid])
    n_sl = p.n_slices
    out = sum(p.out_sizes)
    shrink_b = n_active * p.D * e + n_sl * p.D * e * sum_r_distinct + 4 * n_sl * sum_r_active
    expand_b = 2 * e * out * n_active + e * out * sum_r_distinct + 4 * n_sl * sum_r_active
    shrink_f = 2 * n_sl * p.D * sum_r_active
    expand_f = 2 * out * sum_r_active
    return dict(n_active=n_active, n_distinct=len(slots), shrink_bytes=shrink_b,
                expand_bytes=expand_b, shrink_flops=shrink_f, expand_flops=expand_f)


def segment_bytes(T, n_active):
    return 4 * T + 4 * n_active


# --------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample
# --------------------------------------------------------------------------

def cpu_baseline(wl, seconds):
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle

    rng = np.random.default_rng(0)
    T = wl.T
    # a sample of tokens, the same for every layer of the workload
    n = min(T, 64)
    tokens = np.sort(rng.choice(T, size=n, replace=False))
    done_tokens = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while True:
            for p in wl.problems:
                v = oracle.oracle_shrink(p.x, p.A, p.idx, p.S, dtype=p.dtype, D=p.D,
                                         scale=p.scale, ranks=p.ranks, tokens=tokens)
                if p.timed_expand:
                    oracle.oracle_expand(v, p.B, p.y_in, p.idx, p.S, p.out_offsets,
                                         dtype=p.dtype, ranks=p.ranks, tokens=tokens)
            done_tokens += n
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return dict(value=done_tokens / el, unit="tokens/s", cores=1, kind="oracle",
                sample=f"{n} of the {T} batch tokens (every layer of the step, shrink and "
                       f"timed expand), repeated for {el:.1f} s on 1 host thread "
                       f"(BLAS limited to 1 thread); host has {len(os.sched_getaffinity(0))} "
                       f"usable cores")


# --------------------------------------------------------------------------
# GPU side
# --------------------------------------------------------------------------

def noop_overhead(torch, glsa, st, p, S, capture, reps=20, iters=50):
    """The cost of the LoRA path on an all-base batch, next to the base layer.

    The base layer is the layer's own dense projection, y = x W^T (a
    T x D by D x out fp16 GEMM, as the q_proj of Llama-3-8B at T = 4096).  With
    LoRA enabled and no adapter active the caller passes active = False (the
    host knows the batch holds no adapter) and shrink_expand enqueues nothing.
    Both loops are timed in graph replay and eager, `iters` layers per timing,
    median of `reps`; overhead = with_lora / base - 1.
    """
    import statistics
    d = st["layers"][0]
    x = d["x"]
    W = torch.randn((sum(p.out_sizes), p.D), device=x.device, dtype=x.dtype) * 0.01
    out = torch.empty((x.size(0), W.size(0)), device=x.device, dtype=x.dtype)

    def base():
        torch.matmul(x, W.t(), out=out)

    def with_lora():
        torch.matmul(x, W.t(), out=out)
        glsa.shrink_expand(d["x"], d["A"], d["B"], d["y"], st["seg"], p.out_offsets,
                           workspace=d["ws"], scale=d["scale"], ranks=d["ranks"], v=d["v"],
                           active=False)

    def timed(fn_iter):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        vals = []
        for _ in range(reps):
            torch.cuda.synchronize()
            e0.record()
            fn_iter()
            e1.record()
            torch.cuda.synchronize()
            vals.append(e0.elapsed_time(e1) * 1e3 / iters)
        return statistics.median(vals)

    res = {}
    for mode in ("graph", "eager"):
        t = {}
        for name, fn in (("base", base), ("with_lora", with_lora)):
            if mode == "graph":
                g = capture([fn] * iters)
                t[name] = timed(g.replay)
            else:
                t[name] = timed(lambda fn=fn: [fn() for _ in range(iters)])
        res[mode] = dict(base_us=round(t["base"], 3), with_lora_us=round(t["with_lora"], 3),
                         overhead=round(t["with_lora"] / t["base"] - 1.0, 5))
    res["base_layer"] = f"fp16 GEMM [{x.size(0)} x {p.D}] x [{p.D} x {W.size(0)}] (torch.matmul)"
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(no collectives or sharding); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gemm_lora_shrink_amd as glsa
    from workloads import CONFIGS, make_workload
    from workloads.torch_io import problem_to_device

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    wl = make_workload(args.workload)
    cfg = CONFIGS[args.workload]
    T, S = wl.T, wl.S
    problems = wl.problems

    # one host draw, uploaded once, then cloned on the device into enough sets
    # to exceed the last-level cache
    base = [problem_to_device(p, dev) for p in problems]

    def nbytes(d):
        tot = d["x"].numel() * d["x"].element_size() + d["y"].numel() * d["y"].element_size()
        tot += sum(a.numel() * a.element_size() for a in d["A"])
        tot += sum(b.numel() * b.element_size() for b in d["B"])
        return tot
    set_bytes = sum(nbytes(d) for d in base)
    n_sets = max(2, min(64, math.ceil(2 * MALL_BYTES / set_bytes)))
    # the graph holds `chunk` steps; chunk divides K exactly
    chunk = max(d for d in range(1, min(args.steps, n_sets) + 1) if args.steps % d == 0)
    n_sets = chunk if chunk >= 2 else n_sets

    sets = []
    for i in range(n_sets):
        layers = []
        for p, d in zip(problems, base):
            c = {k: (v.clone() if torch.is_tensor(v) else [t.clone() for t in v] if isinstance(v, list) else v)
                 for k, v in d.items()}
            c["v"] = torch.empty((p.n_slices, T, p.r_max), dtype=torch.float32, device=dev)
            c["ws"] = glsa.alloc_workspace(T, S, p.n_slices, p.r_max, dev)
            layers.append(c)
        seg = glsa.alloc_segments(T, S, dev)
        sets.append(dict(idx=layers[0]["idx"], seg=seg, layers=layers))
    active = bool(np.any((wl.idx >= 0) & (wl.idx < S)))

    def do_segments(st):
        glsa.build_segments(st["idx"], S, mode=args.mode, seg=st["seg"])

    def do_shrink(st, li):
        d = st["layers"][li]
        glsa.shrink(d["x"], d["A"], st["seg"], scale=d["scale"], ranks=d["ranks"], v=d["v"],
                    active=active)

    def do_expand(st, li):
        d, p = st["layers"][li], problems[li]
        glsa.expand(d["v"], d["B"], d["y"], st["seg"], p.out_offsets, ranks=d["ranks"],
                    active=active)

    fused = args.path == "fused"
    # The first layer's shrink_expand call builds the segment record itself
    # when given idx (inside its one launch for 16-bit batches of at most
    # lora_fused_max_tokens() tokens and 256 slots); the later layers read it.
    build_in_call = (fused and not args.separate_build and active and problems[0].timed_expand
                     and wl.dtype in ("f16", "bf16") and T <= glsa.fused_max_tokens() and S <= 256)

    def do_fused(st, li):
        d, p = st["layers"][li], problems[li]
        glsa.shrink_expand(d["x"], d["A"], d["B"], d["y"], st["seg"], p.out_offsets,
                           workspace=d["ws"], scale=d["scale"], ranks=d["ranks"], v=d["v"],
                           idx=st["idx"] if build_in_call and li == 0 else None, active=active)

    def step(st):
        if not build_in_call:
            do_segments(st)
        for li, p in enumerate(problems):
            if fused and p.timed_expand:
                do_fused(st, li)
                continue
            do_shrink(st, li)
            if p.timed_expand:
                do_expand(st, li)

    if args.calibrate_copy > 0:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # warmup (eager)
    for i in range(args.warmup):
        step(sets[i % n_sets])
    torch.cuda.synchronize()

    # eager timing (host-launched), for reference
    n_eager = min(args.steps, 4 * n_sets)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_eager):
        step(sets[i % n_sets])
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / n_eager

    def capture(fn_list):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for fn in fn_list:  # one eager pass on the capture stream first
                fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for fn in fn_list:
                fn()
        torch.cuda.synchronize()
        return g

    timed_mode = "eager" if args.eager else "graph"
    if args.eager:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(sets[i % n_sets])
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    else:
        g_step = capture([(lambda st=st: step(st)) for st in sets[:chunk]])
        g_step.replay()
        torch.cuda.synchronize()
        reps = args.steps // chunk
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            g_step.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    value = T * args.steps / elapsed

    # per-call GPU time: graph of `chunk` calls of one kind, replayed between events
    def call_time_us(fn_of_set, reps=20):
        g = capture([(lambda st=st: fn_of_set(st)) for st in sets[:chunk]])
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * chunk)

    calls = {}
    alg = [algorithmic(p) for p in problems]
    if args.no_calls:
        print(json.dumps(dict(metric=METRIC, value=round(value, 1), unit="tokens/s", n_gpus=1, steps=args.steps,
                              warmup=args.warmup, ms_per_step=round(ms_per_step, 6), timed_mode=timed_mode,
                              config=dict(workload=args.workload), calls=None)), flush=True)
        return
    calls["segments"] = dict(us=call_time_us(do_segments), bytes=segment_bytes(T, alg[0]["n_active"]),
                             flops=0)
    if active:
        for li, p in enumerate(problems):
            if fused and p.timed_expand:
                name = f"{p.name}.shrink_expand" + ("+segments" if build_in_call and li == 0 else "")
                calls[name] = dict(
                    us=call_time_us(lambda st, li=li: do_fused(st, li)),
                    bytes=alg[li]["shrink_bytes"] + alg[li]["expand_bytes"]
                    + (segment_bytes(T, alg[0]["n_active"]) if build_in_call and li == 0 else 0),
                    flops=alg[li]["shrink_flops"] + alg[li]["expand_flops"])
                continue
            calls[f"{p.name}.shrink"] = dict(us=call_time_us(lambda st, li=li: do_shrink(st, li)),
                                             bytes=alg[li]["shrink_bytes"], flops=alg[li]["shrink_flops"])
            if p.timed_expand:
                calls[f"{p.name}.expand"] = dict(us=call_time_us(lambda st, li=li: do_expand(st, li)),
                                                 bytes=alg[li]["expand_bytes"],
                                                 flops=alg[li]["expand_flops"])
    for c in calls.values():
        c["gbs"] = c["bytes"] / (c["us"] * 1e-6) / 1e9 if c["us"] > 0 else 0.0
        c["tflops"] = c["flops"] / (c["us"] * 1e-6) / 1e12 if c["us"] > 0 else 0.0
    dom_name = max(calls, key=lambda k: calls[k]["us"])
    dom = calls[dom_name]
    # (with the record built inside the first call, the separately timed
    # segment build is not part of the step)
    in_step = [c for k, c in calls.items() if not (build_in_call and k == "segments")]
    step_bytes = sum(c["bytes"] for c in in_step)
    step_flops = sum(c["flops"] for c in in_step)

    roofline = dict(bound="hbm", kernel=dom_name, achieved=round(dom["gbs"], 1), peak=HBM_PEAK_GBS,
                    unit="GB/s", frac=round(dom["gbs"] / HBM_PEAK_GBS, 4),
                    traffic=measured_traffic(args.workload, dom_name),
                    alg_bytes_per_launch=dom["bytes"], avg_launch_us=round(dom["us"], 3),
                    source_hash=kernel_source_hash())

    noop = None
    if not active:
        noop = noop_overhead(torch, glsa, sets[0], problems[0], S, capture)

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(wl, args.cpu_seconds)
        cpu["value"] = round(cpu["value"], 2)

    out = dict(
        metric=METRIC, value=round(value, 1), unit="tokens/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=round(ms_per_step, 6), higher_is_better=True,
        scaling="weak", vs_baseline=None, dtype=wl.dtype, data="synthetic",
        config=dict(workload=args.workload, title=cfg["title"], T=T, S=S, r_max=wl.r_max,
                    layers=[dict(name=p.name, D=p.D, out=list(p.out_sizes),
                                 timed_expand=p.timed_expand) for p in problems],
                    n_active=alg[0]["n_active"], n_distinct_slots=alg[0]["n_distinct"],
                    mode=args.mode, path=args.path, record_built_in_first_call=build_in_call,
                    timing=timed_mode, input_sets=n_sets,
                    accumulate="fp32"),
        step_gbs=round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        step_tflops=round(step_flops / (ms_per_step * 1e-3) / 1e12, 3),
        eager_ms_per_step=round(eager_ms, 4),
        calls={k: dict(us=round(c["us"], 3), alg_bytes=c["bytes"], gbs=round(c["gbs"], 1),
                       frac_hbm=round(c["gbs"] / HBM_PEAK_GBS, 4), tflops=round(c["tflops"], 3))
               for k, c in calls.items()},
        roofline=roofline,
        cpu_baseline=cpu,
    )
    if noop is not None:
        out["noop"] = noop
    line = json.dumps(out)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "a") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
