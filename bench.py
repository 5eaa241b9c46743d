#!/usr/bin/env python3
"""Benchmark of the multi-LoRA hot path on one MI355X.

A step is one pass of the whole path over one batch: the segment build, then
for every LoRA layer of the workload its shrink and (where timed) its expand.
Each layer with a timed expand is one shrink_expand call (one launch for
16-bit batches of at most 4096 tokens, else the shrink launch and the expand
launch); the first one is given the batch's idx so that it builds the segment
record itself where it runs as one launch, and otherwise the build kernel runs
first.  The later layers read that record.

The headline (`value`, `ms_per_step`, `roofline`) is the workload named by
--workload, by default prefill_qkv, the largest of the five configurations
(fused QKV prefill of 16 requests x 512 tokens at Llama-3-8B shapes, bf16).
Then, unless --only is given, every configuration is run the same way and
summarised under `configs`.

Inputs are resident in HBM before timing starts.  Steps rotate over device
copies of the inputs whose number is chosen from their size alone, so that
the sets together exceed twice the 256 MB last-level cache at any step count;
the byte rates are then HBM rates, not cache rates.  Steps are replayed from
captured HIP graphs (a graph of one pass over every set, and one of the first
K mod sets steps), exactly K steps between two synchronisations.

After timing, set 0's outputs are restored to their initial values, the step
graph is replayed once more and set 0's y and v are compared with the fp64
oracle on sampled rows; its segment record is compared with the oracle's
grouping bit for bit; every workspace's count of waits that gave up must be 0.
Any failure exits non-zero instead of printing a number.

Prints ONE JSON line on stdout.  `value` is tokens per second (batch tokens T
per step).  `roofline` is for the kernel that takes the most GPU time per
step: its algorithmic bytes (active rows, distinct slots at their real ranks,
the fp32 intermediate's write and read) divided by its average duration,
measured here with HIP events around graph replays of that kernel's call
alone, on the stream the library launches on.  `cpu_baseline` is the fp64
oracle on a bounded sample of the headline workload, timed on every usable
host core (one process per core, BLAS limited to one thread each) before the
GPU is touched.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--only]
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
MFMA_PEAK_TFLOPS_16 = 2500.0   # dense fp16/bf16 MFMA, public datasheet
MALL_BYTES = 256 << 20         # last-level (Infinity) cache
ROTATE_BYTES = 2 * MALL_BYTES  # the input sets together exceed this
MAX_SETS = 128
DEFAULT_WORKLOAD = "prefill_qkv"
CHECK_ROWS = 256               # random rows compared with the oracle (plus each slot's first and last)
Y_TOL = {"f32": 1e-5, "f16": 5e-3, "bf16": 2e-2}
V_TOL = 1e-4


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--only", action="store_true", help="run the headline workload only (no `configs`)")
    ap.add_argument("--mode", default="auto", choices=["auto", "bgmv", "sgmv"])
    ap.add_argument("--separate-build", action="store_true",
                    help="build the segment record with lora_build_segments before the first layer "
                         "instead of inside the first layer's shrink_expand call")
    ap.add_argument("--eager", action="store_true", help="time host launches instead of graph replay")
    ap.add_argument("--b-layout", default="auto", choices=["auto", "padded", "rank_rows"],
                    help="storage of the slots' B rows; auto: rank_rows for workloads with per-slot ranks")
    ap.add_argument("--path", default="fused", choices=["fused", "split"],
                    help="fused: each layer with a timed expand is one shrink_expand call; "
                         "split: a shrink call then an expand call")
    ap.add_argument("--no-calls", action="store_true",
                    help="skip the per-call timing and the checks (counter runs: kernels then run "
                         "in step order only)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock budget of the oracle's CPU timing (0 disables it)")
    ap.add_argument("--cpu-procs", type=int, default=0,
                    help="host processes for the CPU baseline (0: every usable core, at most 16)")
    ap.add_argument("--json-out", default=None, help="also append the JSON line to this file")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="run one device-to-device copy of this many MiB before timing, as the "
                         "known-size reference kernel for FETCH_SIZE/WRITE_SIZE counter runs")
    return ap.parse_args()


def say(*a):
    print(*a, file=sys.stderr, flush=True)


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


def check_rows(idx, S, seed=0):
    """Rows compared with the oracle: each slot's first and last token, a few
    base tokens and CHECK_ROWS random tokens."""
    import numpy as np
    rng = np.random.default_rng(seed)
    T = idx.shape[0]
    picks = set()
    for s in np.unique(idx):
        where = np.nonzero(idx == s)[0]
        picks.update([int(where[0]), int(where[-1])])
    picks.update(int(t) for t in rng.choice(T, size=min(CHECK_ROWS, T), replace=False))
    return np.array(sorted(picks))


# --------------------------------------------------------------------------
# cpu_baseline leg: the fp64 oracle on the host, timed on a bounded sample,
# and its values for the sampled rows the GPU output is checked against
# --------------------------------------------------------------------------

_CPU_JOB = None  # (workload, seconds) for the forked workers


def _cpu_worker(i):
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle

    wl, seconds = _CPU_JOB
    rng = np.random.default_rng(1000 + i)
    done = 0
    n = min(wl.T, 64)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            tokens = np.sort(rng.choice(wl.T, size=n, replace=False))
            for p in wl.problems:
                v = oracle.oracle_shrink(p.x, p.A, p.idx, p.S, dtype=p.dtype, D=p.D,
                                         scale=p.scale, ranks=p.ranks, tokens=tokens)
                if p.timed_expand:
                    oracle.oracle_expand(v, p.B, p.y_in, p.idx, p.S, p.out_offsets,
                                         dtype=p.dtype, ranks=p.ranks, tokens=tokens)
            done += n
            el = time.perf_counter() - t0
            if el >= seconds:
                return done, el


def cpu_baseline(wl, seconds, procs):
    """Oracle tokens/s over `procs` host processes (forked before the GPU is
    initialised; each runs the oracle on random 64-token samples of the batch,
    every layer of the step, for `seconds` of wall clock)."""
    import multiprocessing

    global _CPU_JOB
    _CPU_JOB = (wl, seconds)
    ctx = multiprocessing.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(procs) as pool:
        res = pool.map(_cpu_worker, range(procs))
    wall = time.perf_counter() - t0
    _CPU_JOB = None
    tokens = sum(r[0] for r in res)
    el = max(r[1] for r in res)
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return dict(value=round(tokens / el, 2), unit="tokens/s", cores=procs, kind="oracle",
                sample=f"random 64-token samples of the {wl.T}-token {wl.name} batch (every layer "
                       f"of the step: shrink and timed expand), {tokens} tokens in {el:.1f} s on "
                       f"{procs} host processes of one thread each (BLAS limited to 1 thread); "
                       f"{len(os.sched_getaffinity(0))} usable cores; wall {wall:.1f} s",
                cpu_model=model)


def oracle_refs(wl, rows):
    """The oracle's v and y for the sampled rows of every layer, and its
    grouping of the batch (for the bit-exact record check)."""
    import oracle
    refs = []
    for p in wl.problems:
        v, y = oracle.oracle_apply(p.x, p.A, p.B, p.y_in, p.idx, p.S, p.out_offsets,
                                   dtype=p.dtype, D=p.D, scale=p.scale, ranks=p.ranks,
                                   tokens=rows)
        refs.append((v, y))
    return refs, oracle.oracle_segments(wl.idx, wl.S)


def decode_rows(a, dtype):
    """Exact fp64 values of stored output rows (numpy arrays from the GPU)."""
    import oracle
    return oracle.decode(a, dtype)


# --------------------------------------------------------------------------
# GPU side
# --------------------------------------------------------------------------

def rel_err(got, ref):
    import numpy as np
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    den = float(np.max(np.abs(ref)))
    num = float(np.max(np.abs(got - ref)))
    return num / den if den > 0 else num


def capture(torch, fn_list):
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


def copy_peak_gbs(torch, dev, mib=1024, reps=10):
    """Rate of a device-to-device copy of `mib` MiB (read + write bytes / time)."""
    src = torch.empty(mib << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * (mib << 20) / (us * 1e-6) / 1e9


def noop_overhead(torch, glsa, layer, p, reps=20, iters=50):
    """The cost of the LoRA path on an all-base batch, next to the base layer.

    The base layer is the layer's own dense projection, y = x W^T (a
    T x D by D x out fp16 GEMM, as the q_proj of Llama-3-8B at T = 4096).  With
    LoRA enabled and no adapter active the caller passes active = False (the
    host knows the batch holds no adapter; no segment build is run either) and
    shrink_expand enqueues nothing.  Both loops are timed in graph replay and
    eager, `iters` layers per timing, median of `reps`; overhead = with_lora /
    base - 1.
    """
    import statistics
    d = layer
    x = d["x"]
    W = torch.randn((sum(p.out_sizes), p.D), device=x.device, dtype=x.dtype) * 0.01
    out = torch.empty((x.size(0), W.size(0)), device=x.device, dtype=x.dtype)

    def base():
        torch.matmul(x, W.t(), out=out)

    def with_lora():
        torch.matmul(x, W.t(), out=out)
        glsa.shrink_expand(d["x"], d["A"], d["B"], d["y"], d["seg"], p.out_offsets,
                           workspace=d["ws"], scale=d["scale"], ranks=d["ranks"], v=d["v"],
                           idx=d["idx"], active=False)

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
                g = capture(torch, [fn] * iters)
                t[name] = timed(g.replay)
            else:
                t[name] = timed(lambda fn=fn: [fn() for _ in range(iters)])
        res[mode] = dict(base_us=round(t["base"], 3), with_lora_us=round(t["with_lora"], 3),
                         overhead=round(t["with_lora"] / t["base"] - 1.0, 5))
    res["base_layer"] = f"fp16 GEMM [{x.size(0)} x {p.D}] x [{p.D} x {W.size(0)}] (torch.matmul)"
    res["bar"] = 0.02
    return res


class Failure(Exception):
    """A check of the timed output failed: the bench prints no number."""


def run_config(name, args, torch, glsa, dev, copy_gbs, headline):
    """Time one workload's step; returns its summary (and raises Failure when
    a check fails)."""
    import numpy as np

    from workloads import CONFIGS, make_workload
    from workloads.torch_io import from_torch, problem_to_device

    t_setup = time.perf_counter()
    wl = make_workload(name)
    cfg = CONFIGS[name]
    T, S = wl.T, wl.S
    problems = wl.problems
    active = bool(np.any((wl.idx >= 0) & (wl.idx < S)))
    fused = args.path == "fused"
    is16 = wl.dtype in ("f16", "bf16")
    one_launch = fused and T <= glsa.fused_max_tokens_for(wl.dtype)
    # the first layer's call builds the record inside its one launch
    build_in_call = (one_launch and not args.separate_build and active and problems[0].timed_expand
                     and S <= 256)

    base = [problem_to_device(p, dev) for p in problems]
    # adapters of per-slot ranks are stored rank-compact (each slot's B rows
    # packed with the stride of its rank): an adapter-load-time layout, so
    # that low-rank slots are read without their zero padding
    b_layout = "rank_rows" if args.b_layout == "auto" and problems[0].ranks is not None else \
        ("padded" if args.b_layout == "auto" else args.b_layout)
    if b_layout == "rank_rows":
        for p, d in zip(problems, base):
            rk = p.ranks if p.ranks is not None else [p.r_max] * p.S
            d["B"] = [glsa.pack_b_rank_rows(b, rk) for b in d["B"]]
        torch.cuda.synchronize()

    def nbytes(d):
        tot = d["x"].numel() * d["x"].element_size() + d["y"].numel() * d["y"].element_size()
        tot += sum(a.numel() * a.element_size() for a in d["A"])
        tot += sum(b.numel() * b.element_size() for b in d["B"])
        return tot
    set_bytes = sum(nbytes(d) for d in base)
    n_sets = max(2, min(MAX_SETS, math.ceil(ROTATE_BYTES / set_bytes)))
    sets = []
    for _ in range(n_sets):
        layers = []
        for p, d in zip(problems, base):
            c = {k: (v.clone() if torch.is_tensor(v) else [t.clone() for t in v] if isinstance(v, list) else v)
                 for k, v in d.items()}
            c["v"] = torch.empty((p.n_slices, T, p.r_max), dtype=torch.float32, device=dev)
            c["ws"] = glsa.alloc_workspace(T, S, p.n_slices, p.r_max, dev)
            layers.append(c)
        seg = glsa.alloc_segments(T, S, dev)
        for c in layers:
            c["seg"] = seg
        sets.append(dict(idx=layers[0]["idx"], seg=seg, layers=layers))

    def do_segments(st):
        glsa.build_segments(st["idx"], S, mode=args.mode, seg=st["seg"])

    def do_shrink(st, li):
        d = st["layers"][li]
        glsa.shrink(d["x"], d["A"], st["seg"], scale=d["scale"], ranks=d["ranks"], v=d["v"],
                    active=active)

    def do_expand(st, li):
        d, p = st["layers"][li], problems[li]
        glsa.expand(d["v"], d["B"], d["y"], st["seg"], p.out_offsets, ranks=d["ranks"],
                    active=active, b_layout=b_layout)

    def do_fused(st, li):
        d, p = st["layers"][li], problems[li]
        glsa.shrink_expand(d["x"], d["A"], d["B"], d["y"], st["seg"], p.out_offsets,
                           workspace=d["ws"], scale=d["scale"], ranks=d["ranks"], v=d["v"],
                           idx=st["idx"] if build_in_call and li == 0 else None, active=active,
                           b_layout=b_layout)

    def step(st):
        # a base-only batch: the host knows no adapter is active and runs
        # nothing (no build; the calls enqueue nothing)
        if active and not build_in_call:
            do_segments(st)
        for li, p in enumerate(problems):
            if fused and p.timed_expand:
                do_fused(st, li)
                continue
            do_shrink(st, li)
            if p.timed_expand:
                do_expand(st, li)

    if args.calibrate_copy > 0 and headline:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    say(f"[bench] {name}: T={T} S={S} dtype={wl.dtype} sets={n_sets} x {set_bytes / 1e6:.1f} MB, "
        f"setup {time.perf_counter() - t_setup:.1f} s")
    out = dict(title=cfg["title"], T=T, S=S, dtype=wl.dtype, b_layout=b_layout, input_sets=n_sets,
               input_set_bytes=set_bytes, rotated_bytes=n_sets * set_bytes)

    if not active:
        # nothing is enqueued for this batch: report the overhead next to the
        # layer's base projection
        d = dict(sets[0]["layers"][0])
        d["idx"] = sets[0]["idx"]
        out["noop"] = noop_overhead(torch, glsa, d, problems[0])
        out["step_us"] = 0.0
        return out, None

    for i in range(args.warmup):
        step(sets[i % n_sets])
    torch.cuda.synchronize()

    # eager (host-launched) time, for reference
    n_eager = min(args.steps, 4 * n_sets)
    t0 = time.perf_counter()
    for i in range(n_eager):
        step(sets[i % n_sets])
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / n_eager

    K = args.steps
    g_all = capture(torch, [(lambda st=st: step(st)) for st in sets])
    rem = K % n_sets
    g_rem = capture(torch, [(lambda st=st: step(st)) for st in sets[:rem]]) if rem else None
    g_all.replay()
    torch.cuda.synchronize()
    if args.eager:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            step(sets[i % n_sets])
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K // n_sets):
            g_all.replay()
        if g_rem is not None:
            g_rem.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / K
    out.update(steps=K, step_us=round(ms_per_step * 1e3, 3), tokens_per_s=round(T * K / elapsed, 1),
               eager_step_us=round(eager_ms * 1e3, 3), timing="eager" if args.eager else "graph",
               record_built_in_first_call=build_in_call, one_launch=one_launch)
    say(f"[bench] {name}: {ms_per_step * 1e3:.2f} us/step, {T * K / elapsed:.4g} tokens/s")
    if args.no_calls:
        return out, None

    # ---- per-kernel GPU time: a graph of one call per set, replayed between events
    def call_time_us(fn_of_set, reps=20):
        g = capture(torch, [(lambda st=st: fn_of_set(st)) for st in sets])
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * n_sets)

    alg = [algorithmic(p) for p in problems]
    seg_b = segment_bytes(T, alg[0]["n_active"])
    calls = {}
    # lora_build_segments runs its wide kernel from 512 tokens, the one-workgroup kernel below
    seg_kernel = "build_segments_wide_kernel" if T >= 512 else "build_segments_kernel"
    calls["segments"] = dict(kernel=seg_kernel, us=call_time_us(do_segments), bytes=seg_b, flops=0,
                             in_step=not build_in_call)
    for li, p in enumerate(problems):
        if fused and p.timed_expand and one_launch:
            first = build_in_call and li == 0
            calls[f"{p.name}.shrink_expand" + ("+segments" if first else "")] = dict(
                kernel="fused_kernel", us=call_time_us(lambda st, li=li: do_fused(st, li)),
                bytes=alg[li]["shrink_bytes"] + alg[li]["expand_bytes"] + (seg_b if first else 0),
                flops=alg[li]["shrink_flops"] + alg[li]["expand_flops"], in_step=True)
            continue
        calls[f"{p.name}.shrink"] = dict(kernel="shrink_kernel", us=call_time_us(lambda st, li=li: do_shrink(st, li)),
                                         bytes=alg[li]["shrink_bytes"], flops=alg[li]["shrink_flops"], in_step=True)
        if p.timed_expand:
            kern = "bgmv_expand_kernel" if wl.dtype == "f32" else "mfma_expand_kernel"
            calls[f"{p.name}.expand"] = dict(kernel=kern, us=call_time_us(lambda st, li=li: do_expand(st, li)),
                                             bytes=alg[li]["expand_bytes"], flops=alg[li]["expand_flops"],
                                             in_step=True)
    for c in calls.values():
        c["gbs"] = c["bytes"] / (c["us"] * 1e-6) / 1e9 if c["us"] > 0 else 0.0
        c["tflops"] = c["flops"] / (c["us"] * 1e-6) / 1e12 if c["us"] > 0 else 0.0
    in_step = {k: c for k, c in calls.items() if c["in_step"]}
    dom_name = max(in_step, key=lambda k: in_step[k]["us"])
    dom = calls[dom_name]
    step_bytes = sum(alg[i]["shrink_bytes"] + (alg[i]["expand_bytes"] if p.timed_expand else 0)
                     for i, p in enumerate(problems)) + seg_b
    step_flops = sum(alg[i]["shrink_flops"] + (alg[i]["expand_flops"] if p.timed_expand else 0)
                     for i, p in enumerate(problems))
    traffic = measured_traffic(name, dom_name)
    step_gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    out.update(
        n_active=alg[0]["n_active"], n_distinct=alg[0]["n_distinct"],
        alg_bytes=step_bytes, alg_flops=step_flops,
        step_gbs=round(step_gbs, 1), frac_hbm_peak=round(step_gbs / HBM_PEAK_GBS, 4),
        frac_hbm_measured=round(step_gbs / copy_gbs, 4),
        step_tflops=round(step_flops / (ms_per_step * 1e-3) / 1e12, 3),
        mfma_frac_alg=round(step_flops / (ms_per_step * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS_16, 5)
        if is16 else None,
        calls={k: dict(kernel=c["kernel"], us=round(c["us"], 3), alg_bytes=c["bytes"], gbs=round(c["gbs"], 1),
                       frac_hbm=round(c["gbs"] / HBM_PEAK_GBS, 4), tflops=round(c["tflops"], 3),
                       in_step=c["in_step"])
               for k, c in calls.items()},
        # the same figures under the per-config names of the measurement
        # plan: gbps is the step's algorithmic rate, mfma_util the algorithmic
        # MFMA share (the counter-measured one is in the committed MFMA
        # summary), and the call times by kind (a one-launch call is shrink
        # and expand together)
        gbps=round(step_gbs, 1),
        mfma_util=round(step_flops / (ms_per_step * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS_16, 5) if is16 else None,
        t_segments_us=round(sum(c["us"] for k, c in calls.items() if k == "segments"), 3),
        t_shrink_us=round(sum(c["us"] for k, c in calls.items() if k.endswith(".shrink") and c["in_step"]), 3),
        t_expand_us=round(sum(c["us"] for k, c in calls.items() if k.endswith(".expand") and c["in_step"]), 3),
        t_shrink_expand_us=round(sum(c["us"] for k, c in calls.items()
                                     if ".shrink_expand" in k and c["in_step"]), 3),
        dominant=dict(call=dom_name, kernel=dom["kernel"], us=round(dom["us"], 3), gbs=round(dom["gbs"], 1),
                      frac_hbm=round(dom["gbs"] / HBM_PEAK_GBS, 4),
                      # the kernel's share of the attainable roofline min(P_mfma, AI * BW):
                      # below the MFMA ridge that is the HBM bound
                      frac_attainable=round(dom["gbs"] / HBM_PEAK_GBS, 4)
                      if dom["bytes"] == 0 or dom["flops"] / dom["bytes"] < MFMA_PEAK_TFLOPS_16 * 1e12 / (HBM_PEAK_GBS * 1e9)
                      else round(dom["tflops"] / MFMA_PEAK_TFLOPS_16, 4),
                      traffic_bytes=traffic,
                      traffic_ratio=round(traffic / dom["bytes"], 3) if traffic else None),
    )

    # ---- the mask ("laning") form, where the stacked lanes allow it: the same
    # layers with every token multiplied by all adapters' lanes, no segment
    # build (compared with the gather step above, which includes its build)
    if S * wl.r_max <= glsa.MASK_MAX_LANES and all(p.timed_expand for p in problems) and b_layout == "padded":
        for st in sets:
            for li, p in enumerate(problems):
                d = st["layers"][li]
                d["mws"] = glsa.alloc_mask_workspace(d["x"].dtype, T, p.D, S, p.n_slices, p.r_max, dev)

        def do_mask(st):
            for li, p in enumerate(problems):
                d = st["layers"][li]
                glsa.shrink_expand_mask(d["x"], d["A"], d["B"], d["y"], st["idx"], p.out_offsets,
                                        workspace=d["mws"], scale=d["scale"], ranks=d["ranks"], v=d["v"])
        mask_us = call_time_us(do_mask)
        out["mask_form"] = dict(us=round(mask_us, 3), gather_step_us=out["step_us"],
                                speedup_vs_gather=round(out["step_us"] / mask_us, 3),
                                lanes=S * wl.r_max)
        say(f"[bench] {name}: mask form {mask_us:.2f} us against the gather step {out['step_us']:.2f} us")

    # ---- checks of the timed output: set 0 restored, the step replayed once
    rows = check_rows(wl.idx, S)
    refs, seg_ref = oracle_refs(wl, rows)
    st0 = sets[0]
    for li in range(len(problems)):
        st0["layers"][li]["y"].copy_(base[li]["y"])
        st0["layers"][li]["v"].fill_(float("nan"))
    torch.cuda.synchronize()
    g_all.replay()
    torch.cuda.synchronize()
    errs_y, errs_v = [], []
    for li, p in enumerate(problems):
        v_ref, y_ref = refs[li]
        v_got = st0["layers"][li]["v"][:, torch.from_numpy(rows).to(dev)].cpu().numpy().astype(np.float64)
        errs_v.append(rel_err(v_got, v_ref))
        if p.timed_expand:
            y_got = decode_rows(from_torch(st0["layers"][li]["y"], p.dtype)[rows], p.dtype)
            errs_y.append(rel_err(y_got, y_ref))
    rec = st0["seg"].cpu().numpy()
    fields = {k: glsa.segments_offset(T, S, k) for k in ("perm", "seg_slot", "seg_start")}
    na, ns_ = int(seg_ref["num_active"]), int(seg_ref["num_segments"])
    meta_ok = bool(
        rec[0] == na and rec[1] == ns_ and rec[2] == seg_ref["max_seg_len"] and rec[3] == seg_ref["status"]
        and np.array_equal(rec[fields["perm"]:fields["perm"] + na], seg_ref["perm"])
        and np.array_equal(rec[fields["perm"] + na:fields["perm"] + T], seg_ref["rest"])
        and np.array_equal(rec[fields["seg_slot"]:fields["seg_slot"] + ns_], seg_ref["seg_slot"])
        and np.array_equal(rec[fields["seg_start"]:fields["seg_start"] + ns_ + 1], seg_ref["seg_start"]))
    gave_up = sum(glsa.workspace_errors(l["ws"]) for st in sets for l in st["layers"])
    err_y = max(errs_y) if errs_y else 0.0
    err_v = max(errs_v)
    # err_y is the infinity-norm error of y relative to the oracle's largest
    # |y| on the checked rows (also reported as err_inf)
    out.update(err_y=float(f"{err_y:.3e}"), err_inf=float(f"{err_y:.3e}"), err_v=float(f"{err_v:.3e}"),
               frac_attainable=out["dominant"]["frac_attainable"], y_tol=Y_TOL[wl.dtype], v_tol=V_TOL,
               checked_rows=int(len(rows)), meta_bitexact=meta_ok, workspace_errors=int(gave_up))
    say(f"[bench] {name}: err_y {err_y:.2e} err_v {err_v:.2e} record bit-exact {meta_ok} waits given up {gave_up}")
    if gave_up:
        raise Failure(f"{name}: {gave_up} device-side waits gave up: the timed output is invalid")
    if err_y > Y_TOL[wl.dtype] or err_v > V_TOL or not meta_ok:
        raise Failure(f"{name}: timed output does not match the oracle (err_y {err_y:.3e}, err_v {err_v:.3e}, "
                      f"record bit-exact {meta_ok})")

    roofline = dict(bound="hbm", kernel=dom["kernel"], call=dom_name, achieved=round(dom["gbs"], 1),
                    peak=HBM_PEAK_GBS, unit="GB/s", frac=round(dom["gbs"] / HBM_PEAK_GBS, 4),
                    traffic=traffic, alg_bytes_per_launch=dom["bytes"], avg_launch_us=round(dom["us"], 3),
                    source_hash=kernel_source_hash())
    del sets, base
    torch.cuda.empty_cache()
    return out, roofline


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(no collectives or sharding); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    from workloads import CONFIG_ORDER, make_workload

    # the CPU baseline first, in processes forked before anything touches the GPU
    cpu = None
    if args.cpu_seconds > 0:
        procs = args.cpu_procs or min(16, len(os.sched_getaffinity(0)))
        say(f"[bench] cpu baseline: oracle on {procs} host processes for {args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(make_workload(args.workload), args.cpu_seconds, procs)

    import torch

    import gemm_lora_shrink_amd as glsa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    glsa.lib()
    copy_gbs = copy_peak_gbs(torch, dev)
    say(f"[bench] device copy of 1 GiB: {copy_gbs:.0f} GB/s (read + write)")

    try:
        head, roofline = run_config(args.workload, args, torch, glsa, dev, copy_gbs, headline=True)
        configs = None
        if not args.only:
            configs = {args.workload: head}
            for name in CONFIG_ORDER:
                if name != args.workload:
                    configs[name] = run_config(name, args, torch, glsa, dev, copy_gbs, headline=False)[0]
    except Failure as e:
        print(f"bench.py: FAILED: {e}", file=sys.stderr, flush=True)
        sys.exit(3)

    if cpu is not None and "tokens_per_s" in head:
        cpu["gpu_over_cpu"] = round(head["tokens_per_s"] / cpu["value"], 1)
    K = args.steps
    ms = head.get("step_us", 0.0) / 1e3
    out = dict(
        metric=METRIC, value=head.get("tokens_per_s", 0.0), unit="tokens/s", n_gpus=1, steps=K,
        warmup=args.warmup, ms_per_step=round(ms, 6), higher_is_better=True,
        scaling="weak", vs_baseline=None, dtype=head["dtype"], data="synthetic",
        config=dict(workload=args.workload, title=head["title"], T=head["T"], S=head["S"],
                    mode=args.mode, path=args.path, timing=head.get("timing"),
                    input_sets=head["input_sets"], input_set_bytes=head["input_set_bytes"],
                    rotated_bytes=head["rotated_bytes"], accumulate="fp32",
                    record_built_in_first_call=head.get("record_built_in_first_call")),
        step_gbs=head.get("step_gbs"), frac_hbm_peak=head.get("frac_hbm_peak"),
        frac_hbm_measured=head.get("frac_hbm_measured"), copy_peak_gbs=round(copy_gbs, 1),
        eager_ms_per_step=round(head.get("eager_step_us", 0.0) / 1e3, 6),
        err_y=head.get("err_y"), err_inf=head.get("err_inf"), err_v=head.get("err_v"),
        meta_bitexact=head.get("meta_bitexact"),
        workspace_errors=head.get("workspace_errors"),
        calls=head.get("calls"),
        # the all-base batch's overhead next to the base layer (its own config)
        noop=head.get("noop") or (configs or {}).get("zipf_many_noop", {}).get("noop"),
        roofline=roofline,
        cpu_baseline=cpu,
        configs=configs,
    )
    line = json.dumps(out)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "a") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
