"""GPU: the one-call shrink_expand (one launch for 16-bit data) matches the fp64
oracle to the same bars as shrink followed by expand, on the five workloads
and the edge cases, both reading the segment record and grouping the tokens
itself from idx; it leaves its workspace's counters at zero after every
call, so one workspace serves calls in stream order on batches of any shape;
and a captured step with it (the first layer's call building the record the
later layers read) replays correctly."""

import numpy as np
import pytest
import torch

import gemm_lora_shrink_amd as glsa
import oracle
from gpu_util import (V_TOL, Y_TOL, check_problem, fused_counter_bytes, oracle_ref, rel_err,
                      run_fused, sample_tokens, say)
from test_parity import edge_problems
from workloads import make_workload, random_problem
from workloads.torch_io import from_torch, problem_to_device

pytestmark = pytest.mark.gpu

FULL = [("tiny_bgmv", None), ("decode_qproj", None), ("prefill_qkv", 256),
        ("mixed_rank_mlp", None), ("zipf_many", 512)]


@pytest.mark.parametrize("source", ["record", "idx"])
@pytest.mark.parametrize("name,n_sample", FULL, ids=[f[0] for f in FULL])
def test_fused_workload_parity(name, n_sample, source):
    wl = make_workload(name)
    for p in wl.problems:
        tokens = None if n_sample is None else sample_tokens(p.idx, p.S, n_sample)
        check_problem(p, tokens=tokens, fused=source, label=f"fused-{source}/{name}/{p.name}")


@pytest.mark.parametrize("source", ["record", "idx"])
@pytest.mark.parametrize("case", list(edge_problems()), ids=lambda c: c[0])
def test_fused_edge_parity(case, source):
    label, p, mode = case
    if p.ranks is not None:  # garbage in the rank padding must be ignored
        for s, r in enumerate(p.ranks):
            for a in p.A:
                a[s, r:, :] = a.dtype.type(7) if a.dtype != np.uint16 else np.uint16(0x40e0)
            for b in p.B:
                b[s, :, r:] = b.dtype.type(7) if b.dtype != np.uint16 else np.uint16(0x40e0)
    check_problem(p, mode=mode, fused=source, label=f"fused-{source}/{label}")


def _record_words(seg, T, S):
    """The documented and planned parts of a record (everything the kernels read)."""
    rec = seg.cpu().numpy()
    off = {k: glsa.segments_offset(T, S, k) for k in glsa.SEG_FIELDS}
    info = rec[:16]
    return np.concatenate([
        info, rec[off["perm"]:off["perm"] + T],
        rec[off["seg_slot"]:off["seg_slot"] + info[1]],
        rec[off["seg_start"]:off["seg_start"] + info[1] + 1],
        rec[off["groups"]:off["groups"] + 20 * info[4]],
        rec[off["tiles"]:off["tiles"] + 68 * info[5]]])


def _idx_cases():
    rng = np.random.default_rng(31)
    idx = np.concatenate([np.full(70, 2), rng.integers(-3, 12, 300), np.arange(10)]).astype(np.int32)
    rng.shuffle(idx)
    for dtype in ("f16", "bf16"):
        # one launch, the record built inside it: a slot past 64 tokens (a
        # tile), every group size, base-only and out-of-range tokens
        yield f"in_launch_{dtype}", random_problem(rng, T=idx.size, D=320, out_sizes=(96, 256), r_max=32,
                                                   S=10, dtype=dtype, idx=idx.copy(), with_ranks=True)
    # one launch, S past 256: the build kernel runs first
    yield "build_kernel_S600", random_problem(rng, T=900, D=128, out_sizes=(64,), r_max=16, S=600,
                                              dtype="f16")
    # largest one-launch batch with the build inside; then two launches
    yield "in_launch_T4096", random_problem(rng, T=4096, D=256, out_sizes=(128,), r_max=16, S=256,
                                            dtype="bf16")
    yield "two_launches_T4200", random_problem(rng, T=4200, D=256, out_sizes=(128,), r_max=16, S=40,
                                               dtype="f16")
    # fp32: one launch up to 2048 tokens (chunks expanded on the vector ALUs,
    # per-slot ranks that are not multiples of 4), two launches past it
    yield "fp32_one_launch", random_problem(rng, T=200, D=64, out_sizes=(32, 300), r_max=8, S=5,
                                            dtype="f32", bad_idx_frac=0.1, with_ranks=True)
    yield "fp32_one_launch_T2048", random_problem(rng, T=2048, D=96, out_sizes=(520,), r_max=64, S=20,
                                                  dtype="f32", with_ranks=True)
    yield "fp32_two_launches", random_problem(rng, T=2100, D=64, out_sizes=(32,), r_max=8, S=5,
                                              dtype="f32", bad_idx_frac=0.1)
    yield "fp32_one_launch_strided", random_problem(rng, T=150, D=200, out_sizes=(64, 36), r_max=12, S=7,
                                                    dtype="f32", with_ranks=True, ldx=208, ldy=112)
    # two launches after the build kernel: every slot count, mostly gather
    # groups, a long contraction (K parts with atomics), no adapter at all
    yield "two_launches_S1024", random_problem(rng, T=5000, D=128, out_sizes=(64,), r_max=16, S=1024,
                                                dtype="f16", bad_idx_frac=0.05)
    yield "two_launches_groups", random_problem(rng, T=4500, D=256, out_sizes=(96, 64), r_max=32, S=400,
                                                 dtype="bf16", with_ranks=True)
    yield "two_launches_long_k", random_problem(rng, T=4300, D=8192, out_sizes=(64,), r_max=16, S=8,
                                                 dtype="bf16")
    yield "two_launches_all_base", random_problem(rng, T=4400, D=128, out_sizes=(64,), r_max=16, S=4,
                                                   dtype="f16", idx=np.full(4400, -1, np.int32))


@pytest.mark.parametrize("case", list(_idx_cases()), ids=lambda c: c[0])
def test_fused_idx_mode_builds_the_record(case):
    """With idx given, the call builds the record itself: a record full of
    garbage beforehand comes out equal, word for word, to the one
    lora_build_segments builds, and the layer matches the oracle."""
    label, p = case
    d = problem_to_device(p, "cuda")
    ref = glsa.build_segments(d["idx"], p.S)  # a separate record, the reference
    seg = glsa.alloc_segments(p.T, p.S, "cuda")
    seg.fill_(-7)
    say(f"[fused idx] {label} T={p.T} S={p.S} dtype={p.dtype}")
    v = run_fused(p, d, seg, from_idx=True)
    assert np.array_equal(_record_words(seg, p.T, p.S), _record_words(ref, p.T, p.S)), label
    v_ref, y_ref = oracle_ref(p)
    y = oracle.decode(from_torch(d["y"], p.dtype), p.dtype)
    assert rel_err(y, y_ref) <= Y_TOL[p.dtype]
    assert rel_err(v.cpu().numpy(), v_ref) <= V_TOL
    valid = (p.idx >= 0) & (p.idx < p.S)
    assert np.array_equal(from_torch(d["y"], p.dtype)[~valid], p.y_in[~valid])


def test_fused_workspace_reuse_across_batches():
    """One workspace for calls in stream order on batches of different sizes,
    slices and ranks, twice over: each call matches the oracle and leaves the
    counters at zero (checked inside run_fused)."""
    rng = np.random.default_rng(21)
    probs = [
        random_problem(rng, T=512, D=512, out_sizes=(256, 128), r_max=32, S=8, dtype="f16",
                       with_ranks=True),
        random_problem(rng, T=100, D=256, out_sizes=(128,), r_max=16, S=4, dtype="bf16"),
        random_problem(rng, T=700, D=1024, out_sizes=(64, 64, 64), r_max=64, S=40, dtype="bf16"),
        random_problem(rng, T=20, D=64, out_sizes=(32,), r_max=8, S=3, dtype="f16"),
    ]
    size = max(glsa.workspace_bytes(p.T, p.S, p.n_slices, p.r_max) for p in probs)
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    for rnd in range(2):
        for i, p in enumerate(probs):
            say(f"[fused reuse] round {rnd} problem {i} T={p.T} slices={p.out_sizes} r_max={p.r_max}")
            d = problem_to_device(p, "cuda")
            seg = glsa.build_segments(d["idx"], p.S)
            v = run_fused(p, d, seg, ws=ws, from_idx=(i + rnd) % 2 == 1)
            v_ref, y_ref = oracle_ref(p)
            y = oracle.decode(from_torch(d["y"], p.dtype), p.dtype)
            assert rel_err(y, y_ref) <= Y_TOL[p.dtype]
            assert rel_err(v.cpu().numpy(), v_ref) <= V_TOL


def test_fused_inactive_hint_enqueues_nothing():
    rng = np.random.default_rng(5)
    p = random_problem(rng, T=64, D=64, out_sizes=(64,), r_max=8, S=2, dtype="bf16", base_frac=1.0)
    d = problem_to_device(p, "cuda")
    seg = glsa.build_segments(d["idx"], p.S)
    ws = glsa.alloc_workspace(p.T, p.S, p.n_slices, p.r_max, "cuda")
    y0 = d["y"].clone()
    v = torch.full((1, p.T, p.r_max), 3.0, device="cuda")
    glsa.shrink_expand(d["x"], d["A"], d["B"], d["y"], seg, p.out_offsets, workspace=ws, v=v,
                       active=False)
    torch.cuda.synchronize()
    assert torch.equal(d["y"], y0) and bool(torch.all(v == 3.0)) and not torch.any(ws).item()


@pytest.mark.parametrize("name", ["decode_qproj", "mixed_rank_mlp"])
def test_fused_graph_replays(name):
    """shrink_expand layers, the first building the record, captured once and
    replayed 4 times, with
    the program's own eager work (y reset, v poisoned) and a synchronisation
    between replays; each replay matches the eager run and the oracle."""
    wl = make_workload(name)
    probs = wl.problems
    ds = [problem_to_device(p, "cuda") for p in probs]
    seg = glsa.alloc_segments(wl.T, wl.S, "cuda")
    vs = [torch.empty((p.n_slices, wl.T, p.r_max), dtype=torch.float32, device="cuda") for p in probs]
    wss = [glsa.alloc_workspace(p.T, p.S, p.n_slices, p.r_max, "cuda") for p in probs]
    y_in = [d["y"].clone() for d in ds]

    def step():
        # the first layer's call builds the record (idx given); the later
        # layers read it
        for li, (p, d, v, ws) in enumerate(zip(probs, ds, vs, wss)):
            glsa.shrink_expand(d["x"], d["A"], d["B"], d["y"], seg, p.out_offsets, workspace=ws,
                               scale=d["scale"], ranks=d["ranks"], v=v,
                               idx=d["idx"] if li == 0 else None)

    def reset():
        for d, y0 in zip(ds, y_in):
            d["y"].copy_(y0)
        for v in vs:
            v.fill_(float("nan"))
        seg.fill_(-7)  # rebuilt by every step

    reset()
    step()
    torch.cuda.synchronize()
    y_eager = [oracle.decode(from_torch(d["y"], p.dtype), p.dtype) for p, d in zip(probs, ds)]
    rows = sample_tokens(wl.idx, wl.S, 64)
    refs = [oracle_ref(p, tokens=rows) for p in probs]

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        reset()
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        say(f"[fused graph] {name} replay {rep}")
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for li, (p, d, v, ws) in enumerate(zip(probs, ds, vs, wss)):
            assert glsa.workspace_errors(ws) == 0
            vg = v.cpu().numpy().astype(np.float64)
            yg = oracle.decode(from_torch(d["y"], p.dtype), p.dtype)
            assert np.all(np.isfinite(vg)), f"{name} replay {rep}: v not fully written"
            assert rel_err(yg, y_eager[li]) <= Y_TOL[p.dtype] / 2
            v_ref, y_ref = refs[li]
            assert rel_err(vg[:, rows], v_ref) <= V_TOL
            assert rel_err(yg[rows], y_ref) <= Y_TOL[p.dtype]


def test_fused_wait_give_up_is_bounded_and_recoverable(monkeypatch):
    """Forced from the host: with at most one poll per wait, consumers that
    find their chunk incomplete give up at once.  The call still ends; either
    every wait succeeded (and y is right) or the give-ups are counted in the
    workspace.  Either way the per-chunk counters are back at zero (the last
    unit to count a chunk resets it, producer or consumer), so the next call
    on the same workspace, without clearing it, is right again and adds no
    give-up."""
    wl = make_workload("decode_qproj")
    p = wl.problems[0]
    d = problem_to_device(p, "cuda")
    seg = glsa.build_segments(d["idx"], p.S)
    ws = glsa.alloc_workspace(p.T, p.S, p.n_slices, p.r_max, "cuda")
    y0 = d["y"].clone()
    _, y_ref = oracle_ref(p)
    monkeypatch.setenv("LORA_MI355X_FUSED_SPIN_LIMIT", "0")
    glsa.shrink_expand(d["x"], d["A"], d["B"], d["y"], seg, p.out_offsets, workspace=ws,
                       scale=d["scale"], ranks=d["ranks"])
    torch.cuda.synchronize()  # returns: every wave exited
    gave_up = glsa.workspace_errors(ws)
    err = rel_err(oracle.decode(from_torch(d["y"], p.dtype), p.dtype), y_ref)
    say(f"[fused give-up] waits given up {gave_up}, y error {err:.2e}")
    assert gave_up > 0 or err <= Y_TOL[p.dtype]
    monkeypatch.delenv("LORA_MI355X_FUSED_SPIN_LIMIT")
    counters = ws[256:fused_counter_bytes(ws)]
    assert not torch.any(counters).item(), "a counter was left non-zero after give-ups"
    d["y"].copy_(y0)
    glsa.shrink_expand(d["x"], d["A"], d["B"], d["y"], seg, p.out_offsets, workspace=ws,
                       scale=d["scale"], ranks=d["ranks"])
    torch.cuda.synchronize()
    assert glsa.workspace_errors(ws) == gave_up
    assert rel_err(oracle.decode(from_torch(d["y"], p.dtype), p.dtype), y_ref) <= Y_TOL[p.dtype]
    host = torch.zeros(1, dtype=torch.int32).pin_memory()
    glsa.workspace_errors_async(ws, host)
    torch.cuda.synchronize()
    assert int(host[0]) == gave_up
