"""GPU: a step of the library's calls can be captured in a HIP graph and replayed.

Nothing in the library allocates, synchronises or uses hipMemsetAsync (v is
cleared by a kernel), so segment build, shrink and expand can be captured once
and replayed, as the graph-specialised serving path of "[LoRA] LoRA cuda graph
specialization" does with its LoRA kernels.  Each replay follows eager work of
this program (y reset to its input, v poisoned, the record overwritten) and a
synchronisation, and is checked against the eager run of the same calls and
against the oracle on sampled rows: the record bit for bit (it is deterministic), v and y to
within the rounding of summation order (v may be summed with atomics when the
shrink cuts its contraction into parts).
"""

import numpy as np
import pytest
import torch

import gemm_lora_shrink_amd as glsa
from gpu_util import V_TOL, Y_TOL, fused_counter_bytes, oracle_ref, rel_err, sample_tokens, say
from workloads import make_workload
from workloads.torch_io import from_torch, problem_to_device
import oracle

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _specified(seg, T, S):
    rec = seg.cpu().numpy()
    off = {k: glsa.segments_offset(T, S, k) for k in glsa.SEG_FIELDS}
    info = rec[:16]
    return np.concatenate([
        info, rec[off["perm"]:off["perm"] + T],
        rec[off["seg_slot"]:off["seg_slot"] + info[1]],
        rec[off["seg_start"]:off["seg_start"] + info[1] + 1],
        rec[off["groups"]:off["groups"] + 20 * info[4]],
        rec[off["tiles"]:off["tiles"] + 68 * info[5]]])


@pytest.mark.parametrize("name", ["tiny_bgmv", "decode_qproj", "mixed_rank_mlp", "zipf_many", "prefill_qkv"])
def test_graph_replays_match_eager(name):
    wl = make_workload(name)
    say(f"[graph] {name} T={wl.T} S={wl.S} replays={REPLAYS}")
    probs = wl.problems
    ds = [problem_to_device(p, "cuda") for p in probs]
    idx = ds[0]["idx"]
    seg = glsa.alloc_segments(wl.T, wl.S, "cuda")
    vs = [torch.empty((p.n_slices, wl.T, p.r_max), dtype=torch.float32, device="cuda") for p in probs]
    y_in = [d["y"].clone() for d in ds]

    def step():
        glsa.build_segments(idx, wl.S, seg=seg)
        for p, d, v in zip(probs, ds, vs):
            glsa.shrink(d["x"], d["A"], seg, scale=d["scale"], ranks=d["ranks"], v=v)
            glsa.expand(v, d["B"], d["y"], seg, p.out_offsets, ranks=d["ranks"])

    def reset():
        for d, y0 in zip(ds, y_in):
            d["y"].copy_(y0)
        for v in vs:
            v.fill_(float("nan"))
        seg.fill_(-7)

    # eager reference
    reset()
    step()
    torch.cuda.synchronize()
    rec_ref = _specified(seg, wl.T, wl.S)
    v_eager = [v.cpu().numpy().astype(np.float64) for v in vs]
    y_eager = [oracle.decode(from_torch(d["y"], p.dtype), p.dtype) for p, d in zip(probs, ds)]
    rows = sample_tokens(wl.idx, wl.S, 64)
    refs = [oracle_ref(p, tokens=rows) for p in probs]

    # capture (one pass on the capture stream first, as torch recommends)
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

    for rep in range(REPLAYS):
        reset()  # the program's own eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_specified(seg, wl.T, wl.S), rec_ref), f"{name} replay {rep}: record"
        for li, (p, d, v) in enumerate(zip(probs, ds, vs)):
            vg = v.cpu().numpy().astype(np.float64)
            yg = oracle.decode(from_torch(d["y"], p.dtype), p.dtype)
            assert np.all(np.isfinite(vg)), f"{name} replay {rep}: v not fully written"
            ev = rel_err(vg, v_eager[li])
            ey = rel_err(yg, y_eager[li])
            assert ev <= 1e-6, f"{name} replay {rep}: v differs from eager by {ev:.2e}"
            assert ey <= Y_TOL[p.dtype] / 2, f"{name} replay {rep}: y differs from eager by {ey:.2e}"
            v_ref, y_ref = refs[li]
            assert rel_err(vg[:, rows], v_ref) <= V_TOL, f"{name} replay {rep}: v vs oracle"
            assert rel_err(yg[rows], y_ref) <= Y_TOL[p.dtype], f"{name} replay {rep}: y vs oracle"


def test_two_graphs_chosen_by_host_flag():
    """The serving pattern of "[LoRA] LoRA cuda graph specialization"
    (Implementation): one graph captured with the LoRA call live, one with
    the host flag saying no adapter is active, and per step the host picks.
    The base layer's output is stood in for by a copy into y.  Steps
    alternate between a mixed batch (LoRA graph), an all-base batch (base
    graph) and an all-base batch sent to the LoRA graph anyway, whose kernels
    read the record they build and leave every row untouched."""
    wl = make_workload("decode_qproj")
    p = wl.problems[0]
    say(f"[graph] two graphs decode_qproj T={p.T} S={p.S}")
    d = problem_to_device(p, "cuda")
    y_base = d["y"].clone()                       # the base layer's output
    idx_mixed = d["idx"].clone()
    idx_none = torch.full_like(idx_mixed, -1)
    idx = torch.empty_like(idx_mixed)             # the static input of both graphs
    seg = glsa.alloc_segments(p.T, p.S, "cuda")
    ws = glsa.alloc_workspace(p.T, p.S, p.n_slices, p.r_max, "cuda")
    v = torch.empty((p.n_slices, p.T, p.r_max), dtype=torch.float32, device="cuda")

    def step(active):
        d["y"].copy_(y_base)
        glsa.shrink_expand(d["x"], d["A"], d["B"], d["y"], seg, p.out_offsets, workspace=ws,
                           scale=d["scale"], ranks=d["ranks"], v=v, idx=idx, active=active)

    idx.copy_(idx_mixed)
    step(True)
    torch.cuda.synchronize()
    y_eager = oracle.decode(from_torch(d["y"], p.dtype), p.dtype)
    rec_eager = _specified(seg, p.T, p.S)
    rows = sample_tokens(p.idx, p.S, 64)
    v_ref, y_ref = oracle_ref(p, tokens=rows)

    graphs = {}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(True)
        step(False)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for flag in (True, False):
        graphs[flag] = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graphs[flag]):
            step(flag)
    torch.cuda.synchronize()

    base_bits = from_torch(y_base, p.dtype)
    for k, (batch, flag) in enumerate([("mixed", True), ("none", False), ("mixed", True),
                                       ("none", True), ("none", False), ("mixed", True)]):
        idx.copy_(idx_mixed if batch == "mixed" else idx_none)
        d["y"].fill_(float("nan"))
        v.fill_(float("nan"))
        seg.fill_(-7)
        torch.cuda.synchronize()
        graphs[flag].replay()
        torch.cuda.synchronize()
        assert glsa.workspace_errors(ws) == 0, f"step {k}: a wait gave up"
        assert not torch.any(ws[:fused_counter_bytes(ws)]).item(), f"step {k}: counters not at zero"
        y_bits = from_torch(d["y"], p.dtype)
        if batch == "none":
            assert np.array_equal(y_bits, base_bits), f"step {k} ({batch}, {flag}): y changed"
            if not flag:
                # nothing of the library ran: v and the record keep the poison
                assert torch.all(torch.isnan(v)).item(), f"step {k}: v written by the base graph"
                assert torch.all(seg == -7).item(), f"step {k}: record written by the base graph"
            else:
                assert int(seg[0].item()) == 0, f"step {k}: record counts active tokens"
            continue
        assert np.array_equal(_specified(seg, p.T, p.S), rec_eager), f"step {k}: record"
        yg = oracle.decode(y_bits, p.dtype)
        assert rel_err(yg, y_eager) <= Y_TOL[p.dtype] / 2, f"step {k}: y differs from eager"
        assert rel_err(yg[rows], y_ref) <= Y_TOL[p.dtype], f"step {k}: y vs oracle"
        vg = v.cpu().numpy().astype(np.float64)
        assert rel_err(vg[:, rows], v_ref) <= V_TOL, f"step {k}: v vs oracle"
