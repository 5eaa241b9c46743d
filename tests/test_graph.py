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
from gpu_util import V_TOL, Y_TOL, oracle_ref, rel_err, sample_tokens, say
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


@pytest.mark.parametrize("name", ["tiny_bgmv", "decode_qproj", "mixed_rank_mlp", "zipf_many"])
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
