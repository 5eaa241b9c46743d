"""GPU: independent batches on two streams at once.

The split calls (segment build, shrink, expand) keep no state between calls
and never wait for another workgroup, so two batches whose calls are
interleaved on two streams (their kernels free to run side by side) each get
their own result.  (The one-launch call is the exception the header states:
its grid must be resident alone, so it is not run concurrently here.)  One
batch takes the large multi-slice path (>= 4096 tokens, three slices of rank
64, bf16, tiles cut across slices), the other a decode-sized gather batch
with out-of-range slots; both are checked against the oracle.
"""

import numpy as np
import pytest
import torch

import gemm_lora_shrink_amd as glsa
from gpu_util import V_TOL, Y_TOL, oracle_ref, rel_err, sample_tokens, say
from workloads import random_problem
from workloads.torch_io import from_torch, problem_to_device
import oracle

pytestmark = pytest.mark.gpu


def test_two_streams_independent_batches():
    rng = np.random.default_rng(21)
    probs = [
        random_problem(rng, T=5000, D=512, out_sizes=(256, 128, 128), r_max=64, S=12, dtype="bf16",
                       with_ranks=True),
        random_problem(rng, T=300, D=1024, out_sizes=(512,), r_max=16, S=40, dtype="f16",
                       bad_idx_frac=0.05),
    ]
    say("[streams] " + "; ".join(f"T={p.T} D={p.D} S={p.S} slices={p.out_sizes} {p.dtype}" for p in probs))
    ds = [problem_to_device(p, "cuda") for p in probs]
    segs = [glsa.alloc_segments(p.T, p.S, "cuda") for p in probs]
    vs = [torch.empty((p.n_slices, p.T, p.r_max), dtype=torch.float32, device="cuda") for p in probs]
    y_in = [d["y"].clone() for d in ds]
    rows = [sample_tokens(probs[0].idx, probs[0].S, 128), np.arange(probs[1].T)]
    refs = [oracle_ref(p, tokens=r) for p, r in zip(probs, rows)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]

    for rep in range(3):
        for d, y0 in zip(ds, y_in):
            d["y"].copy_(y0)
        for v in vs:
            v.fill_(float("nan"))
        for st in streams:
            st.wait_stream(torch.cuda.current_stream())
        # the two batches' calls interleaved, each on its own stream
        for i, p in enumerate(probs):
            glsa.build_segments(ds[i]["idx"], p.S, seg=segs[i], stream=streams[i])
        for i, p in enumerate(probs):
            d = ds[i]
            glsa.shrink(d["x"], d["A"], segs[i], scale=d["scale"], ranks=d["ranks"], v=vs[i], stream=streams[i])
        for i, p in enumerate(probs):
            d = ds[i]
            glsa.expand(vs[i], d["B"], d["y"], segs[i], p.out_offsets, ranks=d["ranks"], stream=streams[i])
        torch.cuda.synchronize()

        for i, p in enumerate(probs):
            v_ref, y_ref = refs[i]
            vg = vs[i].cpu().numpy().astype(np.float64)
            yg = oracle.decode(from_torch(ds[i]["y"], p.dtype), p.dtype)
            ev = rel_err(vg[:, rows[i]], v_ref)
            ey = rel_err(yg[rows[i]], y_ref)
            say(f"[streams] rep {rep} batch {i}: err_y={ey:.3e} err_v={ev:.3e}")
            assert ev <= V_TOL, f"rep {rep} batch {i}: v error {ev:.3e}"
            assert ey <= Y_TOL[p.dtype], f"rep {rep} batch {i}: y error {ey:.3e}"
            valid = (p.idx >= 0) & (p.idx < p.S)
            assert np.array_equal(from_torch(ds[i]["y"], p.dtype)[~valid], p.y_in[~valid]), \
                f"rep {rep} batch {i}: base rows changed"
