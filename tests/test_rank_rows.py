"""GPU: B stored in the rank-rows layout (each slot's rows packed with the
stride of its rank rounded up to a 16-byte piece) gives the oracle's result
on every expand path: shrink then expand (MFMA groups and tiles, the fp32
gather kernel), the one-launch shrink_expand reading the record or grouping
from idx, and the allocation-free call.  "Add multi-LoRA support", Features:
adapters of different ranks (to be made more performant); low-rank slots are
then read without their padding.  NaN is written between each slot's rank and
its stride and past its packed rows: a path that touched them would fail."""

import numpy as np
import pytest
import torch

import gemm_lora_shrink_amd as glsa
import oracle
from gpu_util import V_TOL, Y_TOL, oracle_ref, rel_err, sample_tokens, say
from workloads import make_workload, random_problem
from workloads.torch_io import from_torch, problem_to_device

pytestmark = pytest.mark.gpu

NAN16 = {"f16": 0x7E00, "bf16": 0x7FC0}


def packed_with_garbage(b, ranks, dtype):
    """pack_b_rank_rows(b), then NaN wherever the layout leaves a hole."""
    bp = glsa.pack_b_rank_rows(b, ranks)
    torch.cuda.synchronize()
    h = bp.cpu().contiguous()
    flat = h.view(h.shape[0], -1)
    S, out, r_max = b.shape
    unit = 4 if dtype == "f32" else 8
    nan = torch.tensor(float("nan"), dtype=h.dtype)
    for s in range(S):
        r = int(ranks[s])
        ld = min(r_max, max(unit, -(-r // unit) * unit))
        rows = flat[s, :out * ld].view(out, ld)
        rows[:, r:] = nan
        flat[s, out * ld:] = nan
    return h.to(b.device)


def run(p, path):
    d = problem_to_device(p, "cuda")
    B = [packed_with_garbage(b, p.ranks, p.dtype) for b in d["B"]]
    seg = glsa.build_segments(d["idx"], p.S)
    v = torch.full((p.n_slices, p.T, p.r_max), float("nan"), dtype=torch.float32, device="cuda")
    kw = dict(scale=d["scale"], ranks=d["ranks"], v=v, b_layout="rank_rows")
    if path == "split":
        glsa.shrink(d["x"], d["A"], seg, scale=d["scale"], ranks=d["ranks"], v=v)
        glsa.expand(v, B, d["y"], seg, p.out_offsets, ranks=d["ranks"], b_layout="rank_rows")
    elif path == "noalloc":
        glsa.shrink_expand_noalloc(d["x"], d["A"], B, d["y"], seg, p.out_offsets, idx=d["idx"], **kw)
    else:
        ws = glsa.alloc_workspace(p.T, p.S, p.n_slices, p.r_max, "cuda")
        glsa.shrink_expand(d["x"], d["A"], B, d["y"], seg, p.out_offsets, workspace=ws,
                           idx=d["idx"] if path == "idx" else None, **kw)
        torch.cuda.synchronize()
        assert glsa.workspace_errors(ws) == 0
    torch.cuda.synchronize()
    return v.cpu().numpy().astype(np.float64), from_torch(d["y"], p.dtype)


def check(p, path, label, tokens=None):
    say(f"[rank rows] {label} {path}: T={p.T} D={p.D} ranks={sorted(set(p.ranks.tolist()))} dtype={p.dtype}")
    v, y = run(p, path)
    rows = np.arange(p.T) if tokens is None else np.asarray(tokens)
    v_ref, y_ref = oracle_ref(p, tokens=None if tokens is None else rows)
    ey = rel_err(oracle.decode(y[rows], p.dtype), y_ref)
    ev = rel_err(v[:, rows], v_ref)
    say(f"[rank rows] {label} {path}: err_y {ey:.3e} err_v {ev:.3e}")
    assert ey <= Y_TOL[p.dtype] and ev <= V_TOL
    valid = (p.idx >= 0) & (p.idx < p.S)
    assert np.array_equal(y[~valid], p.y_in[~valid])


def _cases():
    rng = np.random.default_rng(81)
    for dtype in ("f32", "f16", "bf16"):
        p = random_problem(rng, T=300, D=264, out_sizes=(64, 16, 24), r_max=64, S=6, dtype=dtype,
                           with_ranks=True)
        p.ranks[:] = [1, 8, 13, 32, 50, 64]
        yield f"ranks_{dtype}", p
    # long segments (tiles) and short ones (groups), ranks 8..64
    idx = np.repeat(np.arange(5, dtype=np.int32), [200, 64, 9, 1, 130])
    p = random_problem(rng, T=idx.size, D=512, out_sizes=(512, 256), r_max=64, S=5, dtype="bf16",
                       idx=idx, with_ranks=True)
    p.ranks[:] = [8, 16, 32, 64, 24]
    yield "tiles_and_groups", p


PATHS = ["split", "record", "idx", "noalloc"]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("case", list(_cases()), ids=lambda c: c[0])
def test_rank_rows_parity(case, path):
    label, p = case
    check(p, path, label)


@pytest.mark.parametrize("path", ["split", "idx"])
def test_rank_rows_mixed_rank_mlp(path):
    for p in make_workload("mixed_rank_mlp").problems:
        check(p, path, f"mixed_rank_mlp/{p.name}", tokens=sample_tokens(p.idx, p.S, 256))
