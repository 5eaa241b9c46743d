"""Helpers for the GPU parity tests: run the HIP library on a workloads.Problem
and compare with the oracle.  Tolerances are the stated bars:

  y:  max|y_gpu - y_ref| / max|y_ref| <= 5e-3 (fp16), 2e-2 (bf16), 1e-5 (fp32)
      where y_ref is the fp64 oracle output (the whole output row set compared)
  v:  max|v_gpu - v_ref| / max|v_ref| <= 1e-4 for every dtype, which an fp32
      intermediate meets (~1e-6) and a 16-bit one (~2e-4 to 2e-3) does not
"""

import sys

import numpy as np
import torch

import gemm_lora_shrink_amd as glsa
import oracle
from workloads.torch_io import from_torch, problem_to_device

Y_TOL = {"f32": 1e-5, "f16": 5e-3, "bf16": 2e-2}
V_TOL = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    den = float(np.max(np.abs(ref)))
    num = float(np.max(np.abs(got - ref)))
    if den == 0.0:
        return num
    return num / den


def fused_counter_bytes(ws):
    """Bytes at the start of a shrink_expand workspace that every call leaves
    zero: the 256-byte header and the counter region (the workspace's first
    quarter, after the header)."""
    return 256 + ws.numel() // 4


def run_fused(p, d, seg, ws=None, from_idx=False):
    """shrink_expand on device tensors d; checks the workspace is left clean.
    from_idx: pass the batch's idx, so that a one-launch call groups the
    tokens itself instead of reading the record."""
    v = torch.full((p.n_slices, p.T, p.r_max), float("nan"), dtype=torch.float32, device=d["x"].device)
    if ws is None:
        ws = glsa.alloc_workspace(p.T, p.S, p.n_slices, p.r_max, d["x"].device)
    glsa.shrink_expand(d["x"], d["A"], d["B"], d["y"], seg, p.out_offsets, workspace=ws,
                       scale=d["scale"], ranks=d["ranks"], v=v,
                       idx=d["idx"] if from_idx else None)
    torch.cuda.synchronize()
    assert glsa.workspace_errors(ws) == 0, "a fused wait gave up"
    if p.T > 0:
        assert not torch.any(ws[:fused_counter_bytes(ws)]).item(), "fused counters not back at zero"
    return v


def run_gpu(p, *, mode="auto", device="cuda", shared_v=False, fused=False):
    """Build segments, shrink and expand on the GPU.  Returns (v, y, info).
    fused: False, "record" (shrink_expand reading the record) or "idx"
    (shrink_expand grouping the tokens itself where it runs as one launch)."""
    d = problem_to_device(p, device)
    seg = glsa.build_segments(d["idx"], p.S, mode=mode)
    if fused:
        v = run_fused(p, d, seg, from_idx=fused == "idx")
    elif shared_v:
        v = glsa.shrink(d["x"], d["A"][:1], seg, scale=d["scale"], ranks=d["ranks"])
        glsa.expand(v, d["B"], d["y"], seg, p.out_offsets, ranks=d["ranks"], v_slice_stride=0)
    else:
        v = glsa.shrink(d["x"], d["A"], seg, scale=d["scale"], ranks=d["ranks"])
        glsa.expand(v, d["B"], d["y"], seg, p.out_offsets, ranks=d["ranks"])
    torch.cuda.synchronize()
    info = seg[:16].cpu().numpy()
    return v.cpu().numpy().astype(np.float64), from_torch(d["y"], p.dtype), info


def oracle_ref(p, tokens=None, shared_v=False):
    A = p.A[:1] if shared_v else p.A
    v = oracle.oracle_shrink(p.x, A, p.idx, p.S, dtype=p.dtype, D=p.D, scale=p.scale,
                             ranks=p.ranks, tokens=tokens)
    if shared_v:
        v = np.repeat(v, p.n_slices, axis=0)
    y = oracle.oracle_expand(v, p.B, p.y_in, p.idx, p.S, p.out_offsets, dtype=p.dtype,
                             ranks=p.ranks, tokens=tokens)
    return v, y


def check_problem(p, *, mode="auto", tokens=None, shared_v=False, fused=False, label=""):
    """Run the GPU path on p and assert parity with the oracle.

    tokens: None compares every row; otherwise only those rows are compared
    with the oracle, while the properties that hold at any size (base rows
    bit-identical, v zero outside active rows/ranks) are checked on all rows.
    """
    say(f"[parity] {label} dtype={p.dtype} T={p.T} D={p.D} S={p.S} r_max={p.r_max} "
        f"slices={p.out_sizes} mode={mode}{' fused' if fused else ''}")
    v_gpu, y_gpu, info = run_gpu(p, mode=mode, shared_v=shared_v, fused=fused)
    rows = np.arange(p.T) if tokens is None else np.asarray(tokens)
    v_ref, y_ref = oracle_ref(p, tokens=None if tokens is None else rows, shared_v=shared_v)
    y_got = oracle.decode(y_gpu[rows], p.dtype)
    ey = rel_err(y_got, y_ref)
    n_v = 1 if shared_v else p.n_slices
    ev = rel_err(v_gpu[:n_v][:, rows], v_ref[:n_v])
    say(f"[parity] {label} err_y={ey:.3e} (bar {Y_TOL[p.dtype]:.0e}) err_v={ev:.3e} (bar {V_TOL:.0e})")
    assert ey <= Y_TOL[p.dtype], f"{label}: y error {ey:.3e}"
    assert ev <= V_TOL, f"{label}: v error {ev:.3e}"

    # properties over all rows
    valid = (p.idx >= 0) & (p.idx < p.S)
    assert np.array_equal(y_gpu[~valid], p.y_in[~valid]), f"{label}: base rows changed"
    assert not np.any(v_gpu[:n_v][:, ~valid]), f"{label}: v of base rows not zero"
    if p.ranks is not None:
        rk = np.where(valid, p.ranks[np.clip(p.idx, 0, p.S - 1)], 0)
        cols = np.arange(p.r_max)[None, :] >= rk[:, None]
        assert not np.any(v_gpu[:n_v][:, cols]), f"{label}: v past rank not zero"
    # columns of y outside every slice are never written
    inside = np.zeros(p.ldy, dtype=bool)
    for off, w in zip(p.out_offsets, p.out_sizes):
        inside[off:off + w] = True
    assert np.array_equal(y_gpu[:, ~inside], p.y_in[:, ~inside]), f"{label}: padding columns changed"
    return ey, ev, info


def sample_tokens(idx, S, n_random, seed=0):
    """First and last token of every slot, some base tokens, and random tokens."""
    rng = np.random.default_rng(seed)
    T = idx.shape[0]
    picks = set()
    for s in np.unique(idx):
        where = np.nonzero(idx == s)[0]
        picks.update([int(where[0]), int(where[-1])])
    picks.update(int(t) for t in rng.choice(T, size=min(n_random, T), replace=False))
    return np.array(sorted(picks))
