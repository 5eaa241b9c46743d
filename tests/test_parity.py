"""GPU: shrink + expand match the fp64 oracle on the five workloads and on
edge cases (ragged sizes, base-only and out-of-range tokens, mixed and zero
ranks, strided rows, several and shared slices, every dtype and mode)."""

import numpy as np
import pytest

from gpu_util import check_problem, sample_tokens
from workloads import make_workload, random_problem

pytestmark = pytest.mark.gpu


def _zero_y(p):
    p.y_in = np.zeros_like(p.y_in)
    return p


# --------------------------------------------------------------------------
# the five workloads at full size, in the launch configuration the bench uses
# --------------------------------------------------------------------------

FULL = [("tiny_bgmv", None), ("decode_qproj", None), ("prefill_qkv", 384),
        ("mixed_rank_mlp", None), ("zipf_many", 1024)]


@pytest.mark.parametrize("y_zero", [False, True], ids=["y_random", "y_zero"])
@pytest.mark.parametrize("name,n_sample", FULL, ids=[f[0] for f in FULL])
def test_workload_parity(name, n_sample, y_zero):
    wl = make_workload(name)
    for p in wl.problems:
        if y_zero:
            _zero_y(p)
        tokens = None if n_sample is None else sample_tokens(p.idx, p.S, n_sample)
        check_problem(p, tokens=tokens, label=f"{name}/{p.name}/{'y0' if y_zero else 'y'}")


@pytest.mark.parametrize("mode", ["bgmv", "sgmv"])
@pytest.mark.parametrize("name,n_sample", [("decode_qproj", None), ("mixed_rank_mlp", 256),
                                           ("zipf_many", 512), ("prefill_qkv", 192)],
                         ids=["decode_qproj", "mixed_rank_mlp", "zipf_many", "prefill_qkv"])
def test_workload_parity_forced_mode(name, n_sample, mode):
    wl = make_workload(name)
    for p in wl.problems[:1]:
        tokens = None if n_sample is None else sample_tokens(p.idx, p.S, n_sample)
        check_problem(p, mode=mode, tokens=tokens, label=f"{name}/{p.name}/{mode}")


# --------------------------------------------------------------------------
# edge cases, compared row by row with the oracle
# --------------------------------------------------------------------------

def edge_problems():
    rng = np.random.default_rng(77)
    for dtype in ("f32", "f16", "bf16"):
        yield f"ragged_{dtype}", random_problem(
            rng, T=37, D=96, out_sizes=(40,), r_max=8, S=3, dtype=dtype), "auto"
        yield f"slices3_ranks_{dtype}", random_problem(
            rng, T=300, D=264, out_sizes=(64, 16, 24), r_max=16, S=5, dtype=dtype,
            with_ranks=True), "auto"
        yield f"strided_{dtype}", random_problem(
            rng, T=130, D=128, out_sizes=(32, 48), r_max=8, S=4, dtype=dtype,
            ldx=136, ldy=96), "auto"
        yield f"bad_idx_{dtype}", random_problem(
            rng, T=200, D=64, out_sizes=(64,), r_max=16, S=6, dtype=dtype,
            bad_idx_frac=0.2), "auto"
    for dtype in ("f32", "f16", "bf16"):
        # a batch large enough that the shrink cuts items into token and rank
        # pieces rather than K parts: ragged tiles (48..200 tokens), gather
        # groups of 1..47 tokens, ranks that are not multiples of 16
        idx = np.concatenate([np.repeat(np.arange(6), [100, 64, 63, 200, 48, 49]),
                              np.repeat(np.arange(6, 24), rng.integers(1, 48, 18)),
                              np.full(600, -1)]).astype(np.int32)
        rng.shuffle(idx)
        p = random_problem(rng, T=idx.size, D=256, out_sizes=(128, 64), r_max=64, S=24,
                           dtype=dtype, idx=idx, with_ranks=True)
        p.ranks[:] = rng.integers(1, 65, 24)
        yield f"pieces_{dtype}", p, "auto"
    for dtype, n_sl, r_max in (("bf16", 3, 64), ("f16", 2, 32), ("f16", 3, 32), ("bf16", 2, 64)):
        # >= 4096 tokens, two or three slices of rank 32 or 64, 16-bit (the
        # shape of fused q/k/v and gate/up prefill): ragged tiles, gather
        # groups beside them, a K tail (D = 520 is not a whole number of
        # 64-element batches), strided x rows, mixed ranks with one slot of
        # rank 0, base tokens.
        counts = [900, 700, 651, 500, 480, 64, 63, 48, 47, 20, 5, 1]
        idx = np.concatenate([np.repeat(np.arange(12), counts), np.full(700, -1)]).astype(np.int32)
        rng.shuffle(idx)
        p = random_problem(rng, T=idx.size, D=520, out_sizes=(64, 32, 48)[:n_sl], r_max=r_max, S=12,
                           dtype=dtype, idx=idx, with_ranks=True, ldx=528)
        p.ranks[:] = rng.integers(1, r_max + 1, 12)
        p.ranks[4] = 0
        yield f"large_slices{n_sl}_r{r_max}_{dtype}", p, "auto"
    # the same with a longer contraction and a tail
    yield "large_slices3_long_K", random_problem(
        rng, T=4100, D=2056, out_sizes=(128, 64, 64), r_max=64, S=3, dtype="bf16",
        with_ranks=True), "auto"
    for mode in ("auto", "bgmv", "sgmv"):
        # long segments (>= 48 tokens go to the segmented path in auto mode)
        idx = np.repeat(np.arange(5, dtype=np.int32), [200, 64, 63, 1, 130])
        idx[::7] = -1
        yield f"long_segments_{mode}", random_problem(
            rng, T=idx.size, D=512, out_sizes=(256, 64), r_max=32, S=5, dtype="bf16",
            idx=idx, with_ranks=True), mode
        yield f"wide_D_{mode}", random_problem(
            rng, T=90, D=14336, out_sizes=(128,), r_max=64, S=2, dtype="f16",
            with_ranks=True), mode
    # mid-size batch with a long contraction: cut along K with atomics
    yield "long_K_mid_size", random_problem(
        rng, T=1000, D=8192, out_sizes=(64,), r_max=64, S=20, dtype="bf16",
        with_ranks=True), "auto"
    yield "one_token", random_problem(rng, T=1, D=8, out_sizes=(8,), r_max=8, S=1,
                                      dtype="f16", base_frac=0.0), "auto"
    yield "all_base_active_hint", random_problem(
        rng, T=64, D=64, out_sizes=(64,), r_max=8, S=2, dtype="bf16", base_frac=1.0), "auto"
    yield "max_rank_8_slices", random_problem(
        rng, T=70, D=64, out_sizes=(8,) * 8, r_max=64, S=3, dtype="bf16"), "auto"
    yield "many_slots", random_problem(
        rng, T=2000, D=64, out_sizes=(32,), r_max=8, S=1024, dtype="f16"), "auto"
    p = random_problem(rng, T=50, D=32, out_sizes=(16,), r_max=8, S=3, dtype="f32",
                       with_ranks=True)
    p.ranks[:] = [0, 3, 8]
    yield "rank_zero", p, "auto"
    for mode in ("auto", "bgmv", "sgmv"):
        # fp32 rows of r_max = 12 (a multiple of 4, not of 8): v rows end
        # halfway through the kernels' 8-float pieces; long and short segments,
        # the last token of the last slice on a slot of full rank
        idx = np.repeat(np.arange(4, dtype=np.int32), [70, 9, 40, 31])
        p = random_problem(rng, T=idx.size, D=72, out_sizes=(24, 40), r_max=12, S=4, dtype="f32",
                           idx=idx, with_ranks=True)
        p.ranks[:] = [5, 12, 8, 12]
        yield f"rmax12_f32_{mode}", p, mode


@pytest.mark.parametrize("case", list(edge_problems()), ids=lambda c: c[0])
def test_edge_parity(case):
    label, p, mode = case
    rng = np.random.default_rng(3)
    # garbage in the rank padding must be ignored
    if p.ranks is not None:
        for s, r in enumerate(p.ranks):
            for a in p.A:
                a[s, r:, :] = a.dtype.type(7) if a.dtype != np.uint16 else np.uint16(0x40e0)
            for b in p.B:
                b[s, :, r:] = b.dtype.type(7) if b.dtype != np.uint16 else np.uint16(0x40e0)
    check_problem(p, mode=mode, label=label)


def test_shared_v_across_slices():
    rng = np.random.default_rng(8)
    p = random_problem(rng, T=120, D=128, out_sizes=(32, 64, 16), r_max=16, S=3,
                       dtype="bf16")
    check_problem(p, shared_v=True, label="shared_v")


def test_empty_batch():
    rng = np.random.default_rng(9)
    p = random_problem(rng, T=0, D=64, out_sizes=(32,), r_max=8, S=2, dtype="f16")
    check_problem(p, label="empty")
