"""CPU tests of the seeded input generators (no LoRA arithmetic lives there)."""

import numpy as np
import pytest
import torch

from workloads import CONFIGS, make_workload, random_problem, round_to_dtype, bf16_bits_to_f32


def test_bf16_rounding_matches_torch():
    """Our bit-level round-to-nearest-even agrees with torch's CPU bf16 cast."""
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.normal(size=20000).astype(np.float32),
                        np.float32([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, 1e-30])])
    # exact ties of the 16-bit truncation (odd and even lower neighbour)
    ties = (np.arange(1, 200, dtype=np.uint32) << 16 | np.uint32(0x8000)).view(np.float32)
    a = np.concatenate([a, ties, -ties])
    ours = round_to_dtype(a, "bf16")
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_fp16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    a = rng.normal(size=10000) * 100
    ours = round_to_dtype(a, "f16")
    ref = torch.from_numpy(a.astype(np.float32)).half().numpy()
    # fp64 -> fp16 directly vs fp64 -> fp32 -> fp16 can differ only on double
    # rounding ties, which a normal draw does not hit at this size.
    assert np.array_equal(ours, ref)


def test_deterministic_and_seeded():
    a = make_workload("tiny_bgmv")
    b = make_workload("tiny_bgmv")
    c = make_workload("tiny_bgmv", seed=1)
    assert np.array_equal(a.idx, b.idx)
    assert np.array_equal(a.problems[0].x, b.problems[0].x)
    assert not np.array_equal(a.problems[0].x, c.problems[0].x)


@pytest.mark.parametrize("name", ["tiny_bgmv", "decode_qproj", "zipf_many", "zipf_many_noop"])
def test_shapes_and_idx_recipes(name):
    c = CONFIGS[name]
    wl = make_workload(name)
    T, S = c["T"], c["S"]
    assert wl.idx.shape == (T,) and wl.idx.dtype == np.int32
    assert wl.idx.min() >= -1 and wl.idx.max() < S
    for p, pc in zip(wl.problems, c["problems"]):
        assert p.x.shape == (T, pc["D"])
        for a, b, o in zip(p.A, p.B, pc["out_sizes"]):
            assert a.shape == (S, c["r_max"], pc["D"])
            assert b.shape == (S, o, c["r_max"])
        assert p.y_in.shape == (T, sum(pc["out_sizes"]))
    kind = c["idx"][0]
    if kind == "uniform_then_base":
        assert int((wl.idx == -1).sum()) == c["idx"][2]
    if kind == "all_base":
        assert np.all(wl.idx == -1)
    if kind == "zipf":
        counts = np.bincount(wl.idx, minlength=S)
        # slot 0 holds about 22.6% of the tokens under Zipf(1.1) over 128 slots
        assert 0.19 < counts[0] / T < 0.26
        assert counts[0] == counts.max()


def test_decode_qproj_variances():
    """Second argument of N(0, s) is read as a variance."""
    p = make_workload("decode_qproj").problems[0]
    a = p.A[0].astype(np.float64)
    assert abs(a.std() - 1 / 64) < 1e-3          # N(0, 1/4096)
    assert abs(p.B[0].astype(np.float64).std() - 0.1) < 2e-3   # N(0, 0.01)
    assert abs(p.x.astype(np.float64).std() - 1.0) < 1e-2


def test_mixed_rank_padding():
    wl = make_workload("mixed_rank_mlp")
    ranks = wl.problems[0].ranks
    assert set(np.unique(ranks)) <= {8, 16, 32, 64}
    for p in wl.problems:
        for a in p.A:
            for s, r in enumerate(ranks):
                assert not np.any(a[s, r:]) and np.any(a[s, :r])
        for b in p.B:
            for s, r in enumerate(ranks):
                assert not np.any(b[s, :, r:])
    assert int((wl.idx == -1).sum()) == 512


def test_random_problem_strides_and_bad_index():
    rng = np.random.default_rng(3)
    p = random_problem(rng, T=50, D=10, out_sizes=(3, 4), r_max=4, S=3, ldx=16,
                       ldy=9, bad_idx_frac=0.3)
    assert p.x.shape == (50, 16) and not np.any(p.x[:, 10:])
    assert p.y_in.shape == (50, 9)
    assert np.any((p.idx < -1) | (p.idx >= 3))
