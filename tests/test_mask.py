"""GPU: the mask ("laning") form of shrink + expand matches the fp64 oracle.

"[Hardware][TPU][V1] Better tpu multilora compilation" reports a masked
formulation beating the per-token gather on TPU and LoRA laning cutting the
number of matrix products.  lora_shrink_expand_mask computes every token's
product with all stacked adapter lanes (S * r_max <= 128) and keeps its own;
its result is the same method's, so it is held to the same bars as the gather
path: the two decode workloads (tiny_bgmv in fp32, decode_qproj in fp16, S *
r_max = 32 and 128), ragged batches, base-only and out-of-range slots, mixed
ranks with garbage past them, strided rows and several slices, and the
once-rounded precision check with y_in = 0."""

import numpy as np
import pytest
import torch

import gemm_lora_shrink_amd as glsa
import oracle
from gpu_util import V_TOL, Y_TOL, oracle_ref, rel_err, say
from precision_util import once_rounded_match, precision_ok, slice_columns, storage_bits
from workloads import make_workload, random_problem
from workloads.torch_io import from_torch, problem_to_device

pytestmark = pytest.mark.gpu


def run_mask(p):
    d = problem_to_device(p, "cuda")
    ws = glsa.alloc_mask_workspace(d["x"].dtype, p.T, p.D, p.S, p.n_slices, p.r_max, "cuda")
    v = torch.full((p.n_slices, p.T, p.r_max), float("nan"), dtype=torch.float32, device="cuda")
    glsa.shrink_expand_mask(d["x"], d["A"], d["B"], d["y"], d["idx"], p.out_offsets, workspace=ws,
                            scale=d["scale"], ranks=d["ranks"], v=v)
    torch.cuda.synchronize()
    return v.cpu().numpy().astype(np.float64), from_torch(d["y"], p.dtype)


def check(p, label):
    say(f"[mask] {label}: T={p.T} D={p.D} S={p.S} r_max={p.r_max} slices={p.out_sizes} dtype={p.dtype}")
    v, y = run_mask(p)
    v_ref, y_ref = oracle_ref(p)
    ey = rel_err(oracle.decode(y, p.dtype), y_ref)
    ev = rel_err(v, v_ref)
    say(f"[mask] {label}: err_y {ey:.3e} err_v {ev:.3e}")
    assert ey <= Y_TOL[p.dtype] and ev <= V_TOL
    valid = (p.idx >= 0) & (p.idx < p.S)
    assert np.array_equal(y[~valid], p.y_in[~valid]), "base rows changed"
    assert not np.any(v[:, ~valid]), "v of base rows not zero"
    inside = slice_columns(p)
    assert np.array_equal(y[:, ~inside], p.y_in[:, ~inside]), "padding columns changed"
    return v, y


@pytest.mark.parametrize("name", ["tiny_bgmv", "decode_qproj"])
def test_mask_decode_workloads(name):
    for p in make_workload(name).problems:
        check(p, name)


def _cases():
    rng = np.random.default_rng(71)
    for dtype in ("f32", "f16", "bf16"):
        yield f"ragged_{dtype}", random_problem(rng, T=45, D=264, out_sizes=(72,), r_max=8, S=5,
                                                dtype=dtype, bad_idx_frac=0.1)
        p = random_problem(rng, T=130, D=512, out_sizes=(256, 64), r_max=32, S=4, dtype=dtype,
                           with_ranks=True, ldx=520, ldy=336)
        yield f"ranks_strided_{dtype}", p
    yield "one_token", random_problem(rng, T=1, D=16, out_sizes=(16,), r_max=16, S=8, dtype="bf16",
                                      base_frac=0.0)
    yield "lanes128_long_D", random_problem(rng, T=200, D=14336, out_sizes=(512,), r_max=64, S=2,
                                            dtype="f16", with_ranks=True)
    yield "all_base", random_problem(rng, T=64, D=64, out_sizes=(64,), r_max=8, S=2, dtype="f16",
                                     base_frac=1.0)


@pytest.mark.parametrize("case", list(_cases()), ids=lambda c: c[0])
def test_mask_parity(case):
    label, p = case
    if p.ranks is not None:  # garbage past every rank must be ignored
        for s, r in enumerate(p.ranks):
            for a in p.A:
                a[s, r:, :] = a.dtype.type(7) if a.dtype != np.uint16 else np.uint16(0x40e0)
            for b in p.B:
                b[s, :, r:] = b.dtype.type(7) if b.dtype != np.uint16 else np.uint16(0x40e0)
    check(p, label)


def test_mask_output_is_once_rounded_oracle():
    p = make_workload("decode_qproj").problems[0]
    p.y_in = np.zeros_like(p.y_in)
    _, y = run_mask(p)
    rows = np.nonzero((p.idx >= 0) & (p.idx < p.S))[0]
    _, y_ref = oracle_ref(p, tokens=rows)
    res = once_rounded_match(storage_bits(y[rows], p.dtype), y_ref, p.dtype, slice_columns(p))
    say(f"[mask] decode_qproj once-rounded: {res}")
    assert precision_ok(res)


def test_mask_refuses_too_many_lanes():
    rng = np.random.default_rng(72)
    p = random_problem(rng, T=32, D=64, out_sizes=(64,), r_max=64, S=3, dtype="f16")
    assert glsa.mask_workspace_bytes(torch.float16, p.T, p.D, p.S, 1, p.r_max) == 0
    d = problem_to_device(p, "cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(glsa.LoraError) as e:
        glsa.shrink_expand_mask(d["x"], d["A"], d["B"], d["y"], d["idx"], p.out_offsets, workspace=ws)
    assert e.value.status == glsa.LORA_ERR_UNSUPPORTED
