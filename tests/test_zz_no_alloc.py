"""GPU: lora_shrink_expand_noalloc, the variant for callers that cannot
allocate, gives the output of lora_shrink_expand on the same inputs.

Two calls in a row on the variant's per-device scratch, the second on a
smaller batch, each compared with lora_shrink_expand on a workspace of its
own: to the oracle's bars (max relative error against the fp64 oracle, v to
1e-4) and, where both run the deterministic one-launch form, bit for bit.
Also: the give-up count copied to host is 0, the scratch's counters were left
at zero by the first call (the second call, which relies on that, is right),
and a call needing more scratch than the limit is refused before anything is
enqueued.
"""

import numpy as np
import pytest
import torch

import gemm_lora_shrink_amd as glsa
from gpu_util import V_TOL, Y_TOL, oracle_ref, rel_err, say
from workloads import random_problem
from workloads.torch_io import from_torch, problem_to_device
import oracle

pytestmark = pytest.mark.gpu


def _both(p, from_idx):
    """(y, v) from lora_shrink_expand and from lora_shrink_expand_noalloc."""
    out = []
    for variant in ("workspace", "noalloc"):
        d = problem_to_device(p, "cuda")
        seg = glsa.build_segments(d["idx"], p.S)
        v = torch.full((p.n_slices, p.T, p.r_max), float("nan"), dtype=torch.float32, device="cuda")
        idx = d["idx"] if from_idx else None
        if variant == "workspace":
            ws = glsa.alloc_workspace(p.T, p.S, p.n_slices, p.r_max, "cuda")
            glsa.shrink_expand(d["x"], d["A"], d["B"], d["y"], seg, p.out_offsets, workspace=ws,
                               scale=d["scale"], ranks=d["ranks"], v=v, idx=idx)
        else:
            err = torch.full((1,), -1, dtype=torch.int32).pin_memory()
            glsa.shrink_expand_noalloc(d["x"], d["A"], d["B"], d["y"], seg, p.out_offsets,
                                       scale=d["scale"], ranks=d["ranks"], v=v, idx=idx,
                                       errors_host=err)
        torch.cuda.synchronize()
        if variant == "noalloc":
            assert int(err[0]) == 0, "a wait gave up in the allocation-free call"
        out.append((from_torch(d["y"], p.dtype), v.cpu().numpy().astype(np.float64)))
    return out


def _problems(seed):
    rng = np.random.default_rng(seed)
    big = random_problem(rng, T=700, D=1024, out_sizes=(512, 256), r_max=32, S=9, dtype="bf16",
                         with_ranks=True, base_frac=0.2)
    small = random_problem(rng, T=40, D=256, out_sizes=(128,), r_max=16, S=3, dtype="f16",
                           base_frac=0.3)
    return big, small


@pytest.mark.parametrize("from_idx", [False, True], ids=["record", "idx"])
def test_noalloc_matches_workspace_call_twice(from_idx):
    big, small = _problems(5 if from_idx else 4)
    for label, p in (("first", big), ("second, smaller", small)):
        say(f"[noalloc] {label}: T={p.T} D={p.D} slices={p.out_sizes} dtype={p.dtype} "
            f"{'idx' if from_idx else 'record'} form")
        (y_ws, v_ws), (y_na, v_na) = _both(p, from_idx)
        v_ref, y_ref = oracle_ref(p)
        assert rel_err(oracle.decode(y_na, p.dtype), y_ref) <= Y_TOL[p.dtype]
        assert rel_err(v_na, v_ref) <= V_TOL
        assert rel_err(oracle.decode(y_na, p.dtype), oracle.decode(y_ws, p.dtype)) <= Y_TOL[p.dtype]
        # both run the same one launch: sums in the same order, same bits
        assert np.array_equal(y_na, y_ws), f"{label}: y differs from lora_shrink_expand's"
        assert np.array_equal(v_na, v_ws), f"{label}: v differs from lora_shrink_expand's"


def test_noalloc_two_launch_forms():
    """Batches past the one-launch limits (4096 tokens of 16-bit data, 2048
    of fp32) run as separate launches on the scratch (v kept in it when the
    caller passes none)."""
    rng = np.random.default_rng(6)
    cases = [random_problem(rng, T=4200, D=256, out_sizes=(128,), r_max=16, S=40, dtype="f16"),
             random_problem(rng, T=2100, D=128, out_sizes=(64,), r_max=8, S=5, dtype="f32")]
    for p in cases:
        say(f"[noalloc] two launches: T={p.T} dtype={p.dtype}")
        (y_ws, _), (y_na, v_na) = _both(p, from_idx=True)
        v_ref, y_ref = oracle_ref(p)
        assert rel_err(oracle.decode(y_na, p.dtype), y_ref) <= Y_TOL[p.dtype]
        assert rel_err(v_na, v_ref) <= V_TOL
        assert rel_err(oracle.decode(y_na, p.dtype), oracle.decode(y_ws, p.dtype)) <= Y_TOL[p.dtype]


def test_noalloc_refuses_calls_past_the_scratch():
    rng = np.random.default_rng(7)
    p = random_problem(rng, T=64, D=64, out_sizes=(64,), r_max=64, S=4, dtype="bf16")
    d = problem_to_device(p, "cuda")
    seg = glsa.build_segments(d["idx"], p.S)
    y0 = d["y"].clone()
    torch.cuda.synchronize()
    # a shape whose workspace exceeds the scratch: 8 slices of a large batch
    T_big = 16384
    assert glsa.workspace_bytes(T_big, 4, 8, 64) > glsa.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T_big, 64), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((T_big, 8 * 64), dtype=torch.bfloat16, device="cuda")
    A = [d["A"][0]] * 8
    B = [d["B"][0]] * 8
    seg_big = glsa.alloc_segments(T_big, p.S, "cuda")
    with pytest.raises(glsa.LoraError) as e:
        glsa.shrink_expand_noalloc(x, A, B, y, seg_big, [64 * i for i in range(8)])
    assert e.value.status == glsa.LORA_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.equal(d["y"].view(torch.int16), y0.view(torch.int16))


def test_noalloc_fp32_one_launch():
    """fp32 batches of up to 2048 tokens run as the one launch too (their
    chunks expanded on the vector ALUs), here on the scratch, in both forms."""
    rng = np.random.default_rng(8)
    p = random_problem(rng, T=300, D=128, out_sizes=(96,), r_max=16, S=6, dtype="f32", with_ranks=True)
    v_ref, y_ref = oracle_ref(p)
    for from_idx in (False, True):
        say(f"[noalloc] fp32 one launch: T={p.T} {'idx' if from_idx else 'record'} form")
        (y_ws, v_ws), (y_na, v_na) = _both(p, from_idx)
        assert rel_err(oracle.decode(y_na, p.dtype), y_ref) <= Y_TOL[p.dtype]
        assert rel_err(v_na, v_ref) <= V_TOL
        assert np.array_equal(y_na, y_ws), "fp32: y differs from lora_shrink_expand's"
        assert np.array_equal(v_na, v_ws), "fp32: v differs from lora_shrink_expand's"
