"""GPU: the embedding adapter (lora_embedding_shrink, then lora_expand) matches
the fp64 oracle ("Add multi-LoRA support", Features: adapters on the
embeddings as well as on every linear layer): random batches in every dtype
with mixed ranks, base-only tokens, slots and token ids outside their range,
and the Llama-3-8B table (V = 128256, H = 4096) at decode and prefill batch
sizes.  Bars as for the linear layers; rows without a delta stay bit-identical.
"""

import numpy as np
import pytest
import torch

import gemm_lora_shrink_amd as glsa
import oracle
from gpu_util import V_TOL, Y_TOL, rel_err, say
from workloads import random_embedding_problem
from workloads.torch_io import from_torch, to_torch

pytestmark = pytest.mark.gpu


def _device(p):
    return dict(tok=torch.from_numpy(p.tok).cuda(), idx=torch.from_numpy(p.idx).cuda(),
                A=to_torch(p.A_emb, p.dtype, "cuda"), B=to_torch(p.B, p.dtype, "cuda"),
                y=to_torch(p.y_in, p.dtype, "cuda"), scale=torch.from_numpy(p.scale).cuda(),
                ranks=None if p.ranks is None else torch.from_numpy(p.ranks).cuda())


def _check(p, label, rows=None):
    say(f"[embedding] {label}: T={p.T} V={p.V} H={p.H} S={p.S} r_max={p.r_max} dtype={p.dtype}")
    d = _device(p)
    seg = glsa.build_segments(d["idx"], p.S)
    v, y = glsa.embedding_apply(d["tok"], d["A"], d["B"], d["y"], seg, d["idx"], scale=d["scale"],
                                ranks=d["ranks"])
    torch.cuda.synchronize()
    rows = np.arange(p.T) if rows is None else np.asarray(rows)
    v_ref, y_ref = oracle.oracle_embedding_apply(p.tok, p.A_emb, p.B, p.y_in, p.idx, p.S, dtype=p.dtype,
                                                 scale=p.scale, ranks=p.ranks, tokens=rows)
    y_got = from_torch(y, p.dtype)
    ey = rel_err(oracle.decode(y_got[rows], p.dtype), y_ref)
    ev = rel_err(v[0].cpu().numpy()[rows], v_ref)
    say(f"[embedding] {label}: err_y {ey:.3e} err_v {ev:.3e}")
    assert ey <= Y_TOL[p.dtype] and ev <= V_TOL
    dead = ~((p.idx >= 0) & (p.idx < p.S)) | (p.tok < 0) | (p.tok >= p.V)
    assert np.array_equal(y_got[dead], p.y_in[dead]), "rows without a delta changed"
    assert not np.any(v[0].cpu().numpy()[dead]), "v of rows without a delta not zero"


def _cases():
    rng = np.random.default_rng(61)
    for dtype in ("f32", "f16", "bf16"):
        yield f"mixed_{dtype}", random_embedding_problem(
            rng, T=300, V=1000, H=136, r_max=16, S=5, dtype=dtype, with_ranks=True,
            bad_tok_frac=0.05, bad_idx_frac=0.05)
    yield "one_token", random_embedding_problem(rng, T=1, V=3, H=8, r_max=8, S=1, dtype="bf16",
                                                base_frac=0.0)
    yield "rank64_ldy", random_embedding_problem(rng, T=90, V=777, H=256, r_max=64, S=3,
                                                 dtype="f16", ldy=264)


@pytest.mark.parametrize("case", list(_cases()), ids=lambda c: c[0])
def test_embedding_parity(case):
    label, p = case
    _check(p, label)


@pytest.mark.parametrize("T,dtype,r", [(256, "f16", 16), (4096, "bf16", 64)])
def test_embedding_llama3_table(T, dtype, r):
    rng = np.random.default_rng(62)
    p = random_embedding_problem(rng, T=T, V=128256, H=4096, r_max=r, S=8, dtype=dtype,
                                 base_frac=0.1, w_var=0.02)
    rows = np.sort(rng.choice(T, size=min(T, 200), replace=False))
    _check(p, f"llama3_T{T}", rows=rows)


def test_embedding_inactive_is_a_no_op():
    rng = np.random.default_rng(63)
    p = random_embedding_problem(rng, T=64, V=50, H=32, r_max=8, S=2, dtype="bf16", base_frac=1.0)
    d = _device(p)
    v = torch.full((1, p.T, p.r_max), float("nan"), device="cuda")
    v0 = v.clone()
    glsa.embedding_shrink(d["tok"], d["A"], d["idx"], v=v, active=False)
    torch.cuda.synchronize()
    assert torch.equal(v.view(torch.int32), v0.view(torch.int32))
