"""GPU: batches served through the adapter cache ("Add multi-LoRA support",
Features: a fixed number of GPU slots behind an LRU host tier, adapters of
different ranks, every linear layer and the embeddings) give the oracle's
result computed from each token's own adapter.

A pool of adapters of ranks 8..64 runs through a cache of 4 slots and a CPU
tier of 6 over several batches, so that slots are reused by adapters of other
ranks; every batch applies two linear layers (one with two slices) and the
embedding from the cache's stacked tensors and is compared with the oracle on
stacks built directly from the batch's adapters."""

import numpy as np
import pytest
import torch

import gemm_lora_shrink_amd as glsa
import oracle
from gemm_lora_shrink_amd.slots import HostAdapter, SlotCache
from gpu_util import V_TOL, Y_TOL, rel_err, say
from workloads import round_to_dtype
from workloads.torch_io import from_torch, to_torch

pytestmark = pytest.mark.gpu

LAYERS = {"q_proj": (512, (512,)), "gate_up_proj": (512, (384, 384))}
V, H = 1000, 256
R_MAX = 64
DT = "bf16"
TORCH_DT = torch.bfloat16


def adapter(name, rank):
    rng = np.random.default_rng(1000 + name)

    def t(shape):
        return torch.from_numpy(round_to_dtype(rng.normal(0, 0.1, shape), "f32"))
    layers = {ln: [(t((rank, D)), t((o, rank))) for o in outs] for ln, (D, outs) in LAYERS.items()}
    return HostAdapter(name=name, rank=rank, scale=16.0 / rank, layers=layers,
                       embedding=(t((rank, V)), t((H, rank))))


RANKS = {n: (8, 16, 32, 64)[n % 4] for n in range(10)}


def _bits(t):
    return round_to_dtype(t.numpy().astype(np.float64), DT)


def test_cache_serves_batches_like_the_oracle():
    cache = SlotCache(LAYERS, 4, R_MAX, TORCH_DT, "cuda", cpu_capacity=6,
                      loader=lambda n: adapter(n, RANKS[n]), embedding=(V, H))
    rng = np.random.default_rng(9)
    T = 96
    for b in range(6):
        pool = rng.choice(10, size=4, replace=False)
        names = [None if rng.random() < 0.2 else int(rng.choice(pool)) for _ in range(T)]
        idx = cache.slots_for(names)
        say(f"[slots] batch {b}: adapters {sorted(set(n for n in names if n is not None))}, "
            f"resident {dict(cache.resident())}")
        seg = glsa.build_segments(idx, cache.n_slots)
        # oracle stacks: slot j of the batch's own list, independent of the cache
        own = sorted(set(n for n in names if n is not None))
        oidx = np.array([own.index(n) if n is not None else -1 for n in names], np.int32)
        S_o = max(1, len(own))
        ranks_o = np.array([RANKS[n] for n in own] + [1] * (S_o - len(own)), np.int32)
        scale_o = np.array([16.0 / RANKS[n] for n in own] + [1.0] * (S_o - len(own)), np.float32)
        ads = [adapter(n, RANKS[n]) for n in own]
        for ln, (D, outs) in LAYERS.items():
            x = round_to_dtype(rng.normal(0, 1, (T, D)), DT)
            y_in = round_to_dtype(rng.normal(0, 1, (T, sum(outs))), DT)
            xd, yd = to_torch(x, DT, "cuda"), to_torch(y_in, DT, "cuda")
            ws = glsa.alloc_workspace(T, cache.n_slots, len(outs), R_MAX, "cuda")
            v = torch.empty((len(outs), T, R_MAX), dtype=torch.float32, device="cuda")
            offs = list(np.concatenate([[0], np.cumsum(outs)[:-1]]).astype(int))
            glsa.shrink_expand(xd, cache.A[ln], cache.B[ln], yd, seg, offs, workspace=ws, scale=cache.scale,
                               ranks=cache.ranks, v=v)
            A_o = [np.zeros((S_o, R_MAX, D), np.uint16) for _ in outs]
            B_o = [np.zeros((S_o, o, R_MAX), np.uint16) for o in outs]
            for j, a in enumerate(ads):
                for i in range(len(outs)):
                    A_o[i][j, :a.rank] = _bits(a.layers[ln][i][0])
                    B_o[i][j, :, :a.rank] = _bits(a.layers[ln][i][1])
            v_ref, y_ref = oracle.oracle_apply(x, A_o, B_o, y_in, oidx, S_o, offs, dtype=DT, scale=scale_o,
                                               ranks=ranks_o)
            torch.cuda.synchronize()
            ey = rel_err(oracle.decode(from_torch(yd, DT), DT), y_ref)
            ev = rel_err(v.cpu().numpy(), v_ref)
            say(f"[slots] batch {b} {ln}: err_y {ey:.2e} err_v {ev:.2e}")
            assert ey <= Y_TOL[DT] and ev <= V_TOL
        # the embedding
        tok = rng.integers(0, V, size=T).astype(np.int32)
        y_in = round_to_dtype(rng.normal(0, 1, (T, H)), DT)
        yd = to_torch(y_in, DT, "cuda")
        ve, _ = glsa.embedding_apply(torch.from_numpy(tok).cuda(), cache.A_emb, cache.B_emb, yd, seg, idx,
                                     scale=cache.scale, ranks=cache.ranks)
        Ae_o = np.zeros((S_o, V, R_MAX), np.uint16)
        Be_o = np.zeros((S_o, H, R_MAX), np.uint16)
        for j, a in enumerate(ads):
            Ae_o[j, :, :a.rank] = _bits(a.embedding[0]).T
            Be_o[j, :, :a.rank] = _bits(a.embedding[1])
        v_ref, y_ref = oracle.oracle_embedding_apply(tok, Ae_o, Be_o, y_in, oidx, S_o, dtype=DT,
                                                     scale=scale_o, ranks=ranks_o)
        torch.cuda.synchronize()
        assert rel_err(oracle.decode(from_torch(yd, DT), DT), y_ref) <= Y_TOL[DT]
        assert rel_err(ve[0].cpu().numpy(), v_ref) <= V_TOL
    st = cache.stats
    say(f"[slots] stats {st}")
    assert st.gpu_evictions > 0 and st.gpu_hits > 0 and st.cpu_hits + st.disk_loads == st.gpu_loads
