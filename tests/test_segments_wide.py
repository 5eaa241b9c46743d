"""GPU: the wide segment build.

From 512 tokens the build runs one workgroup per 1024 tokens; each counts
the whole batch itself and places its own range (LORA_SEG_WIDE_MIN_T moves the
threshold, which lets small and ragged batches take that path here).  Its
record must be the oracle's, word for word, as for the one-workgroup build:
at workgroup edges, with out-of-range indices in several ranges, when the
record held garbage before, under graph replay and at hundreds of
workgroups."""

import numpy as np
import pytest
import torch

import gemm_lora_shrink_amd as glsa
from gpu_util import say
from test_segments import MODES, check_record, specified_words

pytestmark = pytest.mark.gpu


@pytest.fixture
def wide_always(monkeypatch):
    monkeypatch.setenv("LORA_SEG_WIDE_MIN_T", "1")


def wide_cases():
    rng = np.random.default_rng(77)
    yield "one_token", np.array([3], np.int32), 4
    yield "one_block_ragged", rng.integers(-1, 5, size=300).astype(np.int32), 5
    yield "block_edge_1024", rng.integers(-1, 9, size=1024).astype(np.int32), 9
    yield "block_edge_1025", rng.integers(-1, 9, size=1025).astype(np.int32), 9
    yield "chunk_edge_4095", rng.integers(-1, 9, size=4095).astype(np.int32), 9
    yield "all_base", np.full(5000, -1, np.int32), 8
    yield "one_slot", np.zeros(4100, np.int32), 1
    # out-of-range indices in several workgroups' ranges
    bad = rng.integers(-1, 6, size=6000).astype(np.int32)
    bad[[10, 1700, 5999]] = [6, -5, 1 << 30]
    yield "bad_spread", bad, 6
    yield "max_slots", rng.integers(-1, 1024, size=9000).astype(np.int32), 1024
    # slots whose tokens straddle every workgroup boundary
    yield "runs_across_blocks", np.repeat(np.arange(12, dtype=np.int32), 700), 12
    yield "prefill_like", np.repeat(np.arange(16, dtype=np.int32), 512), 16
    p = (np.arange(300) + 1.0) ** -1.1
    yield "zipf_300", rng.choice(300, size=20000, p=p / p.sum()).astype(np.int32), 300


@pytest.mark.parametrize("case", list(wide_cases()), ids=lambda c: c[0])
@pytest.mark.parametrize("mode", MODES)
def test_wide_records(wide_always, case, mode):
    label, idx, S = case
    check_record(idx, S, mode, "wide:" + label)


def test_many_workgroups():
    rng = np.random.default_rng(78)
    # 64 workgroups at S = 1024; 391 workgroups, each counting 6250 chunks
    check_record(rng.integers(-1, 1024, size=65536).astype(np.int32), 1024, "auto", "wide_64_blocks")
    check_record(rng.integers(-1, 37, size=400000).astype(np.int32), 37, "auto", "wide_391_blocks")


def test_wide_equals_block_build(monkeypatch):
    rng = np.random.default_rng(79)
    for T, S in [(4096, 128), (8192, 16), (6000, 1024), (20000, 50), (1024, 257), (700, 3)]:
        idx = torch.from_numpy(rng.integers(-1, S, size=T).astype(np.int32)).cuda()
        say(f"[segments-wide] wide vs block T={T} S={S}")
        monkeypatch.setenv("LORA_SEG_WIDE_MIN_T", "1")
        g = specified_words(glsa.build_segments(idx, S).cpu().numpy(), T, S)
        monkeypatch.setenv("LORA_SEG_WIDE_MIN_T", str(1 << 30))
        one = specified_words(glsa.build_segments(idx, S).cpu().numpy(), T, S)
        assert np.array_equal(g, one)


def test_garbage_record_and_reuse(wide_always):
    rng = np.random.default_rng(80)
    T, S = 8192, 64
    seg = glsa.alloc_segments(T, S, "cuda")
    seg.copy_(torch.from_numpy(rng.integers(-2**31, 2**31 - 1, size=seg.numel(), dtype=np.int64)
                               .astype(np.int32)).cuda())
    for rep in range(3):
        idx = rng.integers(-1, S, size=T).astype(np.int32)
        say(f"[segments-wide] garbage/reuse rep={rep}")
        d = torch.from_numpy(idx).cuda()
        glsa.build_segments(d, S, seg=seg)
        rec = seg.cpu().numpy()
        ref = glsa.build_segments(d, S).cpu().numpy()  # a fresh record
        assert np.array_equal(specified_words(rec, T, S), specified_words(ref, T, S))
    check_record(idx, S, "auto", "wide_reused_record")


def test_graph_replay(wide_always):
    rng = np.random.default_rng(81)
    T, S = 8192, 32
    idx = torch.empty(T, dtype=torch.int32, device="cuda")
    seg = glsa.alloc_segments(T, S, "cuda")
    idx.copy_(torch.from_numpy(rng.integers(-1, S, size=T).astype(np.int32)))
    glsa.build_segments(idx, S, seg=seg)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            glsa.build_segments(idx, S, seg=seg, stream=s)
    torch.cuda.synchronize()
    for rep in range(5):
        host = rng.integers(-1, S, size=T).astype(np.int32)
        idx.copy_(torch.from_numpy(host))
        torch.cuda.synchronize()
        say(f"[segments-wide] graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        rec = seg.cpu().numpy()
        fresh = glsa.build_segments(torch.from_numpy(host).cuda(), S).cpu().numpy()
        assert np.array_equal(specified_words(rec, T, S), specified_words(fresh, T, S)), rep
