"""GPU: the segment record is bit-exact against the oracle's slot grouping."""

import numpy as np
import pytest
import torch

import gemm_lora_shrink_amd as glsa
import oracle
from gpu_util import say
from workloads import CONFIG_ORDER, make_workload

pytestmark = pytest.mark.gpu

MODES = ["auto", "bgmv", "sgmv"]


def gpu_segments(idx, S, mode):
    d = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()
    seg = glsa.build_segments(d, S, mode=mode)
    torch.cuda.synchronize()
    T = idx.shape[0]
    rec = seg.cpu().numpy()
    off = {k: glsa.segments_offset(T, S, k) for k in glsa.SEG_FIELDS}
    return rec, off


def check_record(idx, S, mode, label):
    say(f"[segments] {label} T={idx.shape[0]} S={S} mode={mode}")
    T = idx.shape[0]
    rec, off = gpu_segments(idx, S, mode)
    ref = oracle.oracle_segments(idx, S)
    info = rec[:16]
    na, ns = ref["num_active"], ref["num_segments"]
    assert info[0] == na and info[1] == ns, label
    assert info[2] == ref["max_seg_len"] and info[3] == ref["status"], label
    assert info[6] == T and info[7] == S and not np.any(info[8:]), label
    assert np.array_equal(rec[off["perm"]:off["perm"] + na], ref["perm"]), label
    assert np.array_equal(rec[off["perm"] + na:off["perm"] + T], ref["rest"]), label
    assert np.array_equal(rec[off["seg_slot"]:off["seg_slot"] + ns], ref["seg_slot"]), label
    assert np.array_equal(rec[off["seg_start"]:off["seg_start"] + ns + 1], ref["seg_start"]), label

    # work items: disjoint, cover every active perm position once, single slot,
    # sizes bounded, split by the documented rule
    counts = np.diff(ref["seg_start"])
    thr = glsa.sgmv_min_tokens()
    covered = np.zeros(na, dtype=np.int32)
    for name, cap, n in (("groups", 16, info[4]), ("tiles", 64, info[5])):
        words = 4 + cap
        items = rec[off[name]:off[name] + words * n].reshape(n, words)
        for row in items:
            p0, cnt, slot, segno = (int(v) for v in row[:4])
            assert 1 <= cnt <= cap, label
            # the item's tokens follow its header, then -1 padding
            assert np.array_equal(row[4:4 + cnt], ref["perm"][p0:p0 + cnt]), label
            assert np.all(row[4 + cnt:] == -1), label
            assert ref["seg_slot"][segno] == slot, label
            assert ref["seg_start"][segno] <= p0 and p0 + cnt <= ref["seg_start"][segno + 1], label
            covered[p0:p0 + cnt] += 1
            n_seg = counts[segno]
            to_tiles = mode == "sgmv" or (mode == "auto" and n_seg >= thr)
            assert to_tiles == (name == "tiles"), label
            assert (p0 - ref["seg_start"][segno]) % cap == 0, label
    assert np.all(covered == 1), label


@pytest.mark.parametrize("name", [n for n in CONFIG_ORDER])
@pytest.mark.parametrize("mode", MODES)
def test_config_records(name, mode):
    wl = make_workload(name)
    check_record(wl.idx, wl.S, mode, name)


def edge_cases():
    rng = np.random.default_rng(2024)
    yield "empty", np.zeros(0, np.int32), 4
    yield "single_active", np.array([2], np.int32), 3
    yield "single_base", np.array([-1], np.int32), 3
    yield "all_base", np.full(1000, -1, np.int32), 16
    yield "bad_indices", np.array([0, -2, 5, 1, 99, -1, 1, 0], np.int32), 4
    yield "one_slot_S1", np.zeros(777, np.int32), 1
    yield "max_slots", rng.integers(-1, 1024, size=5000).astype(np.int32), 1024
    yield "ragged_3001", rng.integers(-1, 7, size=3001).astype(np.int32), 7
    yield "long_20000", rng.integers(-1, 50, size=20000).astype(np.int32), 50
    yield "wave_boundaries", np.repeat(np.arange(9, dtype=np.int32), 64 + 1), 9
    yield "descending", np.repeat(np.arange(30, -1, -1, dtype=np.int32), 70), 31
    z = rng.choice(200, size=6000, p=(np.arange(200) + 1.0) ** -1.3 / np.sum((np.arange(200) + 1.0) ** -1.3))
    yield "zipf_200", z.astype(np.int32), 200
    # around the switch between the 4-wave build (T <= 1024, S <= 256) and the
    # 16-wave one: largest small batch, one token more, one slot more
    yield "small_T1024_S256", rng.integers(-1, 256, size=1024).astype(np.int32), 256
    yield "large_T1025_S256", rng.integers(-1, 256, size=1025).astype(np.int32), 256
    yield "large_T1024_S257", rng.integers(-1, 257, size=1024).astype(np.int32), 257
    yield "small_one_slot_full", np.zeros(1024, np.int32), 1
    yield "small_wave_edges", np.repeat(np.arange(4, dtype=np.int32), [255, 257, 1, 511]), 4


@pytest.mark.parametrize("case", list(edge_cases()), ids=lambda c: c[0])
@pytest.mark.parametrize("mode", MODES)
def test_edge_records(case, mode):
    label, idx, S = case
    check_record(idx, S, mode, label)


def specified_words(rec, T, S):
    """The documented and planned parts of a record (everything the kernels read)."""
    off = {k: glsa.segments_offset(T, S, k) for k in glsa.SEG_FIELDS}
    info = rec[:16]
    return np.concatenate([
        info, rec[off["perm"]:off["perm"] + T],
        rec[off["seg_slot"]:off["seg_slot"] + info[1]],
        rec[off["seg_start"]:off["seg_start"] + info[1] + 1],
        rec[off["groups"]:off["groups"] + 20 * info[4]],
        rec[off["tiles"]:off["tiles"] + 68 * info[5]]])


def test_deterministic_over_repeats():
    rng = np.random.default_rng(5)
    T, S = 4096, 64
    idx = rng.integers(-1, S, size=T).astype(np.int32)
    d = torch.from_numpy(idx).cuda()
    first = specified_words(glsa.build_segments(d, S).cpu().numpy(), T, S)
    for _ in range(50):
        again = specified_words(glsa.build_segments(d, S).cpu().numpy(), T, S)
        assert np.array_equal(again, first)


def test_info_host_copy():
    idx = torch.tensor([1, -1, 7, 1, 0], dtype=torch.int32, device="cuda")
    info = torch.zeros(16, dtype=torch.int32, pin_memory=True)
    glsa.build_segments(idx, 4, info_host=info)
    torch.cuda.synchronize()
    assert info[0].item() == 3 and info[3].item() == glsa.LORA_ERR_INDEX
