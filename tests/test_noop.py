"""GPU: a base-only batch is a true no-op.

With active_hint = 0 the library enqueues nothing (the host knows no adapter
is active, as in "[LoRA] LoRA cuda graph specialization", Implementation), so
y and v stay byte-identical.  With active_hint = 1 on an all-base batch the
kernels run, find no active token on the device, clear v and leave y alone.
"""

import time

import numpy as np
import pytest
import torch

import gemm_lora_shrink_amd as glsa
from workloads import make_workload
from workloads.torch_io import problem_to_device

pytestmark = pytest.mark.gpu


def _setup():
    wl = make_workload("zipf_many_noop")
    p = wl.problems[0]
    d = problem_to_device(p, "cuda")
    seg = glsa.build_segments(d["idx"], p.S)
    return p, d, seg


def test_inactive_hint_touches_nothing():
    p, d, seg = _setup()
    v = torch.full((1, p.T, p.r_max), float("nan"), device="cuda")
    y0 = d["y"].clone()
    v0 = v.clone()
    glsa.apply(d["x"], d["A"], d["B"], d["y"], seg, p.out_offsets, v=v, active=False)
    torch.cuda.synchronize()
    assert torch.equal(d["y"].view(torch.int16), y0.view(torch.int16))
    assert torch.equal(v.view(torch.int32), v0.view(torch.int32))


def test_all_base_with_hint_runs_and_changes_nothing_but_v():
    p, d, seg = _setup()
    info = seg[:16].cpu().numpy()
    assert info[0] == 0 and info[4] == 0 and info[5] == 0
    v = torch.full((1, p.T, p.r_max), float("nan"), device="cuda")
    y0 = d["y"].clone()
    glsa.apply(d["x"], d["A"], d["B"], d["y"], seg, p.out_offsets, v=v, active=True)
    torch.cuda.synchronize()
    assert torch.equal(d["y"].view(torch.int16), y0.view(torch.int16))
    assert torch.count_nonzero(v).item() == 0


def test_inactive_hint_enqueues_no_kernel():
    """1000 no-op calls put no work on the stream.

    A queue of large matmuls keeps the GPU busy while the host makes the calls,
    so the two events around the calls run back to back unless a call enqueued
    something between them.
    """
    p, d, seg = _setup()
    v = torch.empty((1, p.T, p.r_max), device="cuda")
    big = torch.randn(8192, 8192, device="cuda", dtype=torch.float16)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    for _ in range(200):
        torch.mm(big, big)
    ev[1].record()
    t0 = time.perf_counter()
    for _ in range(1000):
        glsa.apply(d["x"], d["A"], d["B"], d["y"], seg, p.out_offsets, v=v, active=False)
    host_ms = (time.perf_counter() - t0) * 1e3
    ev[2].record()
    torch.cuda.synchronize()
    blocker_ms = ev[0].elapsed_time(ev[1])
    assert host_ms < blocker_ms, "blocker too short to hide the host loop"
    assert ev[1].elapsed_time(ev[2]) < 0.05
