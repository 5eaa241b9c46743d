"""CPU tests of the C ABI: the library loads, exports what include/lora.h
declares, reports the documented record layout, and rejects bad arguments on
the host before touching the GPU.  No compute call is made here."""

import ctypes
import os
import re

import pytest

import gemm_lora_shrink_amd as glsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = glsa.lib()
    names = declared_functions()
    assert "lora_shrink" in names and "lora_expand" in names and "lora_build_segments" in names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in lora.h but not exported"


def test_version_and_status_strings():
    lib = glsa.lib()
    assert lib.lora_abi_version() == 2
    for code, name in [(0, b"LORA_OK"), (1, b"LORA_ERR_INVALID_ARG"), (2, b"LORA_ERR_UNSUPPORTED"),
                       (3, b"LORA_ERR_INDEX"), (4, b"LORA_ERR_HIP")]:
        assert lib.lora_status_string(code) == name


@pytest.mark.parametrize("T,S", [(0, 1), (1, 1), (64, 4), (256, 8), (8192, 16), (1024, 32),
                                 (4096, 128), (37, 1024)])
def test_segment_record_layout(T, S):
    nbytes = glsa.segments_bytes(T, S)
    assert nbytes % 256 == 0 and nbytes > 0
    off = {k: glsa.segments_offset(T, S, k) for k in glsa.SEG_FIELDS}
    assert off["info"] == 0 and off["perm"] == 16
    assert off["seg_slot"] == 16 + T and off["seg_start"] == 16 + T + S
    assert off["groups"] >= off["seg_start"] + S + 1 and off["groups"] % 4 == 0
    cap_groups = -(-T // 16) + min(S, T)
    cap_tiles = -(-T // 64) + min(S, T)
    # items: a 4-word header then the item's tokens inline (16 per group, 64 per tile)
    assert off["tiles"] == off["groups"] + 20 * cap_groups
    assert (off["tiles"] + 68 * cap_tiles) * 4 <= nbytes


def test_bad_sizes_give_zero_bytes():
    assert glsa.segments_bytes(-1, 4) == 0
    assert glsa.segments_bytes(10, 0) == 0
    assert glsa.segments_bytes(10, 1025) == 0
    assert glsa.segments_offset(10, 0, "perm") == -1


# --------------------------------------------------------------------------
# Host-side validation: every call below is rejected before any HIP call.
# --------------------------------------------------------------------------

FAKE = 0x10000  # a 256-byte aligned, never dereferenced address


def _shrink(**kw):
    a = dict(dt=1, x=FAKE, ldx=64, T=8, D=64, n_slices=1, A=[FAKE], S=4, r_max=16,
             ranks=None, scale=None, seg=FAKE, active=1, v=FAKE)
    a.update(kw)
    A = (ctypes.c_void_p * max(1, len(a["A"])))(*a["A"]) if a["A"] is not None else None
    return glsa.lib().lora_shrink(a["dt"], a["x"], a["ldx"], a["T"], a["D"], a["n_slices"], A,
                                  a["S"], a["r_max"], a["ranks"], a["scale"], a["seg"],
                                  a["active"], a["v"], None)


def _expand(**kw):
    a = dict(dt=2, v=FAKE, vss=0, T=8, n_slices=1, B=[FAKE], sizes=[64], offs=[0], S=4,
             r_max=16, ranks=None, b_layout=0, seg=FAKE, active=1, y=FAKE, ldy=64)
    a.update(kw)
    n = max(1, len(a["B"]))
    B = (ctypes.c_void_p * n)(*a["B"])
    sizes = (ctypes.c_int64 * n)(*a["sizes"])
    offs = (ctypes.c_int64 * n)(*a["offs"])
    return glsa.lib().lora_expand(a["dt"], a["v"], a["vss"], a["T"], a["n_slices"], B, sizes,
                                  offs, a["S"], a["r_max"], a["ranks"], a["b_layout"], a["seg"], a["active"],
                                  a["y"], a["ldy"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=7), glsa.LORA_ERR_INVALID_ARG),
    (dict(T=-1), glsa.LORA_ERR_INVALID_ARG),
    (dict(D=0), glsa.LORA_ERR_INVALID_ARG),
    (dict(ldx=32), glsa.LORA_ERR_INVALID_ARG),
    (dict(x=0), glsa.LORA_ERR_INVALID_ARG),
    (dict(v=0), glsa.LORA_ERR_INVALID_ARG),
    (dict(seg=0), glsa.LORA_ERR_INVALID_ARG),
    (dict(seg=FAKE + 64), glsa.LORA_ERR_INVALID_ARG),
    (dict(A=[0]), glsa.LORA_ERR_INVALID_ARG),
    (dict(n_slices=0), glsa.LORA_ERR_INVALID_ARG),
    (dict(n_slices=9, A=[FAKE] * 9), glsa.LORA_ERR_UNSUPPORTED),
    (dict(S=0), glsa.LORA_ERR_INVALID_ARG),
    (dict(S=1025), glsa.LORA_ERR_UNSUPPORTED),
    (dict(r_max=0), glsa.LORA_ERR_INVALID_ARG),
    (dict(r_max=72), glsa.LORA_ERR_UNSUPPORTED),
    (dict(r_max=12), glsa.LORA_ERR_UNSUPPORTED),      # not a multiple of 8 for fp16
    (dict(D=60, ldx=64), glsa.LORA_ERR_UNSUPPORTED),  # D not a multiple of 8
    (dict(x=FAKE + 8), glsa.LORA_ERR_UNSUPPORTED),    # misaligned
])
def test_shrink_rejects_bad_arguments(kw, status):
    assert _shrink(**kw) == status
    assert glsa.lib().lora_last_error()  # a description is set


@pytest.mark.parametrize("kw,status", [
    (dict(dt=-1), glsa.LORA_ERR_INVALID_ARG),
    (dict(y=0), glsa.LORA_ERR_INVALID_ARG),
    (dict(vss=-4), glsa.LORA_ERR_INVALID_ARG),
    (dict(vss=6), glsa.LORA_ERR_UNSUPPORTED),
    (dict(vss=64), glsa.LORA_ERR_INVALID_ARG),          # smaller than T * r_max
    (dict(sizes=[0]), glsa.LORA_ERR_INVALID_ARG),
    (dict(offs=[8]), glsa.LORA_ERR_INVALID_ARG),        # ends past ldy
    (dict(sizes=[60], ldy=64), glsa.LORA_ERR_UNSUPPORTED),
    (dict(n_slices=2, B=[FAKE, FAKE], sizes=[32, 32], offs=[0, 16]), glsa.LORA_ERR_INVALID_ARG),
    (dict(ldy=0), glsa.LORA_ERR_UNSUPPORTED),
    (dict(B=[FAKE + 4]), glsa.LORA_ERR_UNSUPPORTED),
    (dict(b_layout=2), glsa.LORA_ERR_INVALID_ARG),
    (dict(b_layout=-1), glsa.LORA_ERR_INVALID_ARG),
])
def test_expand_rejects_bad_arguments(kw, status):
    assert _expand(**kw) == status
    assert glsa.lib().lora_last_error()


def test_fp32_allows_rank_multiple_of_four_but_checks_it():
    assert _shrink(dt=0, r_max=12, active=0) == glsa.LORA_OK
    assert _shrink(dt=0, r_max=6, active=0) == glsa.LORA_ERR_UNSUPPORTED


def test_inactive_batch_is_a_host_side_no_op():
    """active_hint = 0 returns OK after validation without any HIP call (no GPU here)."""
    assert _shrink(active=0) == glsa.LORA_OK
    assert _expand(active=0) == glsa.LORA_OK
    assert glsa.lib().lora_last_error() == b""
    # still validated first
    assert _shrink(active=0, D=0) == glsa.LORA_ERR_INVALID_ARG


def test_empty_batch_is_a_no_op():
    assert _shrink(T=0) == glsa.LORA_OK
    assert _expand(T=0) == glsa.LORA_OK


def test_build_segments_rejects_bad_arguments():
    lib = glsa.lib()
    assert lib.lora_build_segments(FAKE, -1, 4, 0, FAKE, None, None) == glsa.LORA_ERR_INVALID_ARG
    assert lib.lora_build_segments(FAKE, 4, 0, 0, FAKE, None, None) == glsa.LORA_ERR_INVALID_ARG
    assert lib.lora_build_segments(FAKE, 4, 2000, 0, FAKE, None, None) == glsa.LORA_ERR_UNSUPPORTED
    assert lib.lora_build_segments(FAKE, 4, 4, 9, FAKE, None, None) == glsa.LORA_ERR_INVALID_ARG
    assert lib.lora_build_segments(FAKE, 4, 4, 0, 0, None, None) == glsa.LORA_ERR_INVALID_ARG
    assert lib.lora_build_segments(FAKE, 4, 4, 0, FAKE + 16, None, None) == glsa.LORA_ERR_INVALID_ARG
    assert lib.lora_build_segments(0, 4, 4, 0, FAKE, None, None) == glsa.LORA_ERR_INVALID_ARG


def test_python_binding_raises_lora_error():
    err = glsa.LoraError(glsa.LORA_ERR_INDEX, "x")
    assert err.status == 3 and "LORA_ERR_INDEX" in str(err)


# --------------------------------------------------------------------------
# lora_shrink_expand: host-side checks (no GPU call)
# --------------------------------------------------------------------------

def _fused(**kw):
    a = dict(dt=1, x=FAKE, ldx=64, T=8, D=64, n_slices=1, A=[FAKE], B=[FAKE], sizes=[64],
             offs=[0], S=4, r_max=16, ranks=None, b_layout=0, scale=None, seg=FAKE, idx=None, active=1,
             v=None, y=FAKE, ldy=64, ws=FAKE, ws_bytes=None)
    a.update(kw)
    n = a["n_slices"]
    if a["ws_bytes"] is None:
        a["ws_bytes"] = glsa.workspace_bytes(a["T"], a["S"], n, a["r_max"]) if a["T"] >= 0 else 0
    A = (ctypes.c_void_p * len(a["A"]))(*a["A"])
    B = (ctypes.c_void_p * len(a["B"]))(*a["B"])
    sizes = (ctypes.c_int64 * len(a["sizes"]))(*a["sizes"])
    offs = (ctypes.c_int64 * len(a["offs"]))(*a["offs"])
    return glsa.lib().lora_shrink_expand(a["dt"], a["x"], a["ldx"], a["T"], a["D"], n, A, B, sizes,
                                         offs, a["S"], a["r_max"], a["ranks"], a["b_layout"], a["scale"],
                                         a["seg"], a["idx"], a["active"], a["v"], a["y"], a["ldy"], a["ws"],
                                         a["ws_bytes"], None)


def test_fused_workspace_bytes():
    # header + one counter per slice and 16-token chunk + the producer slabs
    for T, S, n, r in [(1, 1, 1, 8), (256, 8, 1, 16), (8192, 16, 3, 64), (1024, 32, 2, 64)]:
        b = glsa.workspace_bytes(T, S, n, r)
        assert b % 256 == 0 and b >= 256 + 1024 * 16 * r * 4 * 4 // 3
        assert b >= 256 + n * T * r * 4  # room for v in the two-launch (fp32) form
    assert glsa.workspace_bytes(-1, 4, 1, 8) == 0
    assert glsa.workspace_bytes(4, 4, 9, 8) == 0
    assert glsa.workspace_bytes(4, 4, 1, 72) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(ws=0), glsa.LORA_ERR_INVALID_ARG),
    (dict(ws=FAKE + 16), glsa.LORA_ERR_INVALID_ARG),   # not 256-byte aligned
    (dict(ws_bytes=1024), glsa.LORA_ERR_INVALID_ARG),  # too small
    (dict(dt=5), glsa.LORA_ERR_INVALID_ARG),
    (dict(x=0), glsa.LORA_ERR_INVALID_ARG),
    (dict(y=0), glsa.LORA_ERR_INVALID_ARG),
    (dict(D=60, ldx=64), glsa.LORA_ERR_UNSUPPORTED),
    (dict(sizes=[8], offs=[64]), glsa.LORA_ERR_INVALID_ARG),  # ends past ldy
    (dict(v=FAKE + 8), glsa.LORA_ERR_UNSUPPORTED),      # misaligned v
    (dict(A=[0]), glsa.LORA_ERR_INVALID_ARG),
    (dict(B=[0]), glsa.LORA_ERR_INVALID_ARG),
    (dict(b_layout=5), glsa.LORA_ERR_INVALID_ARG),
])
def test_fused_rejects_bad_arguments(kw, status):
    assert _fused(**kw) == status
    assert glsa.lib().lora_last_error()


def test_fused_inactive_and_empty_are_host_side_no_ops():
    assert _fused(active=0) == glsa.LORA_OK
    assert _fused(active=0, v=FAKE) == glsa.LORA_OK
    assert _fused(T=0) == glsa.LORA_OK
    assert _fused(active=0, D=0) == glsa.LORA_ERR_INVALID_ARG  # still validated first


# --------------------------------------------------------------------------
# Python binding: tensors the kernels would misread are rejected before any
# library call (the C ABI cannot check a bare pointer's device, dtype or size)
# --------------------------------------------------------------------------

class _HostOnlyLib:
    """The loaded library with its enqueueing entry points guarded: a call
    reaching one fails the test, unless `allow` is set (then a call with
    active = 0 only runs the library's host checks and enqueues nothing)."""
    COMPUTE = {"lora_build_segments", "lora_shrink", "lora_expand", "lora_shrink_expand"}

    def __init__(self, lib):
        self._lib = lib
        self.allow = False

    def __getattr__(self, name):
        if name in self.COMPUTE and not self.allow:
            raise AssertionError(f"{name} was reached with an argument the binding must reject")
        return getattr(self._lib, name)


@pytest.fixture
def host_only(monkeypatch):
    import torch
    proxy = _HostOnlyLib(glsa.lib())
    monkeypatch.setattr(glsa, "_lib", proxy)
    # CPU tensors stand in for device tensors of one GPU: the device test
    # becomes "same device as x", and every other check runs as on a GPU
    monkeypatch.setattr(glsa, "_on_device", lambda t, dev: t.device == dev)
    T, S, D, r, out = 8, 4, 64, 16, 64
    t = dict(
        x=torch.zeros(T, D, dtype=torch.float16), y=torch.zeros(T, out, dtype=torch.float16),
        A=[torch.zeros(S, r, D, dtype=torch.float16)], B=[torch.zeros(S, out, r, dtype=torch.float16)],
        v=torch.zeros(1, T, r), ranks=torch.full((S,), r, dtype=torch.int32),
        scale=torch.ones(S), seg=_aligned(torch, glsa.segments_bytes(T, S) // 4, torch.int32),
        idx=torch.zeros(T, dtype=torch.int32),
        ws=_aligned(torch, glsa.workspace_bytes(T, S, 1, r), torch.uint8))
    return proxy, t


def _aligned(torch, n, dtype):
    """A zeroed host tensor of n elements at a 256-byte aligned address (the
    library's own alignment checks still run in these tests)."""
    esz = torch.empty(0, dtype=dtype).element_size()
    buf = torch.zeros(n + 256 // esz, dtype=dtype)
    skip = (-buf.data_ptr() % 256) // esz
    return buf[skip:skip + n]


def _call(kind, t, **over):
    a = dict(t)
    a.update(over)
    if kind == "shrink":
        return glsa.shrink(a["x"], a["A"], a["seg"], scale=a["scale"], ranks=a["ranks"], v=a["v"],
                           active=False, stream=_NoStream())
    if kind == "expand":
        return glsa.expand(a["v"], a["B"], a["y"], a["seg"], [0], ranks=a["ranks"], active=False,
                           stream=_NoStream())
    if kind == "shrink_expand":
        return glsa.shrink_expand(a["x"], a["A"], a["B"], a["y"], a["seg"], [0], workspace=a["ws"],
                                  scale=a["scale"], ranks=a["ranks"], v=a["v"], idx=a["idx"],
                                  active=False, stream=_NoStream())
    return glsa.build_segments(a["idx"], 4, seg=a["seg"], stream=_NoStream())


class _NoStream:
    cuda_stream = 0


def test_binding_accepts_valid_tensors(host_only):
    proxy, t = host_only
    proxy.allow = True
    for kind in ("shrink", "expand", "shrink_expand"):
        _call(kind, t)  # active = 0: host checks only, nothing enqueued


@pytest.mark.parametrize("kind,field,make", [
    ("shrink", "ranks", lambda torch, t: t["ranks"].to(torch.int64)),
    ("shrink", "ranks", lambda torch, t: t["ranks"][:3]),
    ("shrink", "scale", lambda torch, t: t["scale"].to(torch.float64)),
    ("shrink", "scale", lambda torch, t: t["scale"][:2]),
    ("shrink", "seg", lambda torch, t: t["seg"][:64]),
    ("shrink", "A", lambda torch, t: [t["A"][0].transpose(1, 2).contiguous().transpose(1, 2)]),
    ("expand", "v", lambda torch, t: torch.zeros(1, 4, 16)),
    ("expand", "ranks", lambda torch, t: t["ranks"].to(torch.int16)),
    ("expand", "seg", lambda torch, t: t["seg"][:10]),
    ("shrink_expand", "ranks", lambda torch, t: t["ranks"].to(torch.int64)),
    ("shrink_expand", "scale", lambda torch, t: t["scale"].double()),
    ("shrink_expand", "seg", lambda torch, t: t["seg"][:32]),
    ("shrink_expand", "idx", lambda torch, t: t["idx"][::2].clone()),
    ("build_segments", "seg", lambda torch, t: t["seg"][:16]),
], ids=lambda v: v if isinstance(v, str) else "")
def test_binding_rejects_misread_tensors(host_only, kind, field, make):
    import torch
    _, t = host_only
    with pytest.raises(glsa.LoraError):
        _call(kind, t, **{field: make(torch, t)})


def test_binding_rejects_host_tensors_for_device_arguments(monkeypatch):
    """Without the stand-in, a host tensor is refused (it would be a host
    address inside a kernel)."""
    import torch
    monkeypatch.setattr(glsa, "_lib", _HostOnlyLib(glsa.lib()))
    x = torch.zeros(8, 64, dtype=torch.float16)
    A = [torch.zeros(4, 16, 64, dtype=torch.float16)]
    seg = glsa.alloc_segments(8, 4, "cpu")
    with pytest.raises(glsa.LoraError, match="must be on"):
        glsa.shrink(x, A, seg, active=False, stream=_NoStream())


# --------------------------------------------------------------------------
# lora_shrink_expand_noalloc: host-side refusals (no GPU call)
# --------------------------------------------------------------------------

def _noalloc(**kw):
    a = dict(dt=2, x=FAKE, ldx=64, T=8, D=64, n_slices=1, A=[FAKE], B=[FAKE], sizes=[64],
             offs=[0], S=4, r_max=16, ranks=None, b_layout=0, scale=None, seg=FAKE, idx=None, active=1,
             v=None, y=FAKE, ldy=64, err=None)
    a.update(kw)
    n = a["n_slices"]
    A = (ctypes.c_void_p * len(a["A"]))(*a["A"])
    B = (ctypes.c_void_p * len(a["B"]))(*a["B"])
    sizes = (ctypes.c_int64 * len(a["sizes"]))(*a["sizes"])
    offs = (ctypes.c_int64 * len(a["offs"]))(*a["offs"])
    return glsa.lib().lora_shrink_expand_noalloc(
        a["dt"], a["x"], a["ldx"], a["T"], a["D"], n, A, B, sizes, offs, a["S"], a["r_max"], a["ranks"],
        a["b_layout"], a["scale"], a["seg"], a["idx"], a["active"], a["v"], a["y"], a["ldy"], a["err"], None)


def test_noalloc_scratch_limit_matches_header():
    src = open(HEADER).read()
    m = re.search(r"#define LORA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == glsa.NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("kw,status", [
    # needs more scratch than the variant has: refused before anything else
    (dict(T=16384, n_slices=8, r_max=64, A=[FAKE] * 8, B=[FAKE] * 8, sizes=[64] * 8,
          offs=[64 * i for i in range(8)], ldy=512), glsa.LORA_ERR_UNSUPPORTED),
    (dict(dt=9), glsa.LORA_ERR_INVALID_ARG),
    (dict(seg=0), glsa.LORA_ERR_INVALID_ARG),
    (dict(S=0), glsa.LORA_ERR_INVALID_ARG),
    (dict(r_max=72), glsa.LORA_ERR_UNSUPPORTED),
])
def test_noalloc_rejects_on_the_host(kw, status):
    assert glsa.workspace_bytes(16384, 4, 8, 64) > glsa.NOALLOC_SCRATCH_BYTES
    assert _noalloc(**kw) == status
    assert glsa.lib().lora_last_error()


# --------------------------------------------------------------------------
# lora_embedding_shrink and lora_copy_padded: host-side checks (no GPU call)
# --------------------------------------------------------------------------

def _emb(**kw):
    a = dict(dt=1, tok=FAKE, T=8, V=100, A=FAKE, S=4, r_max=16, ranks=None, scale=None, idx=FAKE,
             active=1, v=FAKE)
    a.update(kw)
    return glsa.lib().lora_embedding_shrink(a["dt"], a["tok"], a["T"], a["V"], a["A"], a["S"], a["r_max"],
                                            a["ranks"], a["scale"], a["idx"], a["active"], a["v"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=4), glsa.LORA_ERR_INVALID_ARG), (dict(T=-1), glsa.LORA_ERR_INVALID_ARG),
    (dict(V=0), glsa.LORA_ERR_INVALID_ARG), (dict(S=0), glsa.LORA_ERR_INVALID_ARG),
    (dict(S=2000), glsa.LORA_ERR_UNSUPPORTED), (dict(r_max=12), glsa.LORA_ERR_UNSUPPORTED),
    (dict(r_max=128), glsa.LORA_ERR_UNSUPPORTED), (dict(tok=0), glsa.LORA_ERR_INVALID_ARG),
    (dict(idx=0), glsa.LORA_ERR_INVALID_ARG), (dict(v=0), glsa.LORA_ERR_INVALID_ARG),
    (dict(A=FAKE + 4), glsa.LORA_ERR_UNSUPPORTED),
])
def test_embedding_shrink_rejects_bad_arguments(kw, status):
    assert _emb(**kw) == status
    assert glsa.lib().lora_last_error()


def test_embedding_shrink_inactive_and_empty_are_host_side_no_ops():
    assert _emb(active=0) == glsa.LORA_OK
    assert _emb(T=0, tok=0, idx=0, v=0) == glsa.LORA_OK


@pytest.mark.parametrize("args,status", [
    ((1, FAKE, 4, 8, 8, 0, FAKE, 3, 8, 8), glsa.LORA_ERR_INVALID_ARG),    # more rows than the slot
    ((1, FAKE, 4, 8, 8, 0, FAKE, 4, 6, 8), glsa.LORA_ERR_INVALID_ARG),    # more columns than the slot
    ((1, FAKE, 4, 8, 4, 0, FAKE, 4, 8, 8), glsa.LORA_ERR_INVALID_ARG),    # short source stride
    ((1, FAKE, 4, 8, 8, 0, FAKE, 4, 8, 4), glsa.LORA_ERR_INVALID_ARG),    # short slot stride
    ((1, 0, 4, 8, 8, 0, FAKE, 4, 8, 8), glsa.LORA_ERR_INVALID_ARG),       # null source
    ((1, FAKE, 4, 8, 8, 0, 0, 4, 8, 8), glsa.LORA_ERR_INVALID_ARG),       # null slot
    ((9, FAKE, 4, 8, 8, 0, FAKE, 4, 8, 8), glsa.LORA_ERR_INVALID_ARG),    # dtype
    ((1, FAKE, -1, 8, 8, 0, FAKE, 4, 8, 8), glsa.LORA_ERR_INVALID_ARG),   # negative size
    ((1, FAKE, 8, 4, 4, 1, FAKE, 8, 4, 4), glsa.LORA_ERR_INVALID_ARG),    # transposed: stride < m_rows
])
def test_copy_padded_rejects_bad_arguments(args, status):
    assert glsa.lib().lora_copy_padded(*args, None) == status
