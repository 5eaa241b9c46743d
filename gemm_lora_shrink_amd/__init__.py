"""Python binding of the MI355X multi-LoRA library (liblora_mi355x.so).

Thin ctypes layer over the C ABI in include/lora.h: it turns torch tensors
into pointers, sizes and strides and raises LoraError on a non-OK status.
Every step of the computation runs in the library's HIP kernels; there is no
Python or CPU fallback, and importing this package fails loudly if the
library has not been built (python -m gemm_lora_shrink_amd.build).

Entry points (same names as the C ABI):
    build_segments(idx, S, mode="auto") -> segment record (int32 tensor)
    shrink(x, A, seg, ...)               -> v  [n_slices, T, r_max] fp32
    expand(v, B, y, seg, out_offsets, ...) (y updated in place)
    apply(x, A, B, y, seg, out_offsets, ...) = shrink then expand
    shrink_expand(x, A, B, y, seg, out_offsets, workspace=..., ...)
                                         the same in one call (one launch for 16-bit data)
    shrink_expand_noalloc(x, A, B, y, seg, out_offsets, ...)
                                         the same without a workspace (allocates nothing)
    embedding_shrink(tok, A_emb, idx, ...) -> v of an embedding adapter ([1, T, r_max])
    embedding_apply(tok, A_emb, B_emb, y, seg, idx, ...) = embedding_shrink then expand
    shrink_expand_mask(x, A, B, y, idx, out_offsets, workspace=...)
                                         the mask ("laning") form for S * r_max <= 128
    alloc_workspace(T, S, n_slices, r_max, device) -> zeroed workspace for it
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# LORA_MI355X_LIB names another build of this same library (the host-checks
# test loads one built with the address and undefined-behaviour sanitizers).
LIB_PATH = os.environ.get("LORA_MI355X_LIB") or os.path.join(_HERE, "liblora_mi355x.so")

LORA_OK = 0
LORA_ERR_INVALID_ARG = 1
LORA_ERR_UNSUPPORTED = 2
LORA_ERR_INDEX = 3
LORA_ERR_HIP = 4

MODES = {"auto": 0, "bgmv": 1, "sgmv": 2}
# lora_b_layout: how each slot's B rows are stored in its [out][r_max] region
B_LAYOUTS = {"padded": 0, "rank_rows": 1}
# LORA_NOALLOC_SCRATCH_BYTES of include/lora.h: the per-device scratch of
# shrink_expand_noalloc
NOALLOC_SCRATCH_BYTES = 32 << 20
SEG_FIELDS = {"info": 0, "perm": 1, "seg_slot": 2, "seg_start": 3, "groups": 4, "tiles": 5}
INFO_WORDS = 16
MAX_SLICES = 8

_DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}


class LoraError(RuntimeError):
    """A non-OK status returned by the library."""

    def __init__(self, status, message):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -m gemm_lora_shrink_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.lora_segments_bytes.argtypes = [i32, i32]
    lib.lora_segments_bytes.restype = sz
    lib.lora_segments_offset.argtypes = [i32, i32, ctypes.c_int]
    lib.lora_segments_offset.restype = i64
    lib.lora_sgmv_min_tokens.argtypes = []
    lib.lora_sgmv_min_tokens.restype = i32
    lib.lora_build_segments.argtypes = [vp, i32, i32, i32, vp, vp, vp]
    lib.lora_build_segments.restype = ctypes.c_int
    lib.lora_shrink.argtypes = [ctypes.c_int, vp, i64, i32, i32, i32, vp, i32, i32, vp, vp, vp,
                                i32, vp, vp]
    lib.lora_shrink.restype = ctypes.c_int
    lib.lora_expand.argtypes = [ctypes.c_int, vp, i64, i32, i32, vp, vp, vp, i32, i32, vp, i32, vp,
                                i32, vp, i64, vp]
    lib.lora_expand.restype = ctypes.c_int
    lib.lora_fused_max_tokens.argtypes = []
    lib.lora_fused_max_tokens.restype = i32
    lib.lora_fused_max_tokens_for.argtypes = [i32]
    lib.lora_fused_max_tokens_for.restype = i32
    lib.lora_shrink_expand_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.lora_shrink_expand_workspace_bytes.restype = sz
    lib.lora_shrink_expand.argtypes = [ctypes.c_int, vp, i64, i32, i32, i32, vp, vp, vp, vp, i32,
                                       i32, vp, i32, vp, vp, vp, i32, vp, vp, i64, vp, sz, vp]
    lib.lora_shrink_expand.restype = ctypes.c_int
    lib.lora_shrink_expand_noalloc.argtypes = [ctypes.c_int, vp, i64, i32, i32, i32, vp, vp, vp, vp,
                                               i32, i32, vp, i32, vp, vp, vp, i32, vp, vp, i64, vp, vp]
    lib.lora_shrink_expand_noalloc.restype = ctypes.c_int
    lib.lora_embedding_shrink.argtypes = [ctypes.c_int, vp, i32, i64, vp, i32, i32, vp, vp, vp, i32, vp, vp]
    lib.lora_embedding_shrink.restype = ctypes.c_int
    lib.lora_copy_padded.argtypes = [ctypes.c_int, vp, i64, i64, i64, i32, vp, i64, i64, i64, vp]
    lib.lora_copy_padded.restype = ctypes.c_int
    lib.lora_mask_workspace_bytes.argtypes = [ctypes.c_int, i32, i32, i32, i32, i32]
    lib.lora_mask_workspace_bytes.restype = sz
    lib.lora_shrink_expand_mask.argtypes = [ctypes.c_int, vp, i64, i32, i32, i32, vp, vp, vp, vp, i32, i32,
                                            vp, vp, vp, i32, vp, vp, i64, vp, sz, vp]
    lib.lora_shrink_expand_mask.restype = ctypes.c_int
    lib.lora_workspace_errors.argtypes = [vp, vp, vp]
    lib.lora_workspace_errors.restype = ctypes.c_int
    lib.lora_status_string.argtypes = [ctypes.c_int]
    lib.lora_status_string.restype = ctypes.c_char_p
    lib.lora_last_error.argtypes = []
    lib.lora_last_error.restype = ctypes.c_char_p
    lib.lora_abi_version.argtypes = []
    lib.lora_abi_version.restype = i32
    _lib = lib
    return lib


def lib():
    """The loaded ctypes library (raises ImportError if it is not built)."""
    return _load()


def _status_name(status):
    try:
        return _load().lora_status_string(status).decode()
    except Exception:
        return f"status {status}"


def _check(status):
    if status != LORA_OK:
        raise LoraError(status, _load().lora_last_error().decode())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _on_device(t, device):
    """True when t lives in the memory of GPU `device`."""
    return t.device.type == "cuda" and t.device == device


def _check_tensor(t, name, device, *, dtype=None, min_numel=None, min_bytes=None):
    """Reject, before anything reaches the library, a tensor the kernels would
    misread: not on the call's GPU (a host address faults a kernel), another
    dtype (int64 ranks or float64 scales would be read as 32-bit words), not
    contiguous, or too small for what the call reads or writes.  The C ABI
    takes bare pointers and cannot check any of this itself."""
    if t is None:
        return
    if not _on_device(t, device):
        raise LoraError(LORA_ERR_INVALID_ARG, f"{name} must be on {device} (it is on {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise LoraError(LORA_ERR_INVALID_ARG, f"{name} must be {dtype} (it is {t.dtype})")
    if not t.is_contiguous():
        raise LoraError(LORA_ERR_INVALID_ARG, f"{name} must be contiguous")
    if min_numel is not None and t.numel() < min_numel:
        raise LoraError(LORA_ERR_INVALID_ARG, f"{name} has {t.numel()} elements, the call needs {min_numel}")
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise LoraError(LORA_ERR_INVALID_ARG,
                        f"{name} has {t.numel() * t.element_size()} bytes, the call needs {min_bytes}")


def _check_rows(t, name, device):
    """x or y: on the call's GPU (row strides are checked by _rows)."""
    if not _on_device(t, device):
        raise LoraError(LORA_ERR_INVALID_ARG, f"{name} must be on {device} (it is on {t.device})")


def _check_slot_tables(device, S, ranks, scale=None):
    _check_tensor(ranks, "ranks", device, dtype=torch.int32, min_numel=S)
    _check_tensor(scale, "scale", device, dtype=torch.float32, min_numel=S)


def _check_record(seg, T, S, device):
    if seg is None:
        raise LoraError(LORA_ERR_INVALID_ARG, "segment record is missing")
    _check_tensor(seg, "seg", device, min_bytes=segments_bytes(T, S))


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise LoraError(LORA_ERR_INVALID_ARG, f"unsupported dtype {t.dtype}") from None


def _rows(t, name):
    """(rows, width, row stride) of a 2-D tensor with unit inner stride."""
    if t.dim() == 2 and t.numel() == 0:
        return t.size(0), t.size(1), max(t.size(1), 1)
    if t.dim() != 2 or (t.size(1) > 1 and t.stride(1) != 1):
        raise LoraError(LORA_ERR_INVALID_ARG, f"{name} must be 2-D with contiguous rows")
    return t.size(0), t.size(1), t.stride(0) if t.size(0) > 1 else max(t.stride(0), t.size(1))


def segments_bytes(T, S):
    return int(_load().lora_segments_bytes(T, S))


def segments_offset(T, S, field):
    return int(_load().lora_segments_offset(T, S, SEG_FIELDS[field]))


def sgmv_min_tokens():
    return int(_load().lora_sgmv_min_tokens())


def alloc_segments(T, S, device):
    n = segments_bytes(T, S)
    if n == 0:
        raise LoraError(LORA_ERR_INVALID_ARG, f"bad sizes T={T} S={S}")
    return torch.empty(n // 4, dtype=torch.int32, device=device)


def build_segments(idx, S, *, mode="auto", seg=None, info_host=None, stream=None):
    """Group the batch's tokens by slot; returns the segment record tensor."""
    if idx.dtype != torch.int32 or idx.dim() != 1 or not idx.is_contiguous():
        raise LoraError(LORA_ERR_INVALID_ARG, "idx must be a contiguous 1-D int32 tensor")
    T = idx.numel()
    if seg is None:
        seg = alloc_segments(T, S, idx.device)
    _check_tensor(idx, "idx", idx.device)
    _check_record(seg, T, S, idx.device)
    if info_host is not None and (info_host.device.type != "cpu" or not info_host.is_pinned()
                                  or info_host.dtype != torch.int32 or info_host.numel() < INFO_WORDS
                                  or not info_host.is_contiguous()):
        raise LoraError(LORA_ERR_INVALID_ARG, "info_host must be pinned host memory of 16 int32")
    st = _load().lora_build_segments(_ptr(idx), T, S, MODES[mode], _ptr(seg),
                                     _ptr(info_host), _stream(stream, idx.device))
    _check(st)
    return seg


def segments_view(seg, T, S):
    """Views of the record's documented fields (device tensors)."""
    o = {k: segments_offset(T, S, k) for k in SEG_FIELDS}
    return dict(info=seg[:INFO_WORDS], perm=seg[o["perm"]:o["perm"] + T],
                seg_slot=seg[o["seg_slot"]:o["seg_slot"] + S],
                seg_start=seg[o["seg_start"]:o["seg_start"] + S + 1])


def shrink(x, A, seg, *, scale=None, ranks=None, v=None, active=True, stream=None):
    """v[i][t][k] = scale[s] * A_i[s][k] . x[t] for active tokens.

    x: [T, >=D] (contiguous rows, any row stride); A: list of [S, r_max, D].
    Returns v ([n_slices, T, r_max] float32; allocated if not given).
    """
    A = list(A)
    if not A or len(A) > MAX_SLICES:
        raise LoraError(LORA_ERR_INVALID_ARG if not A else LORA_ERR_UNSUPPORTED,
                        f"need 1..{MAX_SLICES} slices")
    S, r_max, D = A[0].shape
    T, _, ldx = _rows(x, "x")
    for a in A:
        if a.shape != (S, r_max, D) or not a.is_contiguous() or a.dtype != x.dtype:
            raise LoraError(LORA_ERR_INVALID_ARG, "A slices must share shape, dtype and be contiguous")
    if v is None:
        v = torch.empty((len(A), T, r_max), dtype=torch.float32, device=x.device)
    if v.dtype != torch.float32 or not v.is_contiguous() or v.shape != (len(A), T, r_max):
        raise LoraError(LORA_ERR_INVALID_ARG, "v must be contiguous float32 [n_slices, T, r_max]")
    dev = x.device
    _check_rows(x, "x", dev)
    for i, a in enumerate(A):
        _check_tensor(a, f"A[{i}]", dev)
    _check_tensor(v, "v", dev)
    _check_slot_tables(dev, S, ranks, scale)
    _check_record(seg, T, S, dev)
    ptrs = (ctypes.c_void_p * len(A))(*[a.data_ptr() for a in A])
    st = _load().lora_shrink(_dtype_code(x), _ptr(x), ldx, T, D, len(A), ptrs, S, r_max,
                             _ptr(ranks), _ptr(scale), _ptr(seg), 1 if active else 0,
                             _ptr(v), _stream(stream, x.device))
    _check(st)
    return v


def _b_layout(b_layout):
    try:
        return B_LAYOUTS[b_layout]
    except KeyError:
        raise LoraError(LORA_ERR_INVALID_ARG, f"unknown B layout {b_layout!r}") from None


def expand(v, B, y, seg, out_offsets, *, ranks=None, active=True, v_slice_stride=None,
           b_layout="padded", stream=None):
    """y[t, off_i:off_i+out_i] += B_i[s] @ v[i][t] for active tokens (in place)."""
    B = list(B)
    if not B or len(B) > MAX_SLICES:
        raise LoraError(LORA_ERR_INVALID_ARG if not B else LORA_ERR_UNSUPPORTED,
                        f"need 1..{MAX_SLICES} slices")
    S, _, r_max = B[0].shape
    T, _, ldy = _rows(y, "y")
    for b in B:
        if b.shape[0] != S or b.shape[2] != r_max or not b.is_contiguous() or b.dtype != y.dtype:
            raise LoraError(LORA_ERR_INVALID_ARG, "B slices must share S, r_max, dtype and be contiguous")
    if v.dtype != torch.float32 or not v.is_contiguous():
        raise LoraError(LORA_ERR_INVALID_ARG, "v must be contiguous float32")
    if v_slice_stride is None:
        v_slice_stride = T * r_max if v.dim() == 3 and v.size(0) > 1 else 0
    n = len(B)
    if len(out_offsets) != n:
        raise LoraError(LORA_ERR_INVALID_ARG, "one output offset per slice")
    dev = y.device
    _check_rows(y, "y", dev)
    for i, b in enumerate(B):
        _check_tensor(b, f"B[{i}]", dev)
    # the kernels read rows of r_max floats of every slice's v
    _check_tensor(v, "v", dev, min_numel=(n - 1) * max(int(v_slice_stride), 0) + T * r_max)
    _check_slot_tables(dev, S, ranks)
    _check_record(seg, T, S, dev)
    ptrs = (ctypes.c_void_p * n)(*[b.data_ptr() for b in B])
    sizes = (ctypes.c_int64 * n)(*[b.shape[1] for b in B])
    offs = (ctypes.c_int64 * n)(*[int(o) for o in out_offsets])
    st = _load().lora_expand(_dtype_code(y), _ptr(v), v_slice_stride, T, n, ptrs, sizes, offs,
                             S, r_max, _ptr(ranks), _b_layout(b_layout), _ptr(seg), 1 if active else 0,
                             _ptr(y), ldy, _stream(stream, y.device))
    _check(st)
    return y


def apply(x, A, B, y, seg, out_offsets, *, scale=None, ranks=None, v=None, active=True,
          b_layout="padded", stream=None):
    """Shrink then expand; returns (v, y)."""
    v = shrink(x, A, seg, scale=scale, ranks=ranks, v=v, active=active, stream=stream)
    expand(v, B, y, seg, out_offsets, ranks=ranks, active=active, b_layout=b_layout, stream=stream)
    return v, y


def fused_max_tokens():
    return int(_load().lora_fused_max_tokens())


def fused_max_tokens_for(dtype):
    """Largest T that shrink_expand runs as one launch for data of `dtype`
    (a torch dtype, or one of "f32", "f16", "bf16")."""
    codes = {"f32": 0, "f16": 1, "bf16": 2}
    code = codes[dtype] if isinstance(dtype, str) else _DTYPES[dtype]
    return int(_load().lora_fused_max_tokens_for(code))


def workspace_bytes(T, S, n_slices, r_max):
    return int(_load().lora_shrink_expand_workspace_bytes(T, S, n_slices, r_max))


def alloc_workspace(T, S, n_slices, r_max, device):
    """A zeroed workspace for shrink_expand (uint8 tensor, 256-byte aligned)."""
    n = workspace_bytes(T, S, n_slices, r_max)
    if n == 0:
        raise LoraError(LORA_ERR_INVALID_ARG, f"bad sizes T={T} S={S} n_slices={n_slices} r_max={r_max}")
    ws = torch.zeros(n, dtype=torch.uint8, device=device)
    if ws.data_ptr() % 256:
        raise LoraError(LORA_ERR_INVALID_ARG, "allocator returned a workspace not aligned to 256 bytes")
    return ws


def workspace_errors(ws):
    """Device-side waits that gave up in calls on this workspace (0 normally).
    Synchronises with the workspace's stream."""
    return int(ws[:4].view(torch.int32).item())


def workspace_errors_async(ws, host_out, *, stream=None):
    """Enqueue a copy of the workspace's give-up count into host_out (pinned
    int32 host tensor of >= 1 element); read it after the stream syncs."""
    if host_out.device.type != "cpu" or not host_out.is_pinned() or host_out.dtype != torch.int32:
        raise LoraError(LORA_ERR_INVALID_ARG, "host_out must be a pinned int32 host tensor")
    _check_tensor(ws, "workspace", ws.device, dtype=torch.uint8, min_bytes=256)
    _check(_load().lora_workspace_errors(_ptr(ws), _ptr(host_out), _stream(stream, ws.device)))
    return host_out


def _shrink_expand_args(x, A, B, y, seg, out_offsets, scale, ranks, v, idx, record_bytes=None):
    """Checks and marshals the arguments shared by shrink_expand and
    shrink_expand_noalloc (everything before the workspace)."""
    A, B = list(A), list(B)
    if not A or len(A) > MAX_SLICES or len(B) != len(A):
        raise LoraError(LORA_ERR_INVALID_ARG, f"need 1..{MAX_SLICES} slices, as many B as A")
    S, r_max, D = A[0].shape
    T, _, ldx = _rows(x, "x")
    _, _, ldy = _rows(y, "y")
    for a in A:
        if a.shape != (S, r_max, D) or not a.is_contiguous() or a.dtype != x.dtype:
            raise LoraError(LORA_ERR_INVALID_ARG, "A slices must share shape, dtype and be contiguous")
    for b in B:
        if b.shape[0] != S or b.shape[2] != r_max or not b.is_contiguous() or b.dtype != y.dtype:
            raise LoraError(LORA_ERR_INVALID_ARG, "B slices must share S, r_max, dtype and be contiguous")
    if y.dtype != x.dtype:
        raise LoraError(LORA_ERR_INVALID_ARG, "x and y must share one dtype")
    if v is not None and (v.dtype != torch.float32 or not v.is_contiguous()
                          or v.shape != (len(A), T, r_max)):
        raise LoraError(LORA_ERR_INVALID_ARG, "v must be contiguous float32 [n_slices, T, r_max]")
    if idx is not None and (idx.dtype != torch.int32 or idx.dim() != 1 or not idx.is_contiguous()
                            or idx.numel() != T):
        raise LoraError(LORA_ERR_INVALID_ARG, "idx must be a contiguous int32 tensor of T entries")
    if len(out_offsets) != len(B):
        raise LoraError(LORA_ERR_INVALID_ARG, "one output offset per slice")
    dev = x.device
    _check_rows(x, "x", dev)
    _check_rows(y, "y", dev)
    for i, (a, b) in enumerate(zip(A, B)):
        _check_tensor(a, f"A[{i}]", dev)
        _check_tensor(b, f"B[{i}]", dev)
    _check_tensor(v, "v", dev)
    _check_tensor(idx, "idx", dev)
    _check_slot_tables(dev, S, ranks, scale)
    if record_bytes is None:
        _check_record(seg, T, S, dev)
    n = len(A)
    a_ptrs = (ctypes.c_void_p * n)(*[a.data_ptr() for a in A])
    b_ptrs = (ctypes.c_void_p * n)(*[b.data_ptr() for b in B])
    sizes = (ctypes.c_int64 * n)(*[b.shape[1] for b in B])
    offs = (ctypes.c_int64 * n)(*[int(o) for o in out_offsets])
    return [_dtype_code(x), _ptr(x), ldx, T, D, n, a_ptrs, b_ptrs, sizes, offs, S, r_max,
            _ptr(ranks), _ptr(scale), _ptr(seg), _ptr(idx)], dev, ldy


def shrink_expand(x, A, B, y, seg, out_offsets, *, workspace, scale=None, ranks=None, v=None,
                  idx=None, active=True, b_layout="padded", stream=None):
    """Shrink then expand in one call; y updated in place.  Returns y.

    v (optional, [n_slices, T, r_max] float32) receives the intermediate.
    idx (optional, int32 [T]): when given, the call builds the batch's segment
    record into seg itself (as build_segments(idx, S) would) before or beside
    the layer; without it seg must hold the record.
    workspace: from alloc_workspace (zeroed once; every call leaves it reusable).
    """
    head, dev, ldy = _shrink_expand_args(x, A, B, y, seg, out_offsets, scale, ranks, v, idx)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise LoraError(LORA_ERR_INVALID_ARG, "workspace must be a contiguous uint8 tensor")
    _check_tensor(workspace, "workspace", dev)
    st = _load().lora_shrink_expand(*head[:13], _b_layout(b_layout), *head[13:], 1 if active else 0, _ptr(v),
                                    _ptr(y), ldy, _ptr(workspace), workspace.numel(), _stream(stream, dev))
    _check(st)
    return y


def shrink_expand_noalloc(x, A, B, y, seg, out_offsets, *, scale=None, ranks=None, v=None,
                          idx=None, active=True, errors_host=None, b_layout="padded", stream=None):
    """shrink_expand without a workspace: the library's per-device scratch of
    NOALLOC_SCRATCH_BYTES bytes stands in for it, and the call allocates
    nothing.  Calls that may overlap on one device race.  errors_host
    (optional pinned int32 host tensor) receives, asynchronously, the device's
    count of waits that gave up in such calls."""
    head, dev, ldy = _shrink_expand_args(x, A, B, y, seg, out_offsets, scale, ranks, v, idx)
    if errors_host is not None and (errors_host.device.type != "cpu" or not errors_host.is_pinned()
                                    or errors_host.dtype != torch.int32):
        raise LoraError(LORA_ERR_INVALID_ARG, "errors_host must be a pinned int32 host tensor")
    st = _load().lora_shrink_expand_noalloc(*head[:13], _b_layout(b_layout), *head[13:], 1 if active else 0,
                                            _ptr(v), _ptr(y), ldy, _ptr(errors_host), _stream(stream, dev))
    _check(st)
    return y


def embedding_shrink(tok, A_emb, idx, *, scale=None, ranks=None, v=None, active=True, stream=None):
    """v[t][k] = scale[s] * A_emb[s][tok[t]][k] for tokens with a valid slot and
    an id inside the table (zero rows otherwise).  A_emb: [S, V, r_max] (the
    adapters' A tables stacked transposed).  Returns v ([1, T, r_max] fp32)."""
    if tok.dtype != torch.int32 or tok.dim() != 1 or idx.dtype != torch.int32 or idx.dim() != 1 \
            or tok.numel() != idx.numel():
        raise LoraError(LORA_ERR_INVALID_ARG, "tok and idx must be int32 tensors of T entries")
    if A_emb.dim() != 3:
        raise LoraError(LORA_ERR_INVALID_ARG, "A_emb must be [S, V, r_max]")
    S, V, r_max = A_emb.shape
    T = tok.numel()
    dev = A_emb.device
    if v is None:
        v = torch.empty((1, T, r_max), dtype=torch.float32, device=dev)
    if v.dtype != torch.float32 or not v.is_contiguous() or v.numel() != T * r_max:
        raise LoraError(LORA_ERR_INVALID_ARG, "v must be contiguous float32 with T * r_max elements")
    for name, t in (("tok", tok), ("idx", idx), ("A_emb", A_emb), ("v", v)):
        _check_tensor(t, name, dev)
    _check_slot_tables(dev, S, ranks, scale)
    st = _load().lora_embedding_shrink(_dtype_code(A_emb), _ptr(tok), T, V, _ptr(A_emb), S, r_max,
                                       _ptr(ranks), _ptr(scale), _ptr(idx), 1 if active else 0,
                                       _ptr(v), _stream(stream, dev))
    _check(st)
    return v


def embedding_apply(tok, A_emb, B_emb, y, seg, idx, *, scale=None, ranks=None, v=None, active=True,
                    stream=None):
    """The LoRA delta of an embedding layer: embedding_shrink, then the expand
    y[t, :H] += B_emb[s] @ v[t] (B_emb: [S, H, r_max]).  seg is the batch's
    segment record (from build_segments(idx, S)).  Returns (v, y)."""
    v = embedding_shrink(tok, A_emb, idx, scale=scale, ranks=ranks, v=v, active=active, stream=stream)
    expand(v, [B_emb], y, seg, [0], ranks=ranks, active=active, v_slice_stride=0, stream=stream)
    return v, y


def copy_padded(src, dst, *, transpose=False, stream=None):
    """dst (a 2-D slot region, row-contiguous) = src (or src.T) in its top-left
    corner, zeros elsewhere; src and dst on the same GPU, same dtype."""
    if src.dtype != dst.dtype:
        raise LoraError(LORA_ERR_INVALID_ARG, "src and dst must share a dtype")
    if src.dim() != 2 or dst.dim() != 2 or src.stride(1) != 1 or dst.stride(1) != 1:
        raise LoraError(LORA_ERR_INVALID_ARG, "src and dst must be 2-D with contiguous rows")
    dev = dst.device
    _check_rows(src, "src", dev)
    _check_rows(dst, "dst", dev)
    m_rows, m_cols = (src.shape[1], src.shape[0]) if transpose else (src.shape[0], src.shape[1])
    st = _load().lora_copy_padded(_dtype_code(src), _ptr(src), m_rows, m_cols, max(src.stride(0), src.shape[1]),
                                  1 if transpose else 0, _ptr(dst), dst.shape[0], dst.shape[1],
                                  max(dst.stride(0), dst.shape[1]), _stream(stream, dev))
    _check(st)
    return dst


MASK_MAX_LANES = 128


def mask_workspace_bytes(dtype, T, D, S, n_slices, r_max):
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(_load().lora_mask_workspace_bytes(code, T, D, S, n_slices, r_max))


def alloc_mask_workspace(dtype, T, D, S, n_slices, r_max, device):
    n = mask_workspace_bytes(dtype, T, D, S, n_slices, r_max)
    if n == 0:
        raise LoraError(LORA_ERR_UNSUPPORTED, f"no mask form for S={S} r_max={r_max}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def shrink_expand_mask(x, A, B, y, idx, out_offsets, *, workspace, scale=None, ranks=None, v=None,
                       active=True, stream=None):
    """The mask form of shrink + expand: one dense product of every token tile
    with all the stacked adapter lanes, each token keeping its own (S * r_max
    <= 128).  Reads idx directly (no segment record).  Returns y."""
    if idx.dtype != torch.int32 or idx.dim() != 1:
        raise LoraError(LORA_ERR_INVALID_ARG, "idx must be a 1-D int32 tensor")
    # (this form reads no segment record: the arguments are checked as for
    # shrink_expand without one)
    head, dev, ldy = _shrink_expand_args(x, A, B, y, None, out_offsets, scale, ranks, v, None,
                                         record_bytes=0)
    _check_tensor(idx, "idx", dev, min_numel=head[3])
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise LoraError(LORA_ERR_INVALID_ARG, "workspace must be a contiguous uint8 tensor")
    st = _load().lora_shrink_expand_mask(*head[:14], _ptr(idx), 1 if active else 0, _ptr(v), _ptr(y), ldy,
                                         _ptr(workspace), workspace.numel(), _stream(stream, dev))
    _check(st)
    return y


def pack_b_rank_rows(B, ranks_host, *, stream=None):
    """A copy of a stacked B ([S, out, r_max], padded layout) in the rank-rows
    layout: slot s's rows packed with stride roundup(ranks_host[s], 8) (16-bit)
    or roundup(.., 4) (fp32) from the start of its region, zeros between the
    rank and the stride.  Each slot is placed with the library's
    lora_copy_padded; this is adapter-load-time work, not part of a step."""
    S, out, r_max = B.shape
    unit = 4 if B.dtype == torch.float32 else 8
    packed = torch.zeros_like(B)
    for s_ in range(S):
        r = max(0, min(int(ranks_host[s_]), r_max))
        ld = max(unit, -(-r // unit) * unit) if r else unit
        ld = min(ld, r_max)
        dst = packed[s_].view(-1)[:out * ld].view(out, ld)
        copy_padded(B[s_][:, :r] if r else B[s_][:, :0], dst, stream=stream)
    return packed
