"""Move generated numpy arrays to and from torch tensors (no arithmetic).

bf16 arrays are numpy uint16 bit patterns; they are reinterpreted, never
converted, so both sides of a comparison see exactly the same bits.
"""

import numpy as np
import torch

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def to_torch(arr, dtype, device):
    arr = np.ascontiguousarray(arr)
    if dtype == "bf16":
        t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(arr)
    return t.to(device)


def from_torch(t, dtype):
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def problem_to_device(p, device):
    """Device tensors of a workloads.Problem (idx, x, A, B, y_in, scale, ranks)."""
    return dict(
        idx=torch.from_numpy(np.ascontiguousarray(p.idx)).to(device),
        x=to_torch(p.x, p.dtype, device),
        A=[to_torch(a, p.dtype, device) for a in p.A],
        B=[to_torch(b, p.dtype, device) for b in p.B],
        y=to_torch(p.y_in, p.dtype, device),
        scale=torch.from_numpy(np.ascontiguousarray(p.scale)).to(device),
        ranks=None if p.ranks is None else torch.from_numpy(np.ascontiguousarray(p.ranks)).to(device),
    )
