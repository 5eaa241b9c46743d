"""Pure-Python brute force for multi-LoRA application, used to pin the oracle.

No numpy arithmetic: inputs are turned into Python floats element by element
(with a decoder written here, not the oracle's), and each active token's dense
per-token matrix M_t = scale_s * B_s[:, :r] @ A_s[:r, :] is formed first and
then applied to x_t.  That association, (B A) x, differs from the oracle's
B (A x), so agreement is checked to a tolerance, not bitwise.
"""

import struct

import numpy as np


def to_float(value, dtype):
    """One storage element -> Python float, without numpy arithmetic."""
    if dtype == "bf16":
        return struct.unpack("<f", struct.pack("<I", int(value) << 16))[0]
    return float(value)


def to_lists(a, dtype):
    a = np.asarray(a)
    if a.ndim == 1:
        return [to_float(e, dtype) for e in a.tolist()]
    return [to_lists(row, dtype) for row in a]


def brute_apply(p, *, ignore_scale=False):
    """Return y (list of rows of Python floats) for a workloads.Problem `p`."""
    dt = p.dtype
    T, D, S, r_max = p.T, p.D, p.S, p.r_max
    y = [to_lists(p.y_in[t], dt) for t in range(T)]
    for t in range(T):
        s = int(p.idx[t])
        if not (0 <= s < S):
            continue
        r = r_max if p.ranks is None else int(p.ranks[s])
        sc = 1.0 if ignore_scale else float(p.scale[s])
        xt = [to_float(p.x[t, d], dt) for d in range(D)]
        for i, off in enumerate(p.out_offsets):
            A = p.A[i][s]
            B = p.B[i][s]
            out = p.out_sizes[i]
            for j in range(out):
                bj = [to_float(B[j, k], dt) for k in range(r)]
                m_row = [0.0] * D
                for k in range(r):
                    ak = A[k]
                    for d in range(D):
                        m_row[d] += bj[k] * to_float(ak[d], dt)
                acc = 0.0
                for d in range(D):
                    acc += sc * m_row[d] * xt[d]
                y[t][off + j] += acc
    return y


def brute_segments(idx, S):
    """Second formulation of the slot grouping: numpy stable argsort + bincount."""
    idx = np.asarray(idx, dtype=np.int64)
    valid = (idx >= 0) & (idx < S)
    bad = bool(np.any(~valid & (idx != -1)))
    act = np.nonzero(valid)[0]
    order = np.argsort(idx[act], kind="stable")
    perm = act[order].astype(np.int32)
    counts = np.bincount(idx[act], minlength=S) if S > 0 else np.zeros(0, int)
    seg_slot = np.nonzero(counts)[0].astype(np.int32)
    seg_start = np.concatenate([[0], np.cumsum(counts[seg_slot])]).astype(np.int32)
    rest = np.nonzero(~valid)[0].astype(np.int32)
    return dict(perm=perm, rest=rest, seg_slot=seg_slot, seg_start=seg_start,
                num_active=int(act.size), num_segments=int(seg_slot.size),
                max_seg_len=int(counts.max()) if counts.size else 0,
                status=3 if bad else 0)


def brute_expand(p, v):
    """Expand alone in pure Python: y_in + B_s[:, :r] v[i][t][:r] per active token.

    `v` is a float64 array [n_slices, T, r_max]; entries past a slot's rank
    may hold anything and must be ignored.
    """
    dt = p.dtype
    y = [to_lists(p.y_in[t], dt) for t in range(p.T)]
    for t in range(p.T):
        s = int(p.idx[t])
        if not (0 <= s < p.S):
            continue
        r = p.r_max if p.ranks is None else int(p.ranks[s])
        for i, off in enumerate(p.out_offsets):
            B = p.B[i][s]
            vt = [float(v[i, t, k]) for k in range(r)]
            for j in range(p.out_sizes[i]):
                acc = 0.0
                for k in range(r):
                    acc += to_float(B[j, k], dt) * vt[k]
                y[t][off + j] += acc
    return y


def brute_embedding(p):
    """Embedding LoRA in pure Python, through the layer's one-hot input.

    For token id w the layer's input is e_w (length V); the shrink is the PEFT
    table A_s (r x V, i.e. A_emb[s] transposed) times e_w, summed over all V
    entries of the one-hot vector, then the expand B_s (H x r).  Returns
    (v rows, y rows) as lists of Python floats.
    """
    dt = p.dtype
    y = [to_lists(p.y_in[t], dt) for t in range(p.T)]
    v = [[0.0] * p.r_max for _ in range(p.T)]
    for t in range(p.T):
        s = int(p.idx[t])
        if not (0 <= s < p.S):
            continue
        w = int(p.tok[t])
        r = p.r_max if p.ranks is None else int(p.ranks[s])
        sc = float(p.scale[s])
        onehot = [1.0 if c == w else 0.0 for c in range(p.V)]
        for k in range(r):
            acc = 0.0
            for c in range(p.V):
                acc += to_float(p.A_emb[s, c, k], dt) * onehot[c]
            v[t][k] = sc * acc
        for j in range(p.H):
            acc = 0.0
            for k in range(r):
                acc += to_float(p.B[s, j, k], dt) * v[t][k]
            y[t][j] += acc
    return v, y
