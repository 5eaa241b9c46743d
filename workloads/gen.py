"""Seeded draws of multi-LoRA batches.

Storage conventions (shared with the library's C interface):
  x     [T, D]            activations, row-major
  A_i   [S, r_max, D]     shrink weights of slice i, input dim contiguous
  B_i   [S, out_i, r_max] expand weights of slice i, rank dim contiguous
  y     [T, ldy]          output rows; slice i occupies columns
                          [out_offsets[i], out_offsets[i] + out_i)
  idx   [T] int32         adapter slot of each token, -1 for base-model-only
  scale [S] float32       per-slot scaling
  ranks [S] int32 or None real rank of each slot (weights zero-padded to r_max)

Storage dtypes: "f32" -> numpy float32, "f16" -> numpy float16,
"bf16" -> numpy uint16 holding the bfloat16 bit pattern (numpy has no bf16).

Values are drawn in float64 with numpy's PCG64 generator, then rounded to
nearest-even into the storage dtype (bf16 through float32).  The draw order is
fixed: idx, the base-token mask, ranks, then per problem x, A (slice order),
B (slice order), y_in.
"""

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from .configs import CONFIGS

STORAGE_NP = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def round_to_dtype(a, dtype):
    """Round a float64/float32 array to the storage dtype (round-to-nearest-even)."""
    a = np.asarray(a)
    if dtype == "f32":
        return a.astype(np.float32)
    if dtype == "f16":
        return a.astype(np.float16)
    if dtype == "bf16":
        u = np.ascontiguousarray(a.astype(np.float32)).view(np.uint32)
        bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
        return ((u + bias) >> 16).astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def bf16_bits_to_f32(u16):
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(u16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Problem:
    """One LoRA-wrapped linear layer applied to one batch."""

    name: str
    dtype: str
    T: int
    D: int
    S: int
    r_max: int
    out_sizes: tuple
    out_offsets: tuple
    ldy: int
    idx: np.ndarray
    scale: np.ndarray
    ranks: Optional[np.ndarray]
    x: np.ndarray
    A: List[np.ndarray]
    B: List[np.ndarray]
    y_in: np.ndarray
    timed_expand: bool = True

    @property
    def n_slices(self):
        return len(self.out_sizes)

    @property
    def elem_bytes(self):
        return ELEM_BYTES[self.dtype]


@dataclass
class Workload:
    """A named batch: one idx vector shared by one or more layers."""

    name: str
    dtype: str
    T: int
    S: int
    r_max: int
    idx: np.ndarray
    problems: List[Problem] = field(default_factory=list)


def _normal(rng, var, shape):
    return rng.normal(0.0, np.sqrt(var), size=shape)


def _draw_idx(rng, recipe, T):
    kind = recipe[0]
    if kind == "iid_with_base":
        S = recipe[1]
        return rng.integers(-1, S, size=T).astype(np.int32)
    if kind == "uniform_then_base":
        S, n_base = recipe[1], recipe[2]
        idx = rng.integers(0, S, size=T).astype(np.int32)
        base = rng.choice(T, size=n_base, replace=False)
        idx[base] = -1
        return idx
    if kind == "contiguous":
        S, run = recipe[1], recipe[2]
        assert S * run == T
        return np.repeat(np.arange(S, dtype=np.int32), run)
    if kind == "zipf":
        S, s = recipe[1], recipe[2]
        w = (np.arange(S, dtype=np.float64) + 1.0) ** (-s)
        return rng.choice(S, size=T, p=w / w.sum()).astype(np.int32)
    if kind == "all_base":
        return np.full(T, -1, dtype=np.int32)
    raise ValueError(f"unknown idx recipe {recipe!r}")


def _pad_ranks(w_A, w_B, ranks):
    """Zero the rank rows of A and rank columns of B beyond each slot's rank."""
    if ranks is None:
        return
    for s, r in enumerate(ranks):
        for a in w_A:
            a[s, r:, :] = 0.0
        for b in w_B:
            b[s, :, r:] = 0.0


def make_workload(name, seed=None):
    """Draw the named workload.  Returns a Workload of numpy arrays."""
    c = CONFIGS[name]
    rng = np.random.default_rng(c["seed"] if seed is None else seed)
    T, S, r_max, dtype = c["T"], c["S"], c["r_max"], c["dtype"]
    idx = _draw_idx(rng, c["idx"], T)
    ranks = None
    if c["ranks"] is not None:
        ranks = rng.choice(np.asarray(c["ranks"], dtype=np.int32), size=S).astype(np.int32)
    scale = np.full(S, c["scale"], dtype=np.float32)
    wl = Workload(name=name, dtype=dtype, T=T, S=S, r_max=r_max, idx=idx)
    for p in c["problems"]:
        D, outs = p["D"], tuple(p["out_sizes"])
        offs = tuple(int(v) for v in np.concatenate([[0], np.cumsum(outs)[:-1]]))
        x = _normal(rng, p["x_var"], (T, D))
        A = [_normal(rng, p["A_var"], (S, r_max, D)) for _ in outs]
        B = [_normal(rng, p["B_var"], (S, o, r_max)) for o in outs]
        _pad_ranks(A, B, ranks)
        y = _normal(rng, 1.0, (T, sum(outs)))
        wl.problems.append(Problem(
            name=p["name"], dtype=dtype, T=T, D=D, S=S, r_max=r_max,
            out_sizes=outs, out_offsets=offs, ldy=sum(outs), idx=idx,
            scale=scale, ranks=ranks,
            x=round_to_dtype(x, dtype),
            A=[round_to_dtype(a, dtype) for a in A],
            B=[round_to_dtype(b, dtype) for b in B],
            y_in=round_to_dtype(y, dtype),
            timed_expand=p["timed_expand"]))
    return wl


def random_problem(rng, *, T, D, out_sizes, r_max, S, dtype="f32",
                   base_frac=0.25, with_ranks=False, random_scale=True,
                   bad_idx_frac=0.0, idx=None, ldx=None, ldy=None,
                   x_var=1.0, w_var=1.0, y_var=1.0):
    """A small random problem for tests, drawn from `rng`.

    `ldx`/`ldy` (row strides in elements) default to the dense widths; a wider
    stride leaves padding columns that the library must not touch.  A fraction
    `bad_idx_frac` of tokens gets an out-of-range slot (< -1 or >= S).
    """
    out_sizes = tuple(int(o) for o in out_sizes)
    offs = tuple(int(v) for v in np.concatenate([[0], np.cumsum(out_sizes)[:-1]])) \
        if out_sizes else ()
    width = int(sum(out_sizes))
    ldx = D if ldx is None else ldx
    ldy = width if ldy is None else ldy
    if idx is None:
        idx = rng.integers(0, S, size=T).astype(np.int32)
        if T:
            base = rng.random(T) < base_frac
            idx[base] = -1
            if bad_idx_frac > 0:
                bad = rng.random(T) < bad_idx_frac
                idx[bad] = rng.choice(np.array([-7, -2, S, S + 5], dtype=np.int32),
                                      size=int(bad.sum()))
    idx = np.asarray(idx, dtype=np.int32)
    ranks = None
    if with_ranks:
        ranks = rng.integers(1, r_max + 1, size=S).astype(np.int32)
    scale = (rng.uniform(0.5, 4.0, size=S) if random_scale
             else np.ones(S)).astype(np.float32)
    x = np.zeros((T, ldx))
    x[:, :D] = _normal(rng, x_var, (T, D))
    A = [_normal(rng, w_var, (S, r_max, D)) for _ in out_sizes]
    B = [_normal(rng, w_var, (S, o, r_max)) for o in out_sizes]
    _pad_ranks(A, B, ranks)
    y = _normal(rng, y_var, (T, ldy))
    return Problem(
        name="random", dtype=dtype, T=T, D=D, S=S, r_max=r_max,
        out_sizes=out_sizes, out_offsets=offs, ldy=ldy, idx=idx, scale=scale,
        ranks=ranks, x=round_to_dtype(x, dtype),
        A=[round_to_dtype(a, dtype) for a in A],
        B=[round_to_dtype(b, dtype) for b in B],
        y_in=round_to_dtype(y, dtype))


@dataclass
class EmbeddingProblem:
    """A LoRA on an embedding table applied to one batch.

    tok    [T] int32 token ids (row of the table; ids outside [0, V) allowed)
    A_emb  [S, V, r_max]   the adapters' A tables stacked transposed (one rank
                           vector per vocabulary row)
    B      [S, H, r_max]   expand weights
    y_in   [T, ldy]        embedding output rows; the delta goes to columns [0, H)
    """

    name: str
    dtype: str
    T: int
    V: int
    H: int
    S: int
    r_max: int
    ldy: int
    idx: np.ndarray
    tok: np.ndarray
    scale: np.ndarray
    ranks: Optional[np.ndarray]
    A_emb: np.ndarray
    B: np.ndarray
    y_in: np.ndarray

    @property
    def elem_bytes(self):
        return ELEM_BYTES[self.dtype]


def random_embedding_problem(rng, *, T, V, H, r_max, S, dtype="f32", base_frac=0.25,
                             with_ranks=False, random_scale=True, bad_idx_frac=0.0,
                             bad_tok_frac=0.0, ldy=None, w_var=1.0, y_var=1.0, tok=None,
                             idx=None):
    """A random embedding-LoRA batch drawn from `rng` (same conventions as
    random_problem; a fraction bad_tok_frac of tokens gets an id outside
    [0, V))."""
    ldy = H if ldy is None else ldy
    if idx is None:
        idx = rng.integers(0, S, size=T).astype(np.int32)
        if T:
            idx[rng.random(T) < base_frac] = -1
            if bad_idx_frac > 0:
                bad = rng.random(T) < bad_idx_frac
                idx[bad] = rng.choice(np.array([-5, S, S + 9], dtype=np.int32), size=int(bad.sum()))
    idx = np.asarray(idx, dtype=np.int32)
    if tok is None:
        tok = rng.integers(0, V, size=T).astype(np.int32)
        if T and bad_tok_frac > 0:
            bad = rng.random(T) < bad_tok_frac
            tok[bad] = rng.choice(np.array([-1, -7, V, V + 3], dtype=np.int32), size=int(bad.sum()))
    tok = np.asarray(tok, dtype=np.int32)
    ranks = rng.integers(1, r_max + 1, size=S).astype(np.int32) if with_ranks else None
    scale = (rng.uniform(0.5, 4.0, size=S) if random_scale else np.ones(S)).astype(np.float32)
    A = _normal(rng, w_var, (S, V, r_max))
    B = _normal(rng, w_var, (S, H, r_max))
    if ranks is not None:
        for s, r in enumerate(ranks):
            A[s, :, r:] = 0.0
            B[s, :, r:] = 0.0
    y = _normal(rng, y_var, (T, ldy))
    return EmbeddingProblem(
        name="random_embedding", dtype=dtype, T=T, V=V, H=H, S=S, r_max=r_max, ldy=ldy,
        idx=idx, tok=tok, scale=scale, ranks=ranks, A_emb=round_to_dtype(A, dtype),
        B=round_to_dtype(B, dtype), y_in=round_to_dtype(y, dtype))
