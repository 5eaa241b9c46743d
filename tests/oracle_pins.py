"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each pin takes an oracle namespace `o` (the real `oracle` package, or a copy
with a planted mistake) and raises AssertionError when it disagrees with:
  * brute force in pure Python (tiny inputs, different association),
  * the page's gather-then-batched-matvec baseline, re-expressed in numpy,
  * a dense GEMM for a single adapter,
  * closed forms (constant inputs),
  * invariants (base rows untouched, rank padding, linearity, permutation,
    slice decomposition),
  * a hand-worked example in tests/golden/,
  * a second formulation of the slot grouping (stable argsort + bincount).
"""

import os

import numpy as np

from bruteforce import brute_apply, brute_embedding, brute_expand, brute_segments
from workloads import random_embedding_problem, random_problem

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _apply(o, p, **kw):
    kw.setdefault("scale", p.scale)
    kw.setdefault("ranks", p.ranks)
    return o.oracle_apply(p.x, p.A, p.B, p.y_in, p.idx, p.S, p.out_offsets,
                          dtype=p.dtype, D=p.D, **kw)


def _close(a, b, rtol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= rtol * scale, f"{what}: max abs err {err:.3e} > {rtol:.1e} * {scale:.3e}"


# --------------------------------------------------------------------------
# brute force
# --------------------------------------------------------------------------

def brute_cases(n_cases=500, seed=1234):
    """Seeded tiny problems, including the degenerate ones."""
    rng = np.random.default_rng(seed)
    fixed = [
        dict(T=0, D=3, out_sizes=(2,), r_max=2, S=2),
        dict(T=1, D=1, out_sizes=(1,), r_max=1, S=1),
        dict(T=5, D=4, out_sizes=(3,), r_max=2, S=3, base_frac=1.0),  # all base
        dict(T=6, D=5, out_sizes=(4,), r_max=3, S=1, base_frac=0.0),  # one slot
        dict(T=4, D=7, out_sizes=(2, 3, 1), r_max=1, S=2),            # r = 1
        dict(T=8, D=6, out_sizes=(5,), r_max=4, S=3, bad_idx_frac=0.3),
    ]
    for c in fixed:
        yield random_problem(rng, **c)
    dtypes = ["f32", "f16", "bf16"]
    for n in range(n_cases - len(fixed)):
        n_sl = int(rng.integers(1, 4))
        yield random_problem(
            rng,
            T=int(rng.integers(0, 13)),
            D=int(rng.integers(1, 25)),
            out_sizes=tuple(int(v) for v in rng.integers(1, 17, size=n_sl)),
            r_max=int(rng.integers(1, 9)),
            S=int(rng.integers(1, 5)),
            dtype=dtypes[n % 3],
            base_frac=float(rng.uniform(0, 0.6)),
            with_ranks=bool(n % 2),
            bad_idx_frac=0.1 if n % 7 == 0 else 0.0,
            x_var=1.0, w_var=1.0)


def scribble_padding(p, rng):
    """Write non-zero garbage into the rank padding so that ranks must be honoured."""
    if p.ranks is None:
        return p
    for s, r in enumerate(p.ranks):
        for a in p.A:
            a[s, r:, :] = a.dtype.type(3) if a.dtype != np.uint16 else np.uint16(0x4040)
        for b in p.B:
            b[s, :, r:] = b.dtype.type(3) if b.dtype != np.uint16 else np.uint16(0x4040)
    return p


def pin_bruteforce(o, n_cases=500):
    rng = np.random.default_rng(99)
    for n, p in enumerate(brute_cases(n_cases)):
        scribble_padding(p, rng)
        _, y = _apply(o, p)
        yb = np.asarray(brute_apply(p), dtype=np.float64).reshape(p.T, p.ldy)
        _close(y, yb, 1e-12, f"brute force case {n}")


def pin_expand_bruteforce(o, n_cases=150):
    """Expand on its own, fed a v with garbage past each slot's rank."""
    rng = np.random.default_rng(101)
    for n, p in enumerate(brute_cases(n_cases, seed=4321)):
        scribble_padding(p, rng)
        v = rng.normal(size=(p.n_slices, p.T, p.r_max))
        y = o.oracle_expand(v, p.B, p.y_in, p.idx, p.S, p.out_offsets, dtype=p.dtype,
                            ranks=p.ranks)
        yb = np.asarray(brute_expand(p, v), dtype=np.float64).reshape(p.T, p.ldy)
        _close(y, yb, 1e-12, f"expand brute force case {n}")


# --------------------------------------------------------------------------
# the page's gather baseline, re-expressed
# --------------------------------------------------------------------------

def gather_bmv(inputs, loras, idxs):
    """out[t] = loras[idxs[t]] @ inputs[t]: every token multiplied by the
    stacked matrix its index selects, as one contraction over the gathered
    stack.

    This is the per-token gather semantics of the PyTorch baseline in
    "[Hardware][TPU][V1] Better tpu multilora compilation" (review thread),
    written from its definition.  loras is [S, L, D] with the input dimension
    contiguous.  Indices must all be valid here (gathering with -1 would pick
    the last slot, which is why the caller has no base tokens).
    """
    return np.einsum("tld,td->tl", loras[np.asarray(idxs)], inputs)


def pin_gather_baseline(o):
    rng = np.random.default_rng(7)
    for n in range(40):
        p = random_problem(rng, T=int(rng.integers(1, 20)), D=int(rng.integers(1, 40)),
                           out_sizes=(int(rng.integers(1, 30)),),
                           r_max=int(rng.integers(1, 9)), S=int(rng.integers(1, 6)),
                           dtype="f32", base_frac=0.0, random_scale=False)
        xs = o.decode(p.x, "f32")
        A = o.decode(p.A[0], "f32")
        B = o.decode(p.B[0], "f32")
        v_ref = gather_bmv(xs, A, p.idx)
        v, y = _apply(o, p)
        _close(v[0], v_ref, 1e-13, f"gather shrink case {n}")
        d_ref = gather_bmv(v_ref, B, p.idx)
        _close(y - o.decode(p.y_in, "f32"), d_ref, 1e-13, f"gather expand case {n}")


# --------------------------------------------------------------------------
# dense GEMM for one adapter
# --------------------------------------------------------------------------

def pin_single_adapter(o):
    rng = np.random.default_rng(11)
    for n in range(20):
        p = random_problem(rng, T=int(rng.integers(1, 30)), D=int(rng.integers(1, 64)),
                           out_sizes=(int(rng.integers(1, 48)), int(rng.integers(1, 9))),
                           r_max=int(rng.integers(1, 17)), S=3, dtype="f32",
                           base_frac=0.0)
        p.idx[:] = 1
        c = float(p.scale[1])
        X = o.decode(p.x, "f32")
        _, y = _apply(o, p)
        delta = y - o.decode(p.y_in, "f32")
        for i, off in enumerate(p.out_offsets):
            A = o.decode(p.A[i][1], "f32")
            B = o.decode(p.B[i][1], "f32")
            ref = c * (X @ A.T @ B.T)
            _close(delta[:, off:off + p.out_sizes[i]], ref, 1e-12,
                   f"single adapter case {n} slice {i}")


# --------------------------------------------------------------------------
# closed form
# --------------------------------------------------------------------------

def pin_closed_form(o):
    """x = 1, A = alpha, B = beta (inside each rank) gives scale*beta*alpha*r_s*D."""
    rng = np.random.default_rng(5)
    alpha, beta = 0.5, 0.25
    for n in range(12):
        T, D, S, r_max = 9, int(rng.integers(1, 50)), 4, 8
        outs = (3, 5)
        p = random_problem(rng, T=T, D=D, out_sizes=outs, r_max=r_max, S=S,
                           dtype="f32", with_ranks=True, base_frac=0.3)
        p.x[:] = 1.0
        p.scale[:] = np.array([1.0, 2.0, 4.0, 0.5], np.float32)
        for s in range(S):
            for a in p.A:
                a[s] = 0.0
                a[s, :p.ranks[s], :] = alpha
            for b in p.B:
                b[s] = 0.0
                b[s, :, :p.ranks[s]] = beta
        _, y = _apply(o, p)
        y0 = o.decode(p.y_in, "f32")
        for t in range(T):
            s = int(p.idx[t])
            want = 0.0 if not (0 <= s < S) else \
                float(p.scale[s]) * beta * alpha * int(p.ranks[s]) * D
            assert np.all(y[t] - y0[t] == want), f"closed form token {t}"


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

def pin_base_rows_untouched(o):
    rng = np.random.default_rng(13)
    for dtype in ("f32", "f16", "bf16"):
        p = random_problem(rng, T=40, D=17, out_sizes=(9, 4), r_max=5, S=3,
                           dtype=dtype, base_frac=0.4, bad_idx_frac=0.1)
        v, y = _apply(o, p)
        y0 = o.decode(p.y_in, dtype)
        for t in range(p.T):
            if not (0 <= p.idx[t] < p.S):
                assert np.array_equal(y[t], y0[t]), f"base row {t} changed ({dtype})"
                assert not np.any(v[:, t]), f"base row {t} has non-zero v ({dtype})"


def pin_rank_padding(o):
    """Padding a rank up to 64 with zeros changes nothing."""
    rng = np.random.default_rng(17)
    for n in range(10):
        p = random_problem(rng, T=12, D=int(rng.integers(1, 40)), out_sizes=(7,),
                           r_max=int(rng.integers(1, 9)), S=3, dtype="f32")
        v, y = _apply(o, p)
        pad = 64 - p.r_max
        A64 = [np.concatenate([a, np.zeros((p.S, pad, p.D), a.dtype)], axis=1) for a in p.A]
        B64 = [np.concatenate([b, np.zeros((p.S, b.shape[1], pad), b.dtype)], axis=2) for b in p.B]
        v2, y2 = o.oracle_apply(p.x, A64, B64, p.y_in, p.idx, p.S, p.out_offsets,
                                dtype="f32", D=p.D, scale=p.scale)
        _close(y2, y, 1e-14, f"padding case {n}")
        _close(v2[:, :, :p.r_max], v, 1e-14, f"padding v case {n}")
        assert not np.any(v2[:, :, p.r_max:])


def pin_linearity(o):
    rng = np.random.default_rng(19)
    for n in range(10):
        p = random_problem(rng, T=10, D=13, out_sizes=(6, 2), r_max=4, S=3, dtype="f32",
                           with_ranks=True)
        x1 = rng.normal(size=p.x.shape)
        x2 = rng.normal(size=p.x.shape)
        a, b = float(rng.normal()), float(rng.normal())
        y0 = o.decode(p.y_in, "f32")

        def f(x, scale=p.scale, y_in=p.y_in):
            return o.oracle_apply(x, p.A, p.B, y_in, p.idx, p.S, p.out_offsets,
                                  dtype="f64", D=p.D, scale=scale,
                                  ranks=p.ranks)[1]
        lhs = f(a * x1 + b * x2) - y0
        rhs = a * (f(x1) - y0) + b * (f(x2) - y0)
        _close(lhs, rhs, 1e-12, f"linearity in x case {n}")
        # linear in the scale
        _close(f(x1, scale=(2.0 * p.scale)) - y0, 2.0 * (f(x1) - y0), 1e-13,
               f"linearity in scale case {n}")
        # the delta does not depend on y_in
        y_other = rng.normal(size=p.y_in.shape).astype(np.float32)
        _close(f(x1, y_in=y_other) - o.decode(y_other, "f32"), f(x1) - y0, 1e-12,
               f"delta independent of y_in case {n}")


def pin_permutation(o):
    rng = np.random.default_rng(23)
    for n in range(10):
        p = random_problem(rng, T=15, D=9, out_sizes=(5,), r_max=3, S=4, dtype="bf16",
                           with_ranks=True)
        v, y = _apply(o, p)
        pi = rng.permutation(p.T)
        v2, y2 = o.oracle_apply(p.x[pi], p.A, p.B, p.y_in[pi], p.idx[pi], p.S,
                                p.out_offsets, dtype="bf16", D=p.D, scale=p.scale,
                                ranks=p.ranks)
        assert np.array_equal(y2, y[pi]), f"permutation case {n}"
        assert np.array_equal(v2, v[:, pi]), f"permutation v case {n}"


def pin_slice_decomposition(o):
    rng = np.random.default_rng(29)
    for n in range(10):
        p = random_problem(rng, T=11, D=8, out_sizes=(4, 6, 3), r_max=4, S=3,
                           dtype="f16", with_ranks=True)
        v, y = _apply(o, p)
        for i, off in enumerate(p.out_offsets):
            w = p.out_sizes[i]
            vi, yi = o.oracle_apply(p.x, [p.A[i]], [p.B[i]],
                                    np.ascontiguousarray(p.y_in[:, off:off + w]),
                                    p.idx, p.S, (0,), dtype="f16", D=p.D,
                                    scale=p.scale, ranks=p.ranks)
            assert np.array_equal(yi, y[:, off:off + w]), f"slice {i} case {n}"
            assert np.array_equal(vi[0], v[i]), f"slice {i} v case {n}"


def pin_token_subset(o):
    """Asking for a subset of tokens gives exactly those rows of the full result."""
    rng = np.random.default_rng(31)
    p = random_problem(rng, T=30, D=12, out_sizes=(5, 2), r_max=4, S=3, dtype="f16",
                       with_ranks=True)
    v, y = _apply(o, p)
    sub = [29, 3, 3, 0, 17]
    vs, ys = _apply(o, p, tokens=sub)
    assert np.array_equal(ys, y[sub]) and np.array_equal(vs, v[:, sub])


# --------------------------------------------------------------------------
# hand-worked example
# --------------------------------------------------------------------------

def load_golden(name="handworked_two_slots.txt"):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *rest = line.split()
            vals[key] = [float(t) for t in rest]
    return vals


def pin_handworked(o):
    g = load_golden()
    T, D, S, r, out = (int(g[k][0]) for k in ("T", "D", "S", "r_max", "out"))
    x = np.array(g["x"], np.float32).reshape(T, D)
    A = [np.stack([np.array(g["A0"], np.float32).reshape(r, D),
                   np.array(g["A1"], np.float32).reshape(r, D)])]
    B = [np.stack([np.array(g["B0"], np.float32).reshape(out, r),
                   np.array(g["B1"], np.float32).reshape(out, r)])]
    y_in = np.array(g["y_in"], np.float32).reshape(T, out)
    scale = np.array(g["scale"], np.float32)
    idx = np.array(g["idx"], np.int32)

    v, y = o.oracle_apply(x, A, B, y_in, idx, S, (0,), dtype="f32", scale=scale)
    assert np.array_equal(v[0], np.array(g["v"]).reshape(T, r)), "hand-worked v"
    assert np.array_equal(y, np.array(g["y"]).reshape(T, out)), "hand-worked y"
    seg = o.oracle_segments(idx, S)
    for k in ("perm", "rest", "seg_slot", "seg_start"):
        assert list(seg[k]) == [int(t) for t in g[k]], f"hand-worked {k}"
    for k in ("num_active", "num_segments", "max_seg_len", "status"):
        assert seg[k] == int(g[k][0]), f"hand-worked {k}"

    ranks = np.array(g["ranks"], np.int32)
    v, y = o.oracle_apply(x, A, B, y_in, idx, S, (0,), dtype="f32", scale=scale,
                          ranks=ranks)
    assert np.array_equal(v[0], np.array(g["ranks.v"]).reshape(T, r)), "hand-worked ranks v"
    assert np.array_equal(y, np.array(g["ranks.y"]).reshape(T, out)), "hand-worked ranks y"

    bad = np.array(g["bad_index.idx"], np.int32)
    v, y = o.oracle_apply(x, A, B, y_in, bad, S, (0,), dtype="f32", scale=scale)
    assert np.array_equal(y, np.array(g["bad_index.y"]).reshape(T, out)), "hand-worked bad idx"
    seg = o.oracle_segments(bad, S)
    assert seg["status"] == int(g["bad_index.status"][0])
    assert seg["num_active"] == int(g["bad_index.num_active"][0])


# --------------------------------------------------------------------------
# slot grouping
# --------------------------------------------------------------------------

def segment_cases(seed=37):
    rng = np.random.default_rng(seed)
    yield np.zeros(0, np.int32), 3
    yield np.full(9, -1, np.int32), 2
    yield np.array([0], np.int32), 1
    yield np.array([2, 2, 2, -1, 2], np.int32), 4
    yield np.array([3, -2, 0, 7, -1, 3, 0], np.int32), 4
    for n in range(200):
        T = int(rng.integers(0, 300))
        S = int(rng.integers(1, 40))
        idx = rng.integers(-1, S, size=T).astype(np.int32)
        if n % 5 == 0 and T:
            idx[rng.random(T) < 0.05] = S + 3
        yield idx, S


def pin_segments(o):
    for n, (idx, S) in enumerate(segment_cases()):
        a = o.oracle_segments(idx, S)
        b = brute_segments(idx, S)
        for k in ("perm", "rest", "seg_slot", "seg_start"):
            assert np.array_equal(np.asarray(a[k]), b[k]) and a[k].dtype == np.int32, \
                f"segments case {n}: {k}"
        for k in ("num_active", "num_segments", "max_seg_len", "status"):
            assert a[k] == b[k], f"segments case {n}: {k} {a[k]} vs {b[k]}"
        # invariants
        perm = a["perm"]
        assert sorted(perm.tolist()) == [t for t in range(len(idx)) if 0 <= idx[t] < S]
        # perm followed by rest is a permutation of all tokens
        assert sorted(perm.tolist() + a["rest"].tolist()) == list(range(len(idx)))
        assert np.all(np.diff(a["rest"]) > 0)
        sl = idx[perm]
        assert np.all(np.diff(sl) >= 0)
        for g in range(a["num_segments"]):
            seg = perm[a["seg_start"][g]:a["seg_start"][g + 1]]
            assert np.all(idx[seg] == a["seg_slot"][g]) and np.all(np.diff(seg) > 0)


# --------------------------------------------------------------------------
# embedding LoRA
# --------------------------------------------------------------------------

def embedding_cases(n_cases=120, seed=55):
    rng = np.random.default_rng(seed)
    fixed = [dict(T=0, V=3, H=2, r_max=2, S=1), dict(T=1, V=1, H=1, r_max=1, S=1, base_frac=0.0),
             dict(T=6, V=5, H=3, r_max=2, S=2, base_frac=1.0),
             dict(T=9, V=7, H=4, r_max=3, S=3, bad_tok_frac=0.4, bad_idx_frac=0.2)]
    for c in fixed:
        yield random_embedding_problem(rng, **c)
    dtypes = ["f32", "f16", "bf16"]
    for n in range(n_cases - len(fixed)):
        yield random_embedding_problem(
            rng, T=int(rng.integers(0, 12)), V=int(rng.integers(1, 20)), H=int(rng.integers(1, 12)),
            r_max=int(rng.integers(1, 9)), S=int(rng.integers(1, 5)), dtype=dtypes[n % 3],
            base_frac=float(rng.uniform(0, 0.5)), with_ranks=bool(n % 2),
            bad_tok_frac=0.15 if n % 4 == 0 else 0.0, bad_idx_frac=0.1 if n % 5 == 0 else 0.0)


def _embedding_apply(o, p):
    return o.oracle_embedding_apply(p.tok, p.A_emb, p.B, p.y_in, p.idx, p.S, dtype=p.dtype,
                                    scale=p.scale, ranks=p.ranks)


def pin_embedding_bruteforce(o):
    """Against the one-hot product in pure Python (with garbage past each rank)."""
    rng = np.random.default_rng(56)
    for n, p in enumerate(embedding_cases()):
        if p.ranks is not None:
            for s, r in enumerate(p.ranks):
                p.A_emb[s, :, r:] = p.A_emb.dtype.type(5) if p.A_emb.dtype != np.uint16 else np.uint16(0x40a0)
                p.B[s, :, r:] = p.B.dtype.type(5) if p.B.dtype != np.uint16 else np.uint16(0x40a0)
        v, y = _embedding_apply(o, p)
        vb, yb = brute_embedding(p)
        _close(v, np.asarray(vb, dtype=np.float64).reshape(p.T, p.r_max), 1e-12, f"embedding v case {n}")
        _close(y, np.asarray(yb, dtype=np.float64).reshape(p.T, p.ldy), 1e-12, f"embedding y case {n}")


def pin_embedding_is_linear_on_one_hot(o):
    """The embedding adapter is the linear adapter applied to the one-hot rows
    of the token ids, with the table transposed (A_s = A_emb[s]^T): checked
    against the (separately pinned) linear oracle; ids outside [0, V) have an
    all-zero one-hot row."""
    rng = np.random.default_rng(57)
    for n in range(40):
        p = random_embedding_problem(rng, T=int(rng.integers(1, 25)), V=int(rng.integers(1, 40)),
                                     H=int(rng.integers(1, 20)), r_max=int(rng.integers(1, 9)),
                                     S=int(rng.integers(1, 5)), dtype=("f32", "f16", "bf16")[n % 3],
                                     with_ranks=bool(n % 2), bad_tok_frac=0.2 if n % 3 == 0 else 0.0)
        x = np.zeros((p.T, p.V), dtype=np.float32)
        for t, w in enumerate(p.tok):
            if 0 <= w < p.V:
                x[t, w] = 1.0
        x = x.astype(p.A_emb.dtype) if p.dtype != "bf16" else (x.view(np.uint32) >> 16).astype(np.uint16)
        A_lin = np.ascontiguousarray(np.transpose(p.A_emb, (0, 2, 1)))
        v_lin, y_lin = o.oracle_apply(x, [A_lin], [p.B], p.y_in, p.idx, p.S, (0,), dtype=p.dtype,
                                      scale=p.scale, ranks=p.ranks)
        v, y = _embedding_apply(o, p)
        _close(v, v_lin[0], 1e-13, f"embedding vs linear v case {n}")
        _close(y, y_lin, 1e-13, f"embedding vs linear y case {n}")


def pin_embedding_invariants(o):
    """Base rows and rows of ids outside the table are bit-identical to y_in;
    the delta is linear in scale and independent of y_in."""
    rng = np.random.default_rng(58)
    for n in range(30):
        p = random_embedding_problem(rng, T=30, V=11, H=6, r_max=4, S=3, dtype="f32",
                                     bad_tok_frac=0.2, bad_idx_frac=0.1)
        v, y = _embedding_apply(o, p)
        y_in = o.decode(p.y_in, "f32")
        dead = ~((p.idx >= 0) & (p.idx < p.S)) | (p.tok < 0) | (p.tok >= p.V)
        assert np.array_equal(y[dead], y_in[dead]), f"embedding dead rows case {n}"
        assert not np.any(v[dead]), f"embedding dead v case {n}"
        p2 = random_embedding_problem(rng, T=30, V=11, H=6, r_max=4, S=3, dtype="f32",
                                      idx=p.idx, tok=p.tok)
        p2.A_emb, p2.B, p2.scale = p.A_emb, p.B, p.scale * 2
        v2, y2 = _embedding_apply(o, p2)
        _close(v2, 2 * v, 1e-13, f"embedding scale linearity case {n}")
        _close(y2 - o.decode(p2.y_in, "f32"), 2 * (y - y_in), 1e-12, f"embedding delta case {n}")


ALL_PINS = [
    pin_bruteforce,
    pin_expand_bruteforce,
    pin_gather_baseline,
    pin_single_adapter,
    pin_closed_form,
    pin_base_rows_untouched,
    pin_rank_padding,
    pin_linearity,
    pin_permutation,
    pin_slice_decomposition,
    pin_token_subset,
    pin_handworked,
    pin_segments,
    pin_embedding_bruteforce,
    pin_embedding_is_linear_on_one_hot,
    pin_embedding_invariants,
]
