"""fp64 per-token oracle for multi-LoRA batched application.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py.  Nothing here is shared with the HIP library.

What is computed (for every token t whose slot s = idx[t] is valid):

    v[i][t][k] = scale[s] * sum_d A_i[s][k][d] * x[t][d]           k < r_s
    y[t][off_i + j] = y_in[t][off_i + j] + sum_k B_i[s][j][k] * v[i][t][k]

Sources on the pages, stated in this module's own words:

* "[Hardware][TPU][V1] Better tpu multilora compilation", review thread with
  the PyTorch baseline (ref_bgmv) that replaced the Pallas kernels: each token
  picks the stacked LoRA matrix of its index and multiplies it with its own
  input vector; the stacked tensor keeps the input dimension contiguous, so a
  shrink matrix is rank x D and an expand matrix is out x rank.
* "Add multi-LoRA support", Features: one batch may mix LoRA requests and
  base-model-only requests, and adapters may have different ranks.
  Limitations: rank is at most 64; every adapter has one shared dtype; storing
  the intermediate in half precision costs accuracy, so the intermediate here
  is kept in (at least) fp32 — fp64 in this oracle.
* "[LoRA] LoRA cuda graph specialization", Implementation: the intermediate
  buffer is zeroed inside the shrink op, so when no adapter is active nothing
  touches it.

Readings where the pages are silent (each is listed in the design notes):
* idx = -1 means base model only: the token's output row is left exactly as
  it was and its input row is never read.  An index below -1 or at/above S is
  treated the same way and reported with status LORA_ERR_INDEX.
* scale is one fp32 value per slot, applied to the shrink result.
* with per-slot ranks, only the first r_s rank rows/columns take part; the
  intermediate's columns k >= r_s are zero.
* the intermediate of an inactive token is zero.

Precision: all inputs are decoded exactly to float64 (fp16 via numpy's
float16, bf16 by placing its 16 bits at the top of an fp32 word) and every
operation runs in float64.  Results are NOT rounded to the storage dtype.
"""

import numpy as np

LORA_OK = 0
LORA_ERR_INDEX = 3


def decode(a, dtype):
    """Exact widening of a storage-dtype array to float64.

    dtype "f32" / "f16": numpy float32 / float16 arrays ("f64": float64, used by
    tests that need unrounded inputs).
    dtype "bf16": numpy uint16 arrays holding bfloat16 bit patterns; the 16 bits
    are the top half of an IEEE fp32 word, so shifting them left by 16 and
    reinterpreting gives the exact value.
    """
    a = np.asarray(a)
    if dtype in ("f32", "f16", "f64"):
        return a.astype(np.float64)
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _valid_slot(s, S):
    return 0 <= s < S


def oracle_segments(idx, S):
    """Group the active tokens of a batch by adapter slot.

    The per-token index vector is built once per batch and moved to the device
    ("[Hardware][TPU][V1] Better tpu multilora compilation", review comment on
    the token index buffer); grouping tokens by slot is what lets a segmented
    kernel process each adapter's tokens together.

    Returns a dict with
      perm        int32 [num_active]: the active tokens, ordered by slot
                  ascending and, within a slot, by token index ascending;
      seg_slot    int32 [num_segments]: the slots that have at least one token,
                  ascending;
      seg_start   int32 [num_segments + 1]: segment g is perm[seg_start[g] :
                  seg_start[g+1]]; seg_start[-1] == num_active;
      rest        int32 [T - num_active]: the tokens without a valid slot
                  (idx -1 or out of range), ascending.  The pages do not
                  describe this list; it is this library's reading of where
                  the base-only tokens go in a record (after the active ones),
                  so that the shrink can clear their intermediate rows;
      num_active, num_segments, max_seg_len, status.
    """
    idx = [int(v) for v in np.asarray(idx).reshape(-1)]
    T = len(idx)
    status = LORA_OK
    counts = [0] * S
    for t in range(T):
        s = idx[t]
        if _valid_slot(s, S):
            counts[s] += 1
        elif s != -1:
            status = LORA_ERR_INDEX
    # Stable order: slot first, then token.  Python's sort is stable, and the
    # key makes the order total anyway.
    active = [t for t in range(T) if _valid_slot(idx[t], S)]
    perm = sorted(active, key=lambda t: (idx[t], t))
    seg_slot = [s for s in range(S) if counts[s] > 0]
    seg_start = [0]
    for s in seg_slot:
        seg_start.append(seg_start[-1] + counts[s])
    rest = [t for t in range(T) if not _valid_slot(idx[t], S)]
    return dict(
        perm=np.asarray(perm, dtype=np.int32),
        rest=np.asarray(rest, dtype=np.int32),
        seg_slot=np.asarray(seg_slot, dtype=np.int32),
        seg_start=np.asarray(seg_start, dtype=np.int32),
        num_active=len(active),
        num_segments=len(seg_slot),
        max_seg_len=max(counts) if counts else 0,
        status=status,
    )


def _rank(ranks, s, r_max):
    return r_max if ranks is None else int(ranks[s])


def oracle_shrink(x, A, idx, S, *, dtype, D=None, scale=None, ranks=None,
                  tokens=None):
    """Shrink: the fp64 rank-r intermediate of the listed tokens.

    x      [T, >=D] storage dtype        A   list (one per slice) of [S, r_max, D]
    idx    [T] int                       scale [S] fp32 or None (1.0)
    ranks  [S] int or None (r_max)       tokens: token indices to compute
                                          (default: all, in order)

    Returns v of shape [n_slices, len(tokens), r_max], float64.  Row j belongs
    to token tokens[j]; it is zero when that token is inactive, and columns
    k >= r_s are zero.

    One matrix-vector product per token and slice, as in the gather baseline
    of "[Hardware][TPU][V1] Better tpu multilora compilation" (review thread),
    with the scale applied to the shrink result.
    """
    idx = np.asarray(idx).reshape(-1)
    T = idx.shape[0]
    n_sl = len(A)
    r_max = A[0].shape[1] if n_sl else 0
    D = A[0].shape[2] if D is None and n_sl else D
    tokens = list(range(T)) if tokens is None else [int(t) for t in tokens]
    v = np.zeros((n_sl, len(tokens), r_max), dtype=np.float64)
    cache = {}
    for j, t in enumerate(tokens):
        s = int(idx[t])
        if not _valid_slot(s, S):
            continue
        r = _rank(ranks, s, r_max)
        sc = 1.0 if scale is None else float(np.float64(scale[s]))
        xt = decode(x[t, :D], dtype)
        for i in range(n_sl):
            key = (i, s)
            if key not in cache:
                cache[key] = decode(A[i][s], dtype)
            a = cache[key]
            v[i, j, :r] = sc * (a[:r, :] @ xt)
    return v


def oracle_expand(v, B, y_in, idx, S, out_offsets, *, dtype, ranks=None,
                  tokens=None):
    """Expand: add each active token's LoRA delta into its output row.

    v      [n_slices, len(tokens), r_max] float (row j <-> token tokens[j])
    B      list (one per slice) of [S, out_i, r_max]
    y_in   [T, ldy] storage dtype         out_offsets: column offset per slice

    Returns y of shape [len(tokens), ldy], float64: the decoded y_in rows with
    B_i[s] @ v[i][t] added to columns [off_i, off_i + out_i) of active rows.
    Inactive rows are the decoded y_in, unchanged.
    """
    idx = np.asarray(idx).reshape(-1)
    T = idx.shape[0]
    n_sl = len(B)
    r_max = B[0].shape[2] if n_sl else 0
    tokens = list(range(T)) if tokens is None else [int(t) for t in tokens]
    y = decode(y_in[tokens], dtype) if len(tokens) else \
        np.zeros((0, y_in.shape[1]), dtype=np.float64)
    cache = {}
    for j, t in enumerate(tokens):
        s = int(idx[t])
        if not _valid_slot(s, S):
            continue
        r = _rank(ranks, s, r_max)
        for i in range(n_sl):
            key = (i, s)
            if key not in cache:
                cache[key] = decode(B[i][s], dtype)
            b = cache[key]
            off = int(out_offsets[i])
            y[j, off:off + b.shape[0]] += b[:, :r] @ np.asarray(v[i, j, :r], dtype=np.float64)
    return y


def oracle_apply(x, A, B, y_in, idx, S, out_offsets, *, dtype, D=None,
                 scale=None, ranks=None, tokens=None):
    """Shrink followed by expand.  Returns (v, y) for the listed tokens."""
    v = oracle_shrink(x, A, idx, S, dtype=dtype, D=D, scale=scale, ranks=ranks,
                      tokens=tokens)
    y = oracle_expand(v, B, y_in, idx, S, out_offsets, dtype=dtype,
                      ranks=ranks, tokens=tokens)
    return v, y


def oracle_embedding_shrink(tok, A_emb, idx, S, *, dtype, scale=None, ranks=None,
                            tokens=None):
    """Shrink of a LoRA on an embedding table, in fp64.

    "Add multi-LoRA support", Features: adapters cover every linear layer and
    the embeddings, in PEFT format.  In that format an embedding adapter of
    slot s holds A_s (r x V) and B_s (H x r), and the input of the layer for
    token id w is the one-hot vector e_w of length V, so the linear shrink
    A_s @ x reduces to column w of A_s.  This library stacks the tables
    transposed, A_emb[s] = A_s^T of shape [V][r_max] (one contiguous rank
    vector per vocabulary row; reading), so that

        v[t][k] = scale[s] * A_emb[s][tok[t]][k]          (k < r_s)

    tok    [T] int token ids; an id outside [0, V) has no adapter row, and its
           intermediate is zero (reading: such ids, e.g. tokens added by an
           adapter, are looked up elsewhere)
    A_emb  [S, V, r_max] storage dtype      idx [T] slots (-1: base only)
    Returns v of shape [len(tokens), r_max], float64 (zero rows for inactive
    tokens and for ids outside the table).
    """
    idx = np.asarray(idx).reshape(-1)
    tok = np.asarray(tok).reshape(-1)
    T = idx.shape[0]
    V, r_max = A_emb.shape[1], A_emb.shape[2]
    tokens = list(range(T)) if tokens is None else [int(t) for t in tokens]
    v = np.zeros((len(tokens), r_max), dtype=np.float64)
    for j, t in enumerate(tokens):
        s = int(idx[t])
        w = int(tok[t])
        if not _valid_slot(s, S) or not 0 <= w < V:
            continue
        r = _rank(ranks, s, r_max)
        sc = 1.0 if scale is None else float(np.float64(scale[s]))
        v[j, :r] = sc * decode(A_emb[s, w, :r], dtype)
    return v


def oracle_embedding_apply(tok, A_emb, B, y_in, idx, S, *, dtype, scale=None,
                           ranks=None, tokens=None):
    """Embedding LoRA: y[t] = y_in[t] + B_s @ v[t] with v from
    oracle_embedding_shrink (the expand is the linear layers' expand with one
    slice of width H).  Returns (v, y) for the listed tokens."""
    v = oracle_embedding_shrink(tok, A_emb, idx, S, dtype=dtype, scale=scale,
                                ranks=ranks, tokens=tokens)
    y = oracle_expand(v[None], [B], y_in, idx, S, (0,), dtype=dtype, ranks=ranks,
                      tokens=tokens)
    return v, y
