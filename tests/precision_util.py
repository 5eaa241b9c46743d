"""Once-rounded comparison of 16-bit outputs with the fp64 oracle.

The expand adds an fp32 LoRA delta to y and rounds each element once into its
16-bit dtype.  With y_in = 0 the stored y is then RNE(delta), and an fp32
intermediate gives a delta close enough to the exact one that nearly every
element rounds to the same 16-bit value as the exact fp64 result.  An
intermediate re-rounded to 16 bits before the expand ("Add multi-LoRA
support", Limitations: the accuracy loss of a half-precision intermediate)
moves a large share of elements to a neighbouring value, although its error
stays far inside the max-relative-error bars.  These helpers round fp64
values directly (no double rounding through fp32) and measure the distance in
units in the last place.
"""

import numpy as np

# Share of compared elements that must equal the once-rounded oracle value,
# and the largest distance allowed for the others.  Near-zero outputs come
# from cancellation between the rank terms; there the fp32 rounding of the
# terms alone can move the result by several of its own (tiny) ulps, so the
# distance in ulps is required only where |y_ref| >= SMALL * (largest |y_ref|
# of the row), and below that the absolute error must stay within one ulp of
# a value of that threshold size.
MATCH_MIN = 0.99
MAX_ULP = 1
SMALL = 2.0 ** -10
SIG_BITS = {"f16": 11, "bf16": 8}


def rne16_bits(a, dtype):
    """Bit patterns (uint16) of fp64 values rounded to nearest-even into fp16
    or bf16, in one rounding step from fp64."""
    a = np.asarray(a, dtype=np.float64)
    if dtype == "f16":
        bits, min_exp = 11, -14          # significant bits; smallest normal 2^-14
    elif dtype == "bf16":
        bits, min_exp = 8, -126
    else:
        raise ValueError(dtype)
    m, e = np.frexp(a)                   # a = m 2^e with 0.5 <= |m| < 1
    # normal range: keep `bits` significant bits; below it, a fixed spacing
    # of 2^(min_exp - bits + 1) (the subnormal step)
    normal = np.ldexp(np.rint(np.ldexp(m, bits)), e - bits)
    step_exp = min_exp - bits + 1
    sub = np.ldexp(np.rint(np.ldexp(a, -step_exp)), step_exp)
    r = np.where(np.abs(a) < np.ldexp(1.0, min_exp), sub, normal)
    if dtype == "f16":
        return r.astype(np.float16).view(np.uint16)          # exact: r is representable
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)  # exact, likewise


def ordered(bits16):
    """Map 16-bit float patterns to integers whose differences count ulps."""
    b = np.asarray(bits16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp_distance(bits_a, bits_b):
    return np.abs(ordered(bits_a) - ordered(bits_b))


def ulp16(a, dtype):
    """Spacing of the 16-bit dtype at magnitude |a| (normal range)."""
    _, e = np.frexp(np.abs(np.asarray(a, dtype=np.float64)))
    return np.ldexp(1.0, e - SIG_BITS[dtype])


def once_rounded_match(y_bits, y_ref, dtype, cols=None):
    """Compare stored y bits with the fp64 reference rounded once.

    Returns (share of elements equal, largest ulp distance among elements with
    |y_ref| >= SMALL x row max, largest |error| of the other elements in units
    of the ulp at SMALL x row max).  cols restricts the comparison to those
    columns.
    """
    y_bits = np.asarray(y_bits)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if cols is not None:
        y_bits, y_ref = y_bits[:, cols], y_ref[:, cols]
    if y_bits.size == 0:
        return 1.0, 0, 0.0
    ref_bits = rne16_bits(y_ref, dtype)
    d = ulp_distance(y_bits, ref_bits)
    row_max = np.max(np.abs(y_ref), axis=1, keepdims=True)
    big = np.abs(y_ref) >= SMALL * row_max
    u_big = int(d[big].max()) if big.any() else 0
    got = decode16(y_bits, dtype)
    floor_ulp = np.broadcast_to(ulp16(SMALL * row_max, dtype), y_ref.shape)
    small = ~big
    e_small = float(np.max(np.abs(got - y_ref)[small] / floor_ulp[small])) if small.any() else 0.0
    return float(np.mean(d == 0)), u_big, e_small


def decode16(bits16, dtype):
    """Exact fp64 values of 16-bit float patterns."""
    b = np.asarray(bits16).astype(np.uint16)
    if dtype == "f16":
        return b.view(np.float16).astype(np.float64)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def precision_ok(result):
    share, u_big, e_small = result
    return share >= MATCH_MIN and u_big <= MAX_ULP and e_small <= 1.0


def storage_bits(y, dtype):
    """uint16 bit patterns of a stored 16-bit array (numpy float16, or the
    uint16 bf16 patterns the workloads use)."""
    y = np.asarray(y)
    return y.view(np.uint16) if dtype == "f16" else y.astype(np.uint16)


def slice_columns(p):
    """Columns of y that belong to some output slice."""
    inside = np.zeros(p.ldy, dtype=bool)
    for off, w in zip(p.out_offsets, p.out_sizes):
        inside[off:off + w] = True
    return inside
