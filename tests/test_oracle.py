"""CPU tests: the fp64 oracle against its pins, and the pins against planted mistakes."""

import os
import types

import numpy as np
import pytest

import oracle
import oracle_pins as pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "lora_oracle.py")


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle)


# --------------------------------------------------------------------------
# Mutation tests: each plants one plausible mistake in a copy of the oracle's
# source and checks that at least one pin fails on the copy.
# --------------------------------------------------------------------------

MUTANTS = {
    "drop_scale": ("v[i, j, :r] = sc * (a[:r, :] @ xt)", "v[i, j, :r] = (a[:r, :] @ xt)"),
    "wrong_sign": ("y[j, off:off + b.shape[0]] += ", "y[j, off:off + b.shape[0]] -= "),
    "transposed_A": ("v[i, j, :r] = sc * (a[:r, :] @ xt)",
                     "v[i, j, :r] = sc * (a[:r, :r].T @ xt[:r])"),
    "ignore_ranks_shrink": ("v[i, j, :r] = sc * (a[:r, :] @ xt)",
                            "v[i, j, :] = sc * (a @ xt)"),
    "ignore_ranks_expand": ("b[:, :r] @ np.asarray(v[i, j, :r], dtype=np.float64)",
                            "b @ np.asarray(v[i, j, :], dtype=np.float64)"),
    "minus_one_wraps": ("    return 0 <= s < S\n", "    return -1 <= s < S\n"),
    "offset_off_by_one": ("off = int(out_offsets[i])", "off = int(out_offsets[i]) + (1 if i else 0)"),
    "unstable_order": ("key=lambda t: (idx[t], t)", "key=lambda t: (idx[t], -t)"),
    "status_ignored": ("status = LORA_ERR_INDEX", "status = LORA_OK"),
    "max_seg_len_off": ("max_seg_len=max(counts) if counts else 0",
                        "max_seg_len=max(counts) - 1 if counts else 0"),
    "wrong_slot_weights": ("cache[key] = decode(A[i][s], dtype)",
                           "cache[key] = decode(A[i][(s + 1) % S], dtype)"),
    "half_intermediate": ("v[i, j, :r] = sc * (a[:r, :] @ xt)",
                          "v[i, j, :r] = (sc * (a[:r, :] @ xt)).astype(np.float16)"),
    "embedding_wrong_row": ("v[j, :r] = sc * decode(A_emb[s, w, :r], dtype)",
                            "v[j, :r] = sc * decode(A_emb[s, (w + 1) % V, :r], dtype)"),
    "embedding_no_scale": ("v[j, :r] = sc * decode(A_emb[s, w, :r], dtype)",
                           "v[j, :r] = decode(A_emb[s, w, :r], dtype)"),
    "embedding_bad_id_wraps": ("if not _valid_slot(s, S) or not 0 <= w < V:",
                               "if not _valid_slot(s, S) or not -V <= w < V:"),
    "embedding_ignores_rank": ("v[j, :r] = sc * decode(A_emb[s, w, :r], dtype)",
                               "v[j, :] = sc * decode(A_emb[s, w, :], dtype)"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = open(ORACLE_SRC).read()
    assert old in src, f"mutation site for {name} no longer exists in the oracle"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new, 1), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    mod = _mutant(name)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            if pin is pins.pin_bruteforce:
                pin(mod, n_cases=60)
            else:
                pin(mod)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin detects the planted mistake {name!r}"
