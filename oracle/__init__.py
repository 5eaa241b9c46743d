"""fp64 CPU oracle for multi-LoRA shrink/expand — TEST INFRASTRUCTURE ONLY.

This package is the reference that the HIP library is checked against.  It is
plain, slow and meant to be checked by eye against the pages.  It is used only
by tests/, by __graft_entry__.smoke() and by the cpu_baseline leg of bench.py;
the library under gemm_lora_shrink_amd/ never imports, links or calls it, and
it imports nothing from that library.

Every function here is pinned by tests/test_oracle.py to something other than
itself (brute force on tiny inputs, closed forms, invariants, a hand-worked
example and a second formulation taken from the pages' gather baseline).
"""

from .lora_oracle import (
    LORA_OK,
    LORA_ERR_INDEX,
    decode,
    oracle_segments,
    oracle_shrink,
    oracle_expand,
    oracle_apply,
    oracle_embedding_shrink,
    oracle_embedding_apply,
)

__all__ = [
    "LORA_OK",
    "LORA_ERR_INDEX",
    "decode",
    "oracle_segments",
    "oracle_shrink",
    "oracle_expand",
    "oracle_apply",
    "oracle_embedding_shrink",
    "oracle_embedding_apply",
]
