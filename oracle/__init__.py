"""fp64 CPU oracle for exact scaled dot-product attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or
executes this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, header, table
or helper with the HIP library; the only thing both sides see is the seeded
input generator in ``attn_inputs`` (random numbers and dtype casts, none of
the method's arithmetic).

Every function here is pinned by ``tests/test_oracle_pins*.py`` to closed
forms, invariants, library special cases, published known-answer vectors,
brute force and finite differences (see each docstring); none is "parity
unpinned".
"""
from .attention import (
    attention_fwd64,
    attention_rows_fwd64,
    attention_bwd64,
    attention_rows_dq64,
    philox4x32_10,
    dropout_threshold,
    dropout_keep,
)
from .fp8 import e4m3fn_to_float64, attention_fp8_fwd64, attention_fp8_rows_fwd64, fp8_rounding_model

__all__ = [
    "attention_fwd64",
    "attention_rows_fwd64",
    "attention_bwd64",
    "attention_rows_dq64",
    "philox4x32_10",
    "dropout_threshold",
    "dropout_keep",
    "e4m3fn_to_float64",
    "attention_fp8_fwd64",
    "attention_fp8_rows_fwd64",
    "fp8_rounding_model",
]
