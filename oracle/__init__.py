"""CPU oracle for fused inference attention (TEST INFRASTRUCTURE ONLY).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never uses it.
"""
from .fia_oracle import (decode_bf16, decode_e4m3fn, decode_packed_row, fia,
                         fia_case, per_batch_lengths, softmax_rows, sparse_rows,
                         sparse_sharedkv, visible)

__all__ = ["decode_bf16", "decode_e4m3fn", "decode_packed_row", "fia", "fia_case",
           "per_batch_lengths", "softmax_rows", "sparse_rows", "sparse_sharedkv",
           "visible"]
