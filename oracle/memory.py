"""Size of the materialised score matrix (oracle; test infrastructure).

[FA-vs-PA] (FlashAttention §2) works out the memory that standard attention
needs for the N×N score matrix: N² elements per head and sample, times the
element size, times heads and batch.  FlashAttention's tiling brings this
temporary memory from O(N²) down to O(N).  The helper lets tests check that
the library's workspace does not grow like this figure.
"""
from __future__ import annotations


def score_matrix_bytes(seq_len: int, elem_bytes: int, heads: int = 1, batch: int = 1) -> int:
    return int(seq_len) * int(seq_len) * int(elem_bytes) * int(heads) * int(batch)
