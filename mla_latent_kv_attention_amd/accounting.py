"""Algorithmic work of one call: the bytes and flops the method itself must move or
compute, each counted once.  Host arithmetic only (used to report roofline figures).

Decode / verify bytes: every visible latent row of a sequence is read once (all heads
and query positions share it), plus the queries, the outputs, the lse values and the
block-table entries the call consults.  Split-KV workspace traffic is an artefact of
the implementation: it costs time but is not counted.
Flops: 2 * (576 + 512) = 2,176 per (query row, visible key) -- the score dot product
and the value accumulation; the causal triangle only for prefill.
"""
from __future__ import annotations

from typing import Optional, Sequence

DK = 576
DV = 512
FLOPS_PER_ROW_KEY = 2 * (DK + DV)


def row_bytes(kv_dtype: str) -> int:
    """Bytes of one cached latent row: 576 FP8 codes or 576 BF16 values."""
    return DK * (1 if kv_dtype == "fp8" else 2)


def visible_keys(seq_len: int, P: int, j: int, kv_begin: int = 0,
                 kv_end: Optional[int] = None) -> int:
    hi = seq_len - P + j + 1
    if kv_end is not None:
        hi = min(hi, kv_end)
    return max(0, hi - max(0, kv_begin))


def decode_bytes(seq_lens: Sequence[int], P: int, H: int, kv_dtype: str, out_bytes: int = 4,
                 block_size: int = 64, kv_begin: Optional[Sequence[int]] = None,
                 kv_end: Optional[Sequence[int]] = None) -> int:
    total = 0
    for b, L in enumerate(seq_lens):
        lo = 0 if kv_begin is None else max(0, int(kv_begin[b]))
        hi = int(L) if kv_end is None else min(int(L), int(kv_end[b]))
        n = max(0, hi - lo)  # rows of the covered range (the last query sees them all)
        total += n * row_bytes(kv_dtype)
        if n:
            total += 4 * ((hi - 1) // block_size - lo // block_size + 1)  # table entries
    rows = len(seq_lens) * P * H
    return total + rows * (DK * 2 + DV * out_bytes + 4)


def decode_flops(seq_lens: Sequence[int], P: int, H: int,
                 kv_begin: Optional[Sequence[int]] = None,
                 kv_end: Optional[Sequence[int]] = None) -> int:
    f = 0
    for b, L in enumerate(seq_lens):
        for j in range(P):
            f += H * visible_keys(int(L), P, j, 0 if kv_begin is None else int(kv_begin[b]),
                                  None if kv_end is None else int(kv_end[b]))
    return f * FLOPS_PER_ROW_KEY


def prefill_flops(seq_lens: Sequence[int], H: int) -> int:
    return sum(H * int(T) * (int(T) + 1) // 2 for T in seq_lens) * FLOPS_PER_ROW_KEY


def prefill_bytes(seq_lens: Sequence[int], H: int, kv_dtype: str = "bf16",
                  out_bytes: int = 2) -> int:
    T = sum(int(t) for t in seq_lens)
    return T * H * DK * 2 + T * row_bytes(kv_dtype) + T * H * (DV * out_bytes + 4)
