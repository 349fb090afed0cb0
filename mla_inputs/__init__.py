"""Seeded synthetic inputs for MLA latent-KV attention.

Shared by the tests, the bench and the smoke check, and by both sides of every
parity comparison.  This module holds no attention arithmetic: it draws seeded
normal values, rounds them to the storage formats (BF16 round-to-nearest-even,
OCP FP8 E4M3FN with one per-tensor scale), lays rows out in a paged cache
behind a shuffled block table and poisons every slot no sequence owns with NaN.

Recipe (stands in for the serving workloads the pages measure; their traces,
datasets and weights are not used):
  * queries: iid N(0, 1) in float32, rounded to BF16;
  * latent rows: iid N(0, 1) in float32; BF16 by rounding, or FP8 E4M3FN as
    codes = RNE(clamp(x / s, -448, 448)) with s = float32(amax|x| / 448);
  * paged caches: blocks of ``block_size`` tokens; the physical block of every
    (sequence, logical block) is drawn from a seeded permutation of the pool;
    table entries past a sequence's last block point at a NaN-filled spare
    block; slots past a sequence's length and all spare blocks hold NaN;
  * per-sequence lengths: seeded uniform integers in the stated inclusive range;
  * probability rows (input of the top-k renormalisation): logits iid
    N(0, sigma^2) in float64 (sigma = 3 gives a peaked, long-tailed row), turned
    into probabilities by exp(logit - max) / sum in float64 and rounded to
    float32; per-row k: seeded uniform integers in the stated inclusive range.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

DK = 576
DV = 512
FP8_MAX = 448.0
BF16_NAN_BITS = 0x7FC0
FP8_NAN_CODE = 0x7F


def softmax_scale_for(qk_dim: int = 192) -> float:
    """fp32(1 / sqrt(qk_dim)); 192 = 128 + 64 is the pre-absorption query-key width."""
    return float(np.float32(1.0 / math.sqrt(qk_dim)))


def rng_for(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(stream)]))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to BF16 (nearest-even) and return the bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_fp8_codes(x: np.ndarray, scale: float) -> np.ndarray:
    """Quantise float32 values to FP8 E4M3FN codes with a per-tensor scale."""
    y = np.clip(np.asarray(x, dtype=np.float32) / np.float32(scale), -FP8_MAX, FP8_MAX)
    codes = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    if np.any((codes & 0x7F) == FP8_NAN_CODE):
        raise ValueError("quantiser produced a NaN code")
    return codes


def normal_f32(seed: int, stream: int, shape: Sequence[int]) -> np.ndarray:
    return rng_for(seed, stream).standard_normal(tuple(shape), dtype=np.float32)


def normal_bf16_bits(seed: int, stream: int, shape: Sequence[int]) -> np.ndarray:
    return to_bf16_bits(normal_f32(seed, stream, shape))


def _chunked_normal(seed: int, stream: int, n_rows: int, chunk_rows: int = 1 << 16):
    """Yield consecutive [rows, 576] float32 chunks of one seeded stream."""
    rng = rng_for(seed, stream)
    done = 0
    while done < n_rows:
        r = min(chunk_rows, n_rows - done)
        yield done, rng.standard_normal((r, DK), dtype=np.float32)
        done += r


def latent_rows(seed: int, stream: int, n_rows: int, kv_dtype: str):
    """n_rows latent rows drawn from N(0, 1): (codes [n_rows, 576], scale).

    BF16 rows come back as uint16 bit patterns with scale 1.0; FP8 rows come
    back as uint8 E4M3FN codes with scale float32(amax / 448).
    """
    if kv_dtype == "bf16":
        out = np.empty((n_rows, DK), np.uint16)
        for off, x in _chunked_normal(seed, stream, n_rows):
            out[off:off + x.shape[0]] = to_bf16_bits(x)
        return out, 1.0
    if kv_dtype == "fp8":
        x = np.empty((n_rows, DK), np.float32)
        amax = 0.0
        for off, c in _chunked_normal(seed, stream, n_rows):
            x[off:off + c.shape[0]] = c
            amax = max(amax, float(np.abs(c).max()))
        scale = float(np.float32(amax / FP8_MAX))
        t = torch.from_numpy(x)
        t.div_(torch.tensor(scale, dtype=torch.float32)).clamp_(-FP8_MAX, FP8_MAX)
        out = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        if np.any((out & 0x7F) == FP8_NAN_CODE):
            raise ValueError("quantiser produced a NaN code")
        return out, scale
    raise ValueError("kv_dtype must be 'bf16' or 'fp8'")


@dataclasses.dataclass
class PagedCache:
    kv: np.ndarray           # [num_blocks, block_size, 576] uint16 (bf16) or uint8 (fp8)
    kv_dtype: str            # "bf16" | "fp8"
    kv_scale: float
    block_table: np.ndarray  # [B, max_blocks] int32
    seq_lens: np.ndarray     # [B] int32
    block_size: int

    @property
    def num_blocks(self) -> int:
        return self.kv.shape[0]


def paged_cache(seed: int, seq_lens: Sequence[int], block_size: int, kv_dtype: str,
                spare_blocks: int = 4, stream: int = 1) -> PagedCache:
    """Build a paged latent cache holding len(seq_lens) sequences."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    B = len(seq_lens)
    nblk = [int(-(-int(L) // block_size)) for L in seq_lens]
    used = int(sum(nblk))
    num_blocks = used + max(1, spare_blocks)
    max_blocks = max(1, max(nblk) if nblk else 1)
    codes, scale = latent_rows(seed, stream, num_blocks * block_size, kv_dtype)
    kv = codes.reshape(num_blocks, block_size, DK)
    perm = rng_for(seed, stream + 1000).permutation(num_blocks).astype(np.int32)
    spare_ids = perm[used:]
    table = np.full((B, max_blocks), spare_ids[0], dtype=np.int32)
    k = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[k:k + nblk[b]]
        k += nblk[b]
    nan = FP8_NAN_CODE if kv_dtype == "fp8" else BF16_NAN_BITS
    for b in range(B):
        L = int(seq_lens[b])
        if nblk[b] and L % block_size:
            kv[table[b, nblk[b] - 1], L % block_size:, :] = nan
    kv[spare_ids] = nan
    return PagedCache(kv, kv_dtype, scale, table, seq_lens.astype(np.int32), block_size)


def uniform_lengths(seed: int, B: int, lo: int, hi: int, stream: int = 2) -> np.ndarray:
    """B seeded integer lengths, uniform over [lo, hi] inclusive."""
    return rng_for(seed, stream).integers(lo, hi + 1, size=B, dtype=np.int64).astype(np.int32)


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class DecodeWorkload:
    """Decode (P = 1) or speculative verify (P > 1) over a paged latent cache."""
    name: str
    batch: int
    positions: int
    heads: int
    kv_dtype: str
    block_size: int
    seed: int
    lengths: Optional[List[int]] = None        # fixed lengths, or
    length_range: Optional[tuple] = None       # (lo, hi) inclusive uniform
    partitions: int = 1                        # contiguous key-range partitions merged by LSE
    pad_heads_to: int = 0                      # zero-pad query heads up to this count
    softmax_scale: float = dataclasses.field(default_factory=softmax_scale_for)

    def seq_lens(self) -> np.ndarray:
        if self.lengths is not None:
            return np.asarray(self.lengths, dtype=np.int32)
        lo, hi = self.length_range
        return uniform_lengths(self.seed, self.batch, lo, hi)


@dataclasses.dataclass
class PrefillWorkload:
    name: str
    seq_lens: List[int]
    heads: int
    kv_dtype: str
    seed: int
    softmax_scale: float = dataclasses.field(default_factory=softmax_scale_for)

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seq_lens))


def decode_inputs(w: DecodeWorkload) -> Dict[str, object]:
    """Queries and cache for a decode/verify workload (host numpy arrays)."""
    lens = w.seq_lens()
    cache = paged_cache(w.seed, lens, w.block_size, w.kv_dtype)
    H = w.heads
    q = normal_bf16_bits(w.seed, 3, (w.batch, w.positions, H, DK))
    if w.pad_heads_to and w.pad_heads_to > H:
        qp = np.zeros((w.batch, w.positions, w.pad_heads_to, DK), np.uint16)
        qp[:, :, :H] = q
        q = qp
    return {"q": q, "cache": cache}


def partition_bounds(seq_len: int, parts: int) -> List[tuple]:
    """Equal contiguous key ranges [p * n, (p + 1) * n) with n = seq_len / parts (last takes the rest)."""
    n = seq_len // parts
    return [(p * n, seq_len if p == parts - 1 else (p + 1) * n) for p in range(parts)]


def prefill_inputs(w: PrefillWorkload) -> Dict[str, object]:
    T = w.total_tokens
    q = normal_bf16_bits(w.seed, 3, (T, w.heads, DK))
    kv, scale = latent_rows(w.seed, 1, T, w.kv_dtype)
    cu = np.zeros(len(w.seq_lens) + 1, np.int32)
    cu[1:] = np.cumsum(w.seq_lens)
    return {"q": q, "kv": kv, "kv_scale": scale, "cu_seqlens": cu}


def probability_rows(seed: int, rows: int, vocab: int, sigma: float = 3.0,
                     stream: int = 11) -> np.ndarray:
    """[rows, vocab] float32 rows of a softmax over N(0, sigma^2) logits."""
    out = np.empty((rows, vocab), np.float32)
    rng = rng_for(seed, stream)
    for r in range(rows):
        z = rng.standard_normal(vocab) * sigma
        e = np.exp(z - z.max())
        out[r] = (e / e.sum()).astype(np.float32)
    return out


@dataclasses.dataclass
class TopKWorkload:
    name: str
    rows: int
    vocab: int
    k_range: tuple  # inclusive
    seed: int

    def top_k(self) -> np.ndarray:
        lo, hi = self.k_range
        return rng_for(self.seed, 12).integers(lo, hi + 1, size=self.rows).astype(np.int32)

    def probs(self) -> np.ndarray:
        return probability_rows(self.seed, self.rows, self.vocab)


# Top-k renormalisation of the target probabilities after a verify step: 32 sequences x
# 4 verify positions = 128 rows over a 163,840-entry vocabulary (the published Kimi K2
# tokenizer size; the pages give none), k drawn per row in [1, 100].
TOP_K_WORKLOADS = {
    "top_k_renorm_r128_v163840": TopKWorkload("top_k_renorm_r128_v163840", 128, 163840,
                                              (1, 100), seed=808),
}


# The five workloads the measurements are quoted on.
WORKLOADS = {
    # batch 1, one query, 12 heads, 1,024 keys, BF16, one contiguous block
    "decode_b1_h12_l1024_bf16": DecodeWorkload(
        "decode_b1_h12_l1024_bf16", 1, 1, 12, "bf16", 1024, seed=101, lengths=[1024]),
    # batch 32, 12 heads, lengths uniform in [4096, 16384], FP8 paged in 64-token blocks
    "decode_b32_h12_fp8_paged": DecodeWorkload(
        "decode_b32_h12_fp8_paged", 32, 1, 12, "fp8", 64, seed=202, length_range=(4096, 16384)),
    # 4 sequences x 4 verify positions, 12 heads, 32,768 context, BF16 paged
    "verify_b4_p4_h12_l32768_bf16": DecodeWorkload(
        "verify_b4_p4_h12_l32768_bf16", 4, 4, 12, "bf16", 64, seed=303, lengths=[32768] * 4),
    "verify_b4_p4_h8_l32768_bf16": DecodeWorkload(
        "verify_b4_p4_h8_l32768_bf16", 4, 4, 8, "bf16", 64, seed=303, lengths=[32768] * 4),
    "verify_b4_p4_h16_l32768_bf16": DecodeWorkload(
        "verify_b4_p4_h16_l32768_bf16", 4, 4, 16, "bf16", 64, seed=303, lengths=[32768] * 4),
    "verify_b4_p4_h12pad16_l32768_bf16": DecodeWorkload(
        "verify_b4_p4_h12pad16_l32768_bf16", 4, 4, 12, "bf16", 64, seed=303, lengths=[32768] * 4,
        pad_heads_to=16),
    # one sequence x 4 verify positions, 12 heads, 32,768 context, FP8 paged: the short
    # verify whose work-group count the pages discuss
    "verify_b1_p4_h12_l32768_fp8": DecodeWorkload(
        "verify_b1_p4_h12_l32768_fp8", 1, 4, 12, "fp8", 64, seed=707, lengths=[32768]),
    # batch 8, 12 heads, 142,000 keys, FP8 paged, 8 contiguous partitions merged by LSE
    "decode_b8_h12_l142000_fp8_8parts": DecodeWorkload(
        "decode_b8_h12_l142000_fp8_8parts", 8, 1, 12, "fp8", 64, seed=505, lengths=[142000] * 8,
        partitions=8),
    # one causal sequence of 32,768 tokens, 12 heads, BF16
    "prefill_t32768_h12_bf16": PrefillWorkload(
        "prefill_t32768_h12_bf16", [32768], 12, "bf16", seed=404),
}
