"""GPU parity of decode / verify for batches of more than 64 sequences, through the C-ABI.

Batches of up to 64 sequences find each work-group's first sequence with one wave; larger
batches take the work-group-wide path: a sum over the sequences in chunks of 256 (one per
thread), then an exclusive scan chunk by chunk with a carry, stopping at the chunk that
holds the piece's first entry.  These cases cross one chunk (65 sequences), two (257)
and three (600), with empty, short and long sequences mixed, kv_begin / kv_end subranges
(some empty, some at the chunk boundaries), one to four 16-row blocks, BF16 and FP8
caches, and every merge form: one piece per call (no workspace), the automatic plan
(shares merged in the launch) and more than 16 pieces per sequence (the separate merge
launch).  Every output row is compared with the oracle.
"""
import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle
from parity import bf16_tensor, cache_to_device, check_lse, check_out, i32

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SIGMA = mi.softmax_scale_for()


@pytest.fixture(scope="module")
def mla():
    import mla_latent_kv_attention_amd as m
    m.library()
    assert torch.cuda.is_available()
    return m


def mixed_lengths(seed, B, P):
    """40 % short (P .. 64 keys), 50 % medium (65 .. 1,200), 10 % long (1,201 .. 6,000)."""
    rng = np.random.default_rng(seed)
    kind = rng.random(B)
    lens = np.where(kind < 0.4, rng.integers(P, 65, B),
                    np.where(kind < 0.9, rng.integers(65, 1201, B), rng.integers(1201, 6001, B)))
    return lens.astype(np.int32)


def subranges(seed, lens):
    """kv_begin / kv_end: every 7th sequence a middle third, every 11th an empty range, the
    sequences around the 256-chunk boundaries empty or cut, the rest whole."""
    B = len(lens)
    kb = np.zeros(B, np.int32)
    ke = np.array(lens, np.int32)
    for b in range(B):
        L = int(lens[b])
        if b % 11 == 5:
            kb[b] = ke[b] = L // 2
        elif b % 7 == 3:
            kb[b], ke[b] = L // 3, (2 * L) // 3
    for b in (63, 64, 255, 256, 511, 512):
        if b < B:
            kb[b] = ke[b] = 0 if b % 2 else int(lens[b])
    for b in (65, 257, 513):
        if b < B:
            kb[b], ke[b] = 1, max(1, int(lens[b]) - 17)
    return kb, ke


CASES = [
    # (B, P, H, kv_dtype, seed)
    (65, 1, 12, "fp8", 5001),
    (65, 4, 16, "bf16", 5002),
    (257, 1, 12, "bf16", 5003),
    (257, 4, 8, "fp8", 5004),
    (600, 1, 12, "bf16", 5005),
    (600, 3, 12, "fp8", 5006),
]


@pytest.mark.parametrize("B,P,H,kv_dtype,seed", CASES)
def test_large_batches_every_merge_form(mla, B, P, H, kv_dtype, seed):
    lens = mixed_lengths(seed, B, P)
    cache = mi.paged_cache(seed, lens, 64, kv_dtype)
    q_bits = mi.normal_bf16_bits(seed, 3, (B, P, H, 576))
    kb, ke = subranges(seed, lens)
    ref_o, ref_l = oracle.decode(q_bits, cache.kv, kv_dtype == "fp8", cache.kv_scale,
                                 cache.block_table, cache.seq_lens, SIGMA, kv_begin=kb,
                                 kv_end=ke)
    kv, bt, sl = cache_to_device(cache, DEV)
    q = bf16_tensor(q_bits, DEV)
    span = int(np.max(ke - kb))
    auto = mla.decode_num_splits(B, P, H, span)
    separate = 16 * B + 1  # more than 16 pieces per sequence: the separate merge launch
    for splits in (1, 0, separate):
        print("case B=%d P=%d H=%d %s splits=%d (auto %d)" % (B, P, H, kv_dtype, splits, auto),
              flush=True)
        out, lse = mla.verify(q, kv, bt, sl, softmax_scale=SIGMA, kv_scale=cache.kv_scale,
                              kv_begin=i32(kb, DEV), kv_end=i32(ke, DEV), max_kv_len=span,
                              num_splits=splits)
        torch.cuda.synchronize()
        check_out(out, ref_o, "out (splits %d)" % splits)
        check_lse(lse, ref_l, "lse (splits %d)" % splits)
        empty = np.flatnonzero(ke <= kb)
        if empty.size:
            e = torch.from_numpy(empty).to(DEV)
            assert torch.all(out[e] == 0) and torch.all(torch.isneginf(lse[e]))


def test_large_batch_without_subranges_matches_whole_sequences(mla):
    """600 sequences over their whole ranges (kv_begin / kv_end absent), automatic plan."""
    B, P, H = 600, 1, 12
    lens = mixed_lengths(5007, B, P)
    cache = mi.paged_cache(5007, lens, 64, "fp8")
    q_bits = mi.normal_bf16_bits(5007, 3, (B, P, H, 576))
    kv, bt, sl = cache_to_device(cache, DEV)
    out, lse = mla.verify(bf16_tensor(q_bits, DEV), kv, bt, sl, softmax_scale=SIGMA,
                          kv_scale=cache.kv_scale, max_kv_len=int(lens.max()))
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.decode(q_bits, cache.kv, True, cache.kv_scale, cache.block_table,
                                 cache.seq_lens, SIGMA)
    check_out(out, ref_o)
    check_lse(lse, ref_l)


def test_large_batch_with_every_range_empty(mla):
    """No sequence has a visible key: the call writes zeros and lse = -inf everywhere."""
    B, P, H = 300, 2, 12
    lens = mixed_lengths(5008, B, P)
    cache = mi.paged_cache(5008, lens, 64, "bf16")
    q_bits = mi.normal_bf16_bits(5008, 3, (B, P, H, 576))
    kv, bt, sl = cache_to_device(cache, DEV)
    kb = np.array(lens, np.int32)
    out = torch.full((B, P, H, 512), float("nan"), device=DEV)
    lse = torch.full((B, P, H), float("nan"), device=DEV)
    mla.verify(bf16_tensor(q_bits, DEV), kv, bt, sl, softmax_scale=SIGMA, kv_begin=i32(kb, DEV),
               max_kv_len=100, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
