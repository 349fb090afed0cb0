"""GPU parity of the verify kernel whose work-group serves all of a piece's 16-row blocks.

Sequences with more than 16 query rows (positions x heads) over a batch key range of at
least 65,536 tokens (batch x the max_kv_len hint) take the kernel that copies each 32-token
tile of latent rows once into LDS and lets every row block's wave read it.  The hint only
shapes the plan (ranges longer or shorter than it are computed in full), so these small
cases pass a large hint to run that kernel on inputs the oracle checks row by row: 2, 3
and 4 row blocks (with padded last blocks), BF16 and FP8 caches, ragged lengths and
partial tiles, every merge form (one piece, shares merged in the launch, the separate
merge), key subranges, block sizes that put a tile across two blocks, a late key that
makes the work-group run its segment again, and the bitwise head padding / repetition
invariants.
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
HINT = 65536  # batch x hint >= 65,536 tokens: the shared kernel


@pytest.fixture(scope="module")
def mla():
    import mla_latent_kv_attention_amd as m
    m.library()
    assert torch.cuda.is_available()
    return m


def run_gpu(mla, q_bits, cache, *, kv_begin=None, kv_end=None, num_splits=0,
            out_dtype=torch.float32, hint=HINT):
    kv, bt, sl = cache_to_device(cache, DEV)
    out, lse = mla.verify(bf16_tensor(q_bits, DEV), kv, bt, sl, softmax_scale=SIGMA,
                          kv_scale=cache.kv_scale, kv_begin=i32(kv_begin, DEV),
                          kv_end=i32(kv_end, DEV), num_splits=num_splits, out_dtype=out_dtype,
                          max_kv_len=hint)
    torch.cuda.synchronize()
    return out, lse


def run_oracle(q_bits, cache, kv_begin=None, kv_end=None):
    return oracle.decode(q_bits, cache.kv, cache.kv_dtype == "fp8", cache.kv_scale,
                         cache.block_table, cache.seq_lens, SIGMA, kv_begin=kv_begin,
                         kv_end=kv_end)


def case(seed, lens, H, P, kv_dtype, block_size=64):
    cache = mi.paged_cache(seed, lens, block_size, kv_dtype)
    q = mi.normal_bf16_bits(seed, 3, (len(lens), P, H, 576))
    return q, cache


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("H,P", [(12, 4), (16, 4), (8, 4), (12, 2), (5, 7), (16, 3), (64, 1),
                                 (20, 2)])
def test_small_parity(mla, kv_dtype, H, P):
    lens = [P, 17, 64, 300, 1000, 33]
    q, cache = case(6000 + H * 10 + P, lens, H, P, kv_dtype)
    print("shared case", kv_dtype, H, P, flush=True)
    out, lse = run_gpu(mla, q, cache)
    ref_o, ref_l = run_oracle(q, cache)
    check_out(out, ref_o)
    check_lse(lse, ref_l)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("num_splits", [1, 2, 3, 7, 40, 300])
def test_split_counts_cover_every_merge_form(mla, kv_dtype, num_splits):
    """One piece (no workspace), up to 16 pieces per sequence (merged in the launch) and
    more (the separate merge); 300 pieces is more than there are steps."""
    q, cache = case(6101, [5, 333, 2047], 12, 4, kv_dtype)
    out, lse = run_gpu(mla, q, cache, num_splits=num_splits)
    ref_o, ref_l = run_oracle(q, cache)
    check_out(out, ref_o)
    check_lse(lse, ref_l)


@pytest.mark.parametrize("block_size", [16, 48, 64, 256])
def test_block_sizes(mla, block_size):
    """16- and 48-token blocks put the two halves of a 32-token tile in different blocks."""
    q, cache = case(6102, [1, 100, 700, 1234], 16, 4, "bf16", block_size=block_size)
    out, lse = run_gpu(mla, q, cache)
    ref_o, ref_l = run_oracle(q, cache)
    check_out(out, ref_o)
    check_lse(lse, ref_l)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_key_subranges_and_empty_ranges(mla, kv_dtype):
    lens = [200, 1000, 64, 513, 77]
    q, cache = case(6103, lens, 12, 3, kv_dtype)
    kb = np.array([17, 0, 64, 500, 3], np.int32)   # the third range is empty
    ke = np.array([150, 999, 64, 10000, 40], np.int32)
    for splits in (0, 9):
        out, lse = run_gpu(mla, q, cache, kv_begin=kb, kv_end=ke, num_splits=splits)
        ref_o, ref_l = run_oracle(q, cache, kb, ke)
        check_out(out, ref_o)
        check_lse(lse, ref_l)
        assert torch.all(out[2] == 0) and torch.all(torch.isneginf(lse[2]))


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_bf16_output(mla, kv_dtype):
    q, cache = case(6104, [3, 90, 1500], 16, 4, kv_dtype)
    out, lse = run_gpu(mla, q, cache, out_dtype=torch.bfloat16)
    assert out.dtype == torch.bfloat16
    ref_o, ref_l = run_oracle(q, cache)
    check_out(out, ref_o)
    check_lse(lse, ref_l)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("gain", [0.9, 2.0])
def test_late_score_jump(mla, kv_dtype, gain):
    """A key planted late in a sequence parallel to one row's query: ~54 (gain 0.9) or
    ~120 (gain 2) log2 units above the row's first tile maximum, below and above the cap
    of 64; above it the work-group runs its segment again from the true maximum."""
    lens = [900, 2500]
    q, cache = case(6105, lens, 12, 4, kv_dtype)
    qf = (q[1, 2, 5].astype(np.uint32) << 16).view(np.float32)
    t = 2301
    blk = cache.block_table[1, t // cache.block_size]
    if kv_dtype == "bf16":
        cache.kv[blk, t % cache.block_size] = mi.to_bf16_bits(gain * qf)
    else:
        cache.kv[blk, t % cache.block_size] = mi.to_fp8_codes(gain * qf, cache.kv_scale)
    for splits in (0, 3):
        out, lse = run_gpu(mla, q, cache, num_splits=splits)
        ref_o, ref_l = run_oracle(q, cache)
        check_out(out, ref_o)
        check_lse(lse, ref_l)
    assert ref_l[1, 2, 5] > ref_l[1, 2, 4] + 15


def test_padded_and_repeated_heads_are_bitwise_invariant(mla):
    """12 heads zero-padded to 16 (3 -> 4 row blocks) and 8 heads repeated to 16 (2 -> 4
    row blocks): the real rows come out bitwise equal at a fixed piece count."""
    q12, cache = case(6106, [900, 2048, 40], 12, 4, "bf16")
    q16 = np.zeros((3, 4, 16, 576), np.uint16)
    q16[:, :, :12] = q12
    o12, l12 = run_gpu(mla, q12, cache, num_splits=5)
    o16, l16 = run_gpu(mla, q16, cache, num_splits=5)
    assert torch.equal(o16[:, :, :12], o12) and torch.equal(l16[:, :, :12], l12)
    ref_o, ref_l = run_oracle(q16, cache)
    check_out(o16, ref_o)
    check_lse(l16, ref_l)
    q8 = np.ascontiguousarray(q12[:, :, :8])
    o8, l8 = run_gpu(mla, q8, cache, num_splits=7)
    o16r, l16r = run_gpu(mla, np.repeat(q8, 2, axis=2), cache, num_splits=7)
    for c in range(2):
        assert torch.equal(o16r[:, :, c::2], o8) and torch.equal(l16r[:, :, c::2], l8)


def test_runs_repeat_bitwise_and_every_piece_count_meets_the_bar(mla):
    """A fixed piece count gives bitwise the same result on every run; different piece
    counts round the weights against different references and sum in a different order,
    so each is checked against the oracle on its own."""
    q, cache = case(6107, [4000, 2500, 700], 12, 4, "fp8")
    ref_o, ref_l = run_oracle(q, cache)
    for splits in (1, 9, 33):
        a, la = run_gpu(mla, q, cache, num_splits=splits)
        a2, la2 = run_gpu(mla, q, cache, num_splits=splits)
        assert torch.equal(a, a2) and torch.equal(la, la2)
        check_out(a, ref_o)
        check_lse(la, ref_l)


def test_noalloc_entry_point_takes_the_shared_kernel(mla):
    """mla_verify_noalloc on the same plan: bitwise equal to mla_verify."""
    q_np, cache = case(6108, [300, 1500, 64], 12, 4, "bf16")
    kv, bt, sl = cache_to_device(cache, DEV)
    q = bf16_tensor(q_np, DEV)
    for splits in (0, 12):
        ref_o, ref_l = mla.verify(q, kv, bt, sl, softmax_scale=SIGMA, max_kv_len=HINT,
                                  num_splits=splits)
        out = torch.full_like(ref_o, float("nan"))
        lse = torch.full_like(ref_l, float("nan"))
        mla.verify_noalloc(q, kv, bt, sl, softmax_scale=SIGMA, max_kv_len=HINT,
                           num_splits=splits, out=out, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
