"""GPU parity of decode / verify with more than 64 query rows per sequence.

A sequence's P x H query rows go to the kernels in groups of at most 64 rows, one launch
each: whole positions when the heads fit in a group (5 positions x 16 heads: 4 + 1),
otherwise 64-head slices of one position (128 heads: 64 + 64; 100 heads: 64 + 36 per
position).  Each group keeps its rows' causal limits (position j of P sees keys
< seq_lens - P + j + 1), its place in q, out and lse, and shares the workspace with the
others.  Checked against the oracle on every row: both caches, both output dtypes, key
subranges, ragged lengths shorter than some groups' positions, every merge form (one
piece, shares merged in the launch, the separate merge), the shared verify kernel
(a long batch hint), and the allocation-free entry point (bitwise equal to mla_verify).
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


def case(seed, lens, P, H, kv_dtype, block_size=64):
    cache = mi.paged_cache(seed, lens, block_size, kv_dtype)
    q = mi.normal_bf16_bits(seed, 3, (len(lens), P, H, 576))
    return q, cache


def run_gpu(mla, q_bits, cache, *, kv_begin=None, kv_end=None, num_splits=0,
            out_dtype=torch.float32, hint=None):
    kv, bt, sl = cache_to_device(cache, DEV)
    out, lse = mla.verify(bf16_tensor(q_bits, DEV), kv, bt, sl, softmax_scale=SIGMA,
                          kv_scale=cache.kv_scale, kv_begin=i32(kv_begin, DEV),
                          kv_end=i32(kv_end, DEV), num_splits=num_splits,
                          out_dtype=out_dtype, max_kv_len=hint)
    torch.cuda.synchronize()
    return out, lse


def run_oracle(q_bits, cache, kv_begin=None, kv_end=None):
    return oracle.decode(q_bits, cache.kv, cache.kv_dtype == "fp8", cache.kv_scale,
                         cache.block_table, cache.seq_lens, SIGMA, kv_begin=kv_begin,
                         kv_end=kv_end)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("P,H", [(5, 16), (1, 128), (3, 100), (9, 8), (2, 65), (70, 1)])
def test_parity(mla, kv_dtype, P, H):
    lens = [P, 40, 300, 1500]
    q, cache = case(7400 + P * 7 + H, lens, P, H, kv_dtype)
    print("row groups", kv_dtype, P, H, flush=True)
    out, lse = run_gpu(mla, q, cache)
    ref_o, ref_l = run_oracle(q, cache)
    check_out(out, ref_o)
    check_lse(lse, ref_l)


@pytest.mark.parametrize("num_splits", [1, 3, 40, 300])
def test_every_merge_form(mla, num_splits):
    """One piece (no workspace), shares merged in the launch, and the separate merge, for
    each of the groups (here 4 + 4 + 2 positions x 16 heads)."""
    q, cache = case(7501, [10, 700, 2100], 10, 16, "fp8")
    out, lse = run_gpu(mla, q, cache, num_splits=num_splits)
    ref_o, ref_l = run_oracle(q, cache)
    check_out(out, ref_o)
    check_lse(lse, ref_l)


def test_shared_kernel_and_bf16_output(mla):
    """A long batch hint sends each 64-row group to the kernel whose work-group serves all
    four row blocks; BF16 outputs."""
    q, cache = case(7502, [6, 900, 3000], 6, 12, "bf16")
    out, lse = run_gpu(mla, q, cache, hint=65536, out_dtype=torch.bfloat16)
    assert out.dtype == torch.bfloat16
    ref_o, ref_l = run_oracle(q, cache)
    check_out(out, ref_o)
    check_lse(lse, ref_l)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_key_subranges(mla, kv_dtype):
    """kv_begin / kv_end with several groups of positions: the later groups' positions see
    more keys, and a range ending before a group's first position leaves its rows empty."""
    lens = [300, 1000, 520, 64]
    q, cache = case(7503, lens, 6, 16, kv_dtype)
    kb = np.array([17, 0, 500, 3], np.int32)
    ke = np.array([150, 1000, 517, 40], np.int32)
    for splits in (0, 9):
        out, lse = run_gpu(mla, q, cache, kv_begin=kb, kv_end=ke, num_splits=splits)
        ref_o, ref_l = run_oracle(q, cache, kb, ke)
        check_out(out, ref_o)
        check_lse(lse, ref_l)


def test_noalloc_matches(mla):
    """mla_verify_noalloc runs the same groups over its own scratch: bitwise equal."""
    q_np, cache = case(7504, [7, 800, 2000], 7, 16, "fp8")
    kv, bt, sl = cache_to_device(cache, DEV)
    q = bf16_tensor(q_np, DEV)
    for splits in (0, 5, 100):
        ref_o, ref_l = mla.verify(q, kv, bt, sl, softmax_scale=SIGMA, kv_scale=cache.kv_scale,
                                  max_kv_len=2000, num_splits=splits)
        out = torch.full_like(ref_o, float("nan"))
        lse = torch.full_like(ref_l, float("nan"))
        mla.verify_noalloc(q, kv, bt, sl, softmax_scale=SIGMA, kv_scale=cache.kv_scale,
                           max_kv_len=2000, num_splits=splits, out=out, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
    ref_o2, ref_l2 = run_oracle(q_np, cache)
    check_out(out, ref_o2)
    check_lse(lse, ref_l2)


def test_prefill_more_than_64_heads(mla):
    """The prefill tiles (token, head) rows of any head count: 80 and 128 heads."""
    for H, lens, seed in ((80, [1, 50, 77], 7505), (128, [33, 70], 7506)):
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        T = int(cu[-1])
        q_np = mi.normal_bf16_bits(seed, 3, (T, H, 576))
        kv_np = mi.normal_bf16_bits(seed, 4, (T, 576))
        out, lse = mla.prefill(bf16_tensor(q_np, DEV), bf16_tensor(kv_np, DEV),
                               torch.from_numpy(cu).to(DEV), softmax_scale=SIGMA,
                               max_seqlen=max(lens))
        torch.cuda.synchronize()
        ref_o, ref_l = oracle.prefill(q_np, kv_np, False, 1.0, cu, SIGMA)
        check_out(out, ref_o)
        check_lse(lse, ref_l)
