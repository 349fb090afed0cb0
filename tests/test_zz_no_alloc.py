"""mla_verify_noalloc (the entry point for callers that cannot allocate) against
mla_verify with a workspace, through the C-ABI: the same kernels and plan, so the
results must be bitwise equal, and both within the bar of the oracle.  Two calls in a
row into the library's shared scratch, the second with a smaller input (and the other
merge form), then a call too large for the scratch, refused before any launch."""
import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle
from parity import bf16_tensor, cache_to_device, check_lse, check_out

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SIGMA = mi.softmax_scale_for()


@pytest.fixture(scope="module")
def mla():
    import mla_latent_kv_attention_amd as m
    m.library()
    assert torch.cuda.is_available()
    return m


def one_case(mla, seed, lens, P, H, kv_dtype, splits, out_dtype):
    cache = mi.paged_cache(seed, lens, 64, kv_dtype)
    q_np = mi.normal_bf16_bits(seed, 3, (len(lens), P, H, 576))
    kv, bt, sl = cache_to_device(cache, DEV)
    q = bf16_tensor(q_np, DEV)
    B, L = len(lens), max(lens)
    print("noalloc case B=%d P=%d H=%d %s splits=%d" % (B, P, H, kv_dtype, splits), flush=True)
    ref_o, ref_l = mla.verify(q, kv, bt, sl, softmax_scale=SIGMA, kv_scale=cache.kv_scale,
                              max_kv_len=L, num_splits=splits, out_dtype=out_dtype)
    out = torch.full((B, P, H, 512), float("nan"), dtype=out_dtype, device=DEV)
    lse = torch.full((B, P, H), float("nan"), device=DEV)
    mla.verify_noalloc(q, kv, bt, sl, softmax_scale=SIGMA, kv_scale=cache.kv_scale,
                       max_kv_len=L, num_splits=splits, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
    o_np, l_np = oracle.decode(q_np, cache.kv, kv_dtype == "fp8", cache.kv_scale,
                               cache.block_table, cache.seq_lens, SIGMA)
    check_out(out, o_np)
    check_lse(lse, l_np)
    return mla.decode_workspace_size(B, P, H, L, splits)


def test_noalloc_matches_verify_on_two_calls_in_a_row(mla):
    lib = mla.library()
    # 1: 24 sequences, automatic plan (shares merged in the launch), FP32 out
    lens1 = list(np.random.default_rng(9001).integers(200, 9000, 24))
    need1 = one_case(mla, 9001, lens1, 1, 12, "fp8", 0, torch.float32)
    # 2: smaller -- 3 sequences x 4 positions, more than 16 pieces per sequence (the
    # separate merge), BF16 out
    need2 = one_case(mla, 9002, [37, 700, 2100], 4, 12, "bf16", 60, torch.bfloat16)
    assert 0 < need2 < need1 <= (32 << 20)
    # 3: the first case again after the second (the scratch keeps the last call's data)
    one_case(mla, 9001, lens1, 1, 12, "fp8", 0, torch.float32)


def test_noalloc_refuses_a_call_beyond_its_scratch(mla):
    B, P, H = 64, 4, 16
    need = mla.decode_workspace_size(B, P, H, 100000, 60000)
    assert need > (32 << 20)
    cache = mi.paged_cache(9003, [64] * B, 64, "bf16")
    kv, bt, sl = cache_to_device(cache, DEV)
    q = torch.zeros((B, P, H, 576), dtype=torch.bfloat16, device=DEV)
    out = torch.zeros((B, P, H, 512), device=DEV)
    with pytest.raises(mla.MlaError) as e:
        mla.verify_noalloc(q, kv, bt, sl, softmax_scale=SIGMA, max_kv_len=100000,
                           num_splits=60000, out=out)
    assert e.value.status == -5
