"""The decode workspace's error flags and the in-launch merge under repetition, on the GPU.

Error flags are forced from the host, and every kernel still runs to its normal end:
  * stale completion counters: a zero-filled workspace whose counter block is then set
    high, as an interrupted or overlapping call would leave it; the call flags it, the
    binding's check raises and re-zeroes, and the next call is right again;
  * lengths outside the contract (a sequence shorter than its P query positions, a
    negative kv_begin), which the kernels clamp: flagged, nothing else breaks.
The soak: about 2,000 calls whose split sequences are merged in the launch by the last
piece to finish (agent-coherent stores, a relaxed counter, agent-coherent loads), over
several piece counts and both decode kernels, each call bitwise equal to the first call
with the same piece count; it stops at the first mismatch.
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


@pytest.mark.parametrize("hint", [2100, 65536])  # the one-row-block-per-work-group and shared kernels
def test_stale_counters_are_flagged_and_reset(mla, hint):
    lens = [37, 700, 2100]
    cache = mi.paged_cache(7301, lens, 64, "fp8")
    q_np = mi.normal_bf16_bits(7301, 3, (3, 4, 12, 576))
    kv, bt, sl = cache_to_device(cache, DEV)
    q = bf16_tensor(q_np, DEV)
    splits = 20  # at most 16 per sequence on average: merged in the launch
    ws = torch.zeros(mla.decode_workspace_size(3, 4, 12, hint, splits), dtype=torch.uint8,
                     device=DEV)
    ref_o, ref_l = oracle.decode(q_np, cache.kv, True, cache.kv_scale, cache.block_table,
                                 cache.seq_lens, SIGMA)

    def call():
        o, l = mla.verify(q, kv, bt, sl, softmax_scale=SIGMA, kv_scale=cache.kv_scale,
                          max_kv_len=hint, num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        return o, l

    o, l = call()
    mla.check_decode_workspace(ws)  # clean
    check_out(o, ref_o)
    check_lse(l, ref_l)
    ws[:4 * 64].view(torch.int32).fill_(1000)  # counters far above any piece count
    call()
    assert mla.decode_workspace_flags(ws) & mla.FLAG_STALE_COUNTERS
    with pytest.raises(mla.WorkspaceError):
        mla.check_decode_workspace(ws)
    assert mla.decode_workspace_flags(ws) == 0
    assert torch.all(ws[:4 * 65536].view(torch.int32) == 0)
    o, l = call()
    mla.check_decode_workspace(ws)
    check_out(o, ref_o)
    check_lse(l, ref_l)


@pytest.mark.parametrize("hint", [2000, 65536])
def test_lengths_outside_the_contract_are_flagged(mla, hint):
    """Sequence 1 holds 2 keys but 4 query positions, sequence 2 starts at kv_begin -5
    (clamped to 0); the other sequences are checked against the oracle as usual."""
    lens = [500, 2, 900]
    cache = mi.paged_cache(7302, lens, 64, "bf16")
    q_np = mi.normal_bf16_bits(7302, 3, (3, 4, 12, 576))
    kv, bt, sl = cache_to_device(cache, DEV)
    kb = np.array([0, 0, -5], np.int32)
    ws = torch.zeros(mla.decode_workspace_size(3, 4, 12, hint, 9), dtype=torch.uint8, device=DEV)
    o, l = mla.verify(bf16_tensor(q_np, DEV), kv, bt, sl, softmax_scale=SIGMA,
                      kv_begin=i32(kb, DEV), max_kv_len=hint, num_splits=9, workspace=ws)
    torch.cuda.synchronize()
    assert mla.decode_workspace_flags(ws) == mla.FLAG_BAD_LENGTHS
    ref_o, ref_l = oracle.decode(q_np, cache.kv, False, 1.0, cache.block_table, cache.seq_lens,
                                 SIGMA, kv_begin=np.maximum(kb, 0))
    check_out(o[0], ref_o[0])
    check_lse(l[0], ref_l[0])
    check_out(o[2], ref_o[2])
    check_lse(l[2], ref_l[2])
    mla.reset_decode_workspace(ws)


def test_in_launch_merge_soak(mla):
    """About 2,000 calls with the shares merged in the launch, bitwise against the first
    call of each piece count."""
    lens = list(np.random.default_rng(7303).integers(100, 6000, 8))
    cache = mi.paged_cache(7303, lens, 64, "fp8")
    kv, bt, sl = cache_to_device(cache, DEV)
    cases = []
    for P, hint in ((1, 6000), (4, 65536)):  # decode kernel; shared verify kernel
        q = bf16_tensor(mi.normal_bf16_bits(7303 + P, 3, (8, P, 12, 576)), DEV)
        for splits in (3, 8, 17, 31, 64, 100, 128):
            ws = torch.zeros(mla.decode_workspace_size(8, P, 12, hint, splits), dtype=torch.uint8,
                             device=DEV)
            out = torch.empty((8, P, 12, 512), device=DEV)
            lse = torch.empty((8, P, 12), device=DEV)
            f = mla.verify_launcher(q, kv, bt, sl, softmax_scale=SIGMA, kv_scale=cache.kv_scale,
                                    max_kv_len=hint, out=out, lse=lse, workspace=ws,
                                    num_splits=splits)
            f()
            torch.cuda.synchronize()
            cases.append((P, splits, f, out, lse, out.clone(), lse.clone(), ws))
    calls = 0
    for rnd in range(2000 // len(cases) + 1):
        for P, splits, f, out, lse, ref_o, ref_l, ws in cases:
            out.fill_(float("nan"))
            f()
            calls += 1
            if not (torch.equal(out, ref_o) and torch.equal(lse, ref_l)):
                raise AssertionError("call %d (P=%d, %d pieces) differs from the first"
                                     % (calls, P, splits))
    for case in cases:
        mla.check_decode_workspace(case[7])
    print("soak: %d calls bitwise equal" % calls, flush=True)
    assert calls >= 2000


@pytest.mark.parametrize("hint", [2000, 65536])  # the one-row-block-per-work-group and shared kernels
def test_negative_block_ids_are_flagged_and_read_as_block_zero(mla, hint):
    """A negative block-table entry (outside the contract) for a visible block of sequence 1:
    the kernels read block 0 in its place (never memory before the cache) and flag the call;
    the other sequences are checked against the oracle as usual.  The allocation-free entry
    point (no flags) reads block 0 the same way."""
    lens = [300, 700, 900]
    cache = mi.paged_cache(7304, lens, 64, "fp8")
    q_np = mi.normal_bf16_bits(7304, 3, (3, 4, 12, 576))
    kv, bt, sl = cache_to_device(cache, DEV)
    bt[1, 2] = -3  # tokens 128 .. 191 of sequence 1
    q = bf16_tensor(q_np, DEV)
    ws = torch.zeros(mla.decode_workspace_size(3, 4, 12, hint, 9), dtype=torch.uint8, device=DEV)
    o, l = mla.verify(q, kv, bt, sl, softmax_scale=SIGMA, kv_scale=cache.kv_scale,
                      max_kv_len=hint, num_splits=9, workspace=ws)
    torch.cuda.synchronize()
    assert mla.decode_workspace_flags(ws) == mla.FLAG_BAD_BLOCKS
    with pytest.raises(mla.WorkspaceError):
        mla.check_decode_workspace(ws)
    ref_o, ref_l = oracle.decode(q_np, cache.kv, True, cache.kv_scale, cache.block_table,
                                 cache.seq_lens, SIGMA)
    for b in (0, 2):
        check_out(o[b], ref_o[b])
        check_lse(l[b], ref_l[b])
    o2 = torch.full_like(o, float("nan"))
    l2 = torch.full_like(l, float("nan"))
    mla.verify_noalloc(q, kv, bt, sl, softmax_scale=SIGMA, kv_scale=cache.kv_scale,
                       max_kv_len=hint, num_splits=9, out=o2, lse=l2)
    torch.cuda.synchronize()
    for b in (0, 2):
        check_out(o2[b], ref_o[b])
        check_lse(l2[b], ref_l[b])
