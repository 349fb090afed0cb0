"""Guard bands: every entry point writes exactly its outputs and nothing around them.

Each output, lse and workspace buffer handed to the library is the middle of a larger
allocation whose head and tail hold a sentinel bit pattern; after the call (and after a
second call into the same buffers) the sentinels must be untouched, bit for bit.  The
decode workspace's counter block must be zero again after every call, and the parts of
a workspace beyond the size the library asked for must be untouched.  Cases cover the
decode / verify merge forms (one piece, shares merged in the launch, the separate merge
under the automatic plan and forced),
FP32 and BF16 outputs, prefill, the stand-alone merge, the cache write (slots not named
stay as they were) and the top-k renormalisation.
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
GUARD_BYTES = 4096
SENTINEL = 0xA5


@pytest.fixture(scope="module")
def mla():
    import mla_latent_kv_attention_amd as m
    m.library()
    assert torch.cuda.is_available()
    return m


class Guarded:
    """A contiguous tensor of `shape` / `dtype` inside a byte buffer with sentinel guards."""

    def __init__(self, shape, dtype, fill=None):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.raw = torch.full((GUARD_BYTES + n + GUARD_BYTES,), SENTINEL, dtype=torch.uint8,
                              device=DEV)
        self.n = n
        self.t = self.raw[GUARD_BYTES:GUARD_BYTES + n].view(dtype).view(shape)
        if fill is not None:
            self.t.fill_(fill)

    def check(self, what):
        head = self.raw[:GUARD_BYTES]
        tail = self.raw[GUARD_BYTES + self.n:]
        assert torch.all(head == SENTINEL), what + ": head guard overwritten"
        assert torch.all(tail == SENTINEL), what + ": tail guard overwritten"


def guarded_workspace(need):
    """A workspace of `need` bytes (counters zero, the rest sentinel) inside guards, plus
    an extra tail the library must not touch either."""
    raw = torch.full((GUARD_BYTES + need + GUARD_BYTES,), SENTINEL, dtype=torch.uint8,
                     device=DEV)
    ws = raw[GUARD_BYTES:GUARD_BYTES + need]
    ws[:65536 * 4].zero_()
    return raw, ws


def check_workspace(raw, need, what):
    assert torch.all(raw[:GUARD_BYTES] == SENTINEL), what + ": workspace head guard"
    assert torch.all(raw[GUARD_BYTES + need:] == SENTINEL), what + ": workspace tail guard"
    ws = raw[GUARD_BYTES:GUARD_BYTES + need]
    assert torch.all(ws[:65536 * 4].view(torch.int32) == 0), what + ": counters not zero"


@pytest.mark.parametrize("splits", [1, 12, 0, 300])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_verify_writes_only_its_outputs(mla, splits, out_dtype):
    lens = [70, 2000, 777, 5]
    B, P, H = 4, 3, 12
    cache = mi.paged_cache(7201, lens, 64, "fp8")
    q_np = mi.normal_bf16_bits(7201, 3, (B, P, H, 576))
    kv, bt, sl = cache_to_device(cache, DEV)
    q = bf16_tensor(q_np, DEV)
    kb = np.array([0, 100, 0, 5], np.int32)  # the last range is empty
    ke = np.array(lens, np.int32)
    ref_o, ref_l = oracle.decode(q_np, cache.kv, True, cache.kv_scale, cache.block_table,
                                 cache.seq_lens, SIGMA, kv_begin=kb, kv_end=ke)
    need = mla.decode_workspace_size(B, P, H, 2000, splits)
    out = Guarded((B, P, H, 512), out_dtype)
    lse = Guarded((B, P, H), torch.float32)
    raw, ws = guarded_workspace(max(need, 65536 * 4))
    for call in range(2):
        print("verify splits=%d %s call %d" % (splits, out_dtype, call), flush=True)
        mla.verify(q, kv, bt, sl, softmax_scale=SIGMA, kv_scale=cache.kv_scale,
                   kv_begin=i32(kb, DEV), kv_end=i32(ke, DEV), max_kv_len=2000,
                   num_splits=splits, out_dtype=out_dtype, out=out.t, lse=lse.t,
                   workspace=ws if need else None)
        torch.cuda.synchronize()
        out.check("out")
        lse.check("lse")
        check_workspace(raw, max(need, 65536 * 4), "workspace")
        check_out(out.t, ref_o)
        check_lse(lse.t, ref_l)


def test_decode_without_lse_writes_only_out(mla):
    lens = [3000, 64]
    cache = mi.paged_cache(7202, lens, 64, "bf16")
    q_np = mi.normal_bf16_bits(7202, 3, (2, 16, 576))
    kv, bt, sl = cache_to_device(cache, DEV)
    out = Guarded((2, 16, 512), torch.float32)
    mla.decode(bf16_tensor(q_np, DEV), kv, bt, sl, softmax_scale=SIGMA, max_kv_len=3000,
               out=out.t, return_lse=False)
    torch.cuda.synchronize()
    out.check("out")
    ref_o, _ = oracle.decode(q_np.reshape(2, 1, 16, 576), cache.kv, False, 1.0,
                             cache.block_table, cache.seq_lens, SIGMA)
    check_out(out.t, ref_o.reshape(2, 16, 512))


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_prefill_writes_only_its_outputs(mla, out_dtype):
    lens = [129, 0, 33, 300]
    H = 12
    d = mi.prefill_inputs(mi.PrefillWorkload("guard", lens, H, "fp8", seed=7203))
    T = sum(lens)
    out = Guarded((T, H, 512), out_dtype)
    lse = Guarded((T, H), torch.float32)
    for call in range(2):
        mla.prefill(bf16_tensor(d["q"], DEV), torch.from_numpy(d["kv"]).to(DEV),
                    i32(d["cu_seqlens"], DEV), softmax_scale=SIGMA, kv_scale=d["kv_scale"],
                    out_dtype=out_dtype, max_seqlen=300, out=out.t, lse=lse.t)
        torch.cuda.synchronize()
        out.check("prefill out")
        lse.check("prefill lse")
    ref_o, ref_l = oracle.prefill(d["q"], d["kv"], True, d["kv_scale"], d["cu_seqlens"], SIGMA)
    check_out(out.t, ref_o)
    check_lse(lse.t, ref_l)


@pytest.mark.parametrize("S", [3, 8, 11])
def test_merge_lse_writes_only_its_outputs(mla, S):
    rng = np.random.default_rng(7204 + S)
    N = 29
    po = torch.from_numpy(rng.standard_normal((S, N, 512)).astype(np.float32)).to(DEV)
    pl_np = (rng.standard_normal((S, N)) * 2).astype(np.float32)
    pl_np[:, 4] = -np.inf
    pl = torch.from_numpy(pl_np).to(DEV)
    out = Guarded((N, 512), torch.bfloat16)
    lse = Guarded((N,), torch.float32)
    mla.merge_lse(po, pl, out_dtype=torch.bfloat16, out=out.t, lse=lse.t)
    torch.cuda.synchronize()
    out.check("merge out")
    lse.check("merge lse")
    ref_o, ref_l = oracle.merge(po.cpu().numpy().astype(np.float64), pl_np.astype(np.float64))
    check_out(out.t, ref_o)
    check_lse(lse.t, ref_l)


def test_cache_write_touches_only_the_named_slots(mla):
    N, num_blocks, bs = 300, 12, 64
    latent_np = mi.normal_bf16_bits(7205, 1, (N, 576))
    slots = np.random.default_rng(7205).permutation(num_blocks * bs)[:N].astype(np.int32)
    slots[::17] = -1                 # padding rows are skipped
    slots[5] = num_blocks * bs + 3   # out of range: skipped
    cache = Guarded((num_blocks, bs, 576), torch.uint8, fill=0x3C)
    mla.cache_write(bf16_tensor(latent_np, DEV), cache.t, i32(slots, DEV), kv_scale=0.01)
    torch.cuda.synchronize()
    cache.check("cache")
    want = oracle.cache_write(latent_np, slots, np.full((num_blocks, bs, 576), 0x3C, np.uint8),
                              True, 0.01)
    assert np.array_equal(cache.t.cpu().numpy(), want)


def test_top_k_renorm_writes_only_its_output(mla):
    rows, vocab = 5, 20000
    p_np = mi.probability_rows(7206, rows, vocab)
    k_np = np.array([1, 7, 0, 3000, 50], np.int32)
    out = Guarded((rows, vocab), torch.float32)
    need = mla.top_k_renorm_workspace_size(rows, vocab)
    raw = torch.full((GUARD_BYTES + need + GUARD_BYTES,), SENTINEL, dtype=torch.uint8, device=DEV)
    ws = raw[GUARD_BYTES:GUARD_BYTES + need]
    mla.top_k_renorm_prob(torch.from_numpy(p_np).to(DEV), i32(k_np, DEV), out=out.t, workspace=ws)
    torch.cuda.synchronize()
    out.check("top-k out")
    assert torch.all(raw[:GUARD_BYTES] == SENTINEL) and torch.all(raw[-GUARD_BYTES:] == SENTINEL)
    want = oracle.top_k_renorm_prob(p_np, k_np)
    got = out.t.cpu().numpy()
    assert np.array_equal(got != 0, want != 0)
    m = want != 0
    assert np.max(np.abs(got[m] - want[m]) / want[m]) <= 2e-6
