"""GPU parity of decode / verify / merge against the FP64 oracle, through the C-ABI.

Small cases (the oracle computes every row) span several 16-token steps, several
pieces of the batch's step list, ragged tails, partial last blocks, empty key ranges, 8 / 12 / 16 heads, one to
four query positions, BF16 and FP8 caches, FP32 and BF16 outputs.  The full-size
workloads run in the launch configuration the bench times (automatic split plan) and
are checked on every row.  Invariants: piece count, head padding and head repetition
(bitwise), power-of-two scalings of q, the softmax scale and the FP8 scale (bitwise),
paging layout, run-to-run determinism, and the workspace contract (counters left zero).
"""
import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle
from parity import bf16_tensor, cache_to_device, check_lse, check_out, i32, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SIGMA = mi.softmax_scale_for()


@pytest.fixture(scope="module")
def mla():
    import mla_latent_kv_attention_amd as m
    m.library()
    assert torch.cuda.is_available()
    return m


def run_gpu(mla, q_bits, cache, *, kv_begin=None, kv_end=None, num_splits=0,
            out_dtype=torch.float32, max_kv_len=None):
    kv, bt, sl = cache_to_device(cache, DEV)
    q = bf16_tensor(q_bits, DEV)
    out, lse = mla.verify(q, kv, bt, sl, softmax_scale=SIGMA, kv_scale=cache.kv_scale,
                          kv_begin=i32(kv_begin, DEV), kv_end=i32(kv_end, DEV),
                          num_splits=num_splits, out_dtype=out_dtype, max_kv_len=max_kv_len)
    torch.cuda.synchronize()
    return out, lse


def run_oracle(q_bits, cache, kv_begin=None, kv_end=None, rows=None):
    return oracle.decode(q_bits, cache.kv, cache.kv_dtype == "fp8", cache.kv_scale,
                         cache.block_table, cache.seq_lens, SIGMA, kv_begin=kv_begin,
                         kv_end=kv_end, rows=rows)


def small_case(seed, lens, H, P, kv_dtype, block_size=64):
    cache = mi.paged_cache(seed, lens, block_size, kv_dtype)
    q = mi.normal_bf16_bits(seed, 3, (len(lens), P, H, 576))
    return q, cache


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("H,P", [(12, 1), (8, 1), (16, 1), (12, 4), (16, 4), (8, 2), (1, 1), (5, 3)])
def test_small_parity(mla, kv_dtype, H, P):
    lens = [P, 17, 64, 300, 1000]
    q, cache = small_case(1000 + H * 10 + P, lens, H, P, kv_dtype)
    print("case", kv_dtype, H, P, flush=True)
    out, lse = run_gpu(mla, q, cache)
    ref_o, ref_l = run_oracle(q, cache)
    check_out(out, ref_o)
    check_lse(lse, ref_l)


@pytest.mark.parametrize("num_splits", [1, 2, 3, 7, 40, 300])
def test_explicit_split_counts(mla, num_splits):
    """Pieces of the concatenated 16-token step list (152 steps here); 300 pieces is more
    than there are steps, so only the first 152 take work."""
    q, cache = small_case(2001, [5, 333, 2047], 12, 2, "fp8")
    out, lse = run_gpu(mla, q, cache, num_splits=num_splits)
    ref_o, ref_l = run_oracle(q, cache)
    check_out(out, ref_o)
    check_lse(lse, ref_l)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("block_size", [16, 48, 64, 256])
def test_block_sizes(mla, block_size, kv_dtype):
    q, cache = small_case(2002, [1, 100, 700], 12, 1, kv_dtype, block_size=block_size)
    out, lse = run_gpu(mla, q, cache)
    ref_o, ref_l = run_oracle(q, cache)
    check_out(out, ref_o)
    check_lse(lse, ref_l)


@pytest.mark.parametrize("num_splits", [0, 9, 40])
def test_fp8_steps_and_starts_inside_steps(mla, num_splits):
    """FP8 caches load whole 16-token steps, poisoned rows past a sequence's end
    included, and take steps in pairs: lengths and key ranges that start and end inside
    a step, with piece counts that leave waves zero, one, two or more steps (an unpaired
    last step, prefetches past a wave's end), every row against the oracle."""
    lens = [2, 15, 16, 17, 47, 63, 64, 65, 130, 257, 1001]
    kb = np.array([0, 3, 0, 9, 1, 62, 0, 33, 100, 0, 517], np.int32)
    q, cache = small_case(2020, lens, 12, 2, "fp8", block_size=16)
    out, lse = run_gpu(mla, q, cache, kv_begin=kb, num_splits=num_splits)
    ref_o, ref_l = run_oracle(q, cache, kb)
    check_out(out, ref_o)
    check_lse(lse, ref_l)


@pytest.mark.parametrize("num_splits", [0, 200])
def test_bf16_output(mla, num_splits):
    """Automatic plan (the separate merge over whole rows) and 200 pieces for 3
    sequences (the separate merge over row quarters)."""
    q, cache = small_case(2003, [3, 90, 1500], 16, 4, "bf16")
    out, lse = run_gpu(mla, q, cache, out_dtype=torch.bfloat16, num_splits=num_splits)
    assert out.dtype == torch.bfloat16
    ref_o, ref_l = run_oracle(q, cache)
    check_out(out, ref_o)
    check_lse(lse, ref_l)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_key_subranges_and_empty_ranges(mla, kv_dtype):
    lens = [200, 1000, 64, 513]
    P = 3
    q, cache = small_case(2004, lens, 12, P, kv_dtype)
    kb = np.array([17, 0, 64, 500], np.int32)   # the third range is empty
    ke = np.array([150, 999, 64, 10000], np.int32)
    out, lse = run_gpu(mla, q, cache, kv_begin=kb, kv_end=ke)
    ref_o, ref_l = run_oracle(q, cache, kb, ke)
    check_out(out, ref_o)
    check_lse(lse, ref_l)
    assert torch.all(out[2] == 0) and torch.all(torch.isneginf(lse[2]))


def test_hint_smaller_than_the_range_still_covers_it(mla):
    q, cache = small_case(2005, [3000], 12, 1, "fp8")
    out, lse = run_gpu(mla, q, cache, max_kv_len=100)
    ref_o, ref_l = run_oracle(q, cache)
    check_out(out, ref_o)
    check_lse(lse, ref_l)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("gain", [0.9, 2.0])
def test_late_score_jump(mla, kv_dtype, gain):
    """A key planted late in a sequence, parallel to one head's query: its score is about
    gain * |q|^2 / sqrt(192) (~54 log2 units at gain 0.9, ~120 at gain 2), far above the
    reference maximum the row started from.  Below the kernel's cap of 64 log2 units the
    row keeps its reference and carries large probabilities; above it the wave runs its
    steps again from the true maximum.  Both must match the oracle."""
    lens = [900, 2500]
    q, cache = small_case(2014, lens, 12, 1, kv_dtype)
    qf = (q[1, 0, 5].astype(np.uint32) << 16).view(np.float32)
    t = 2301  # late in sequence 1
    blk = cache.block_table[1, t // cache.block_size]
    if kv_dtype == "bf16":
        cache.kv[blk, t % cache.block_size] = mi.to_bf16_bits(gain * qf)
    else:
        cache.kv[blk, t % cache.block_size] = mi.to_fp8_codes(gain * qf, cache.kv_scale)
    out, lse = run_gpu(mla, q, cache, num_splits=3)
    ref_o, ref_l = run_oracle(q, cache)
    check_out(out, ref_o)
    check_lse(lse, ref_l)
    assert ref_l[1, 0, 5] > ref_l[1, 0, 4] + 15  # the planted key dominates that row


@pytest.mark.parametrize("S", [5, 8, 13, 20])
def test_merge_lse_matches_oracle(mla, S):
    """Partials are combined in batches of eight: one batch, exactly one, and several
    with a ragged last batch."""
    rng = np.random.default_rng(7 + S)
    N = 37
    po = rng.standard_normal((S, N, 512)).astype(np.float32)
    pl = (rng.standard_normal((S, N)) * 3).astype(np.float32)
    pl[:, 3] = -np.inf                 # a row with no keys anywhere
    pl[1:4, 5] = -np.inf               # a row with some empty pieces
    po[1:4, 5] = np.nan                # their partial outputs are never read
    out, lse = mla.merge_lse(torch.from_numpy(po).to(DEV), torch.from_numpy(pl).to(DEV))
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.merge(np.nan_to_num(po.astype(np.float64)), pl.astype(np.float64))
    check_out(out, ref_o)
    check_lse(lse, ref_l)


def test_split_results_agree_and_are_deterministic(mla):
    q, cache = small_case(2006, [4000, 2500], 12, 1, "fp8")
    a, la = run_gpu(mla, q, cache, num_splits=1)
    b, lb = run_gpu(mla, q, cache, num_splits=9)
    b2, lb2 = run_gpu(mla, q, cache, num_splits=9)
    assert torch.equal(b, b2) and torch.equal(lb, lb2)
    assert (a - b).abs().max().item() < 1e-3
    assert (la - lb).abs().max().item() < 1e-5


def test_zero_padded_heads_are_bitwise_invariant(mla):
    q12, cache = small_case(2007, [900, 2048], 12, 4, "bf16")
    q16 = np.zeros((2, 4, 16, 576), np.uint16)
    q16[:, :, :12] = q12
    o12, l12 = run_gpu(mla, q12, cache, num_splits=5)
    o16, l16 = run_gpu(mla, q16, cache, num_splits=5)
    assert torch.equal(o16[:, :, :12], o12) and torch.equal(l16[:, :, :12], l12)
    # the padded heads see all-zero scores: the mean of the visible values, lse = ln n
    ref_o, ref_l = run_oracle(q16, cache)
    check_out(o16[:, :, 12:], ref_o[:, :, 12:])
    check_lse(l16[:, :, 12:], ref_l[:, :, 12:])


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_repeated_heads_are_bitwise_invariant(mla, kv_dtype):
    """Head repetition 8 -> 16 (each head's query twice, as a caller that needs 16 heads
    would feed 8 real ones): both copies of every head come out bitwise equal to the
    8-head call at the same piece count, whichever 16-row block they land in."""
    q8, cache = small_case(2015, [900, 2048, 37], 8, 4, kv_dtype)
    q16 = np.repeat(q8, 2, axis=2)
    o8, l8 = run_gpu(mla, q8, cache, num_splits=5)
    o16, l16 = run_gpu(mla, q16, cache, num_splits=5)
    for c in range(2):
        assert torch.equal(o16[:, :, c::2], o8) and torch.equal(l16[:, :, c::2], l8)
    ref_o, ref_l = run_oracle(q8, cache)
    check_out(o8, ref_o)
    check_lse(l8, ref_l)


def scaled_bf16_bits(bits: np.ndarray, c: float) -> np.ndarray:
    """BF16 bit patterns multiplied by a power of two c (exact for these magnitudes)."""
    f = (bits.astype(np.uint32) << 16).view(np.float32) * np.float32(c)
    out = mi.to_bf16_bits(f)
    assert np.array_equal((out.astype(np.uint32) << 16).view(np.float32), f)
    return out


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("splits", [1, 6, 200])
def test_power_of_two_scale_invariants(mla, kv_dtype, splits):
    """Scores depend on q and the softmax scale only through their product, and an FP8
    cache's values through code x kv_scale: (q * c, scale / c) gives bitwise the same
    out and lse for a power of two c, and (kv_scale * c, scale / c) gives out * c and the
    same lse, in every merge form (one piece, shares merged in the launch, the separate
    merge)."""
    q, cache = small_case(2016, [700, 1500, 64], 12, 2, kv_dtype)
    kv, bt, sl = cache_to_device(cache, DEV)

    def run(q_bits, scale, kv_scale):
        o, l = mla.verify(bf16_tensor(q_bits, DEV), kv, bt, sl, softmax_scale=scale,
                          kv_scale=kv_scale, num_splits=splits, max_kv_len=1500)
        torch.cuda.synchronize()
        return o, l
    base_o, base_l = run(q, SIGMA, cache.kv_scale)
    for c in (2.0, 0.25):
        o, l = run(scaled_bf16_bits(q, c), SIGMA / c, cache.kv_scale)
        assert torch.equal(o, base_o) and torch.equal(l, base_l)
    if kv_dtype == "fp8":
        for c in (4.0, 0.5):
            o, l = run(q, SIGMA / c, cache.kv_scale * c)
            assert torch.equal(o, base_o * c) and torch.equal(l, base_l)
    ref_o, ref_l = run_oracle(q, cache)
    check_out(base_o, ref_o)
    check_lse(base_l, ref_l)


def test_paging_layout_is_bitwise_invariant(mla):
    lens = [700, 1200]
    q, paged = small_case(2008, lens, 12, 2, "fp8", block_size=64)
    contig = mi.paged_cache(2008, lens, 1216, "fp8", stream=77)
    contig.kv_scale = paged.kv_scale
    for b, L in enumerate(lens):
        for t in range(L):
            contig.kv[contig.block_table[b, 0], t] = paged.kv[paged.block_table[b, t // 64], t % 64]
    a, la = run_gpu(mla, q, paged, num_splits=4)
    c, lc = run_gpu(mla, q, contig, num_splits=4)
    assert torch.equal(a, c) and torch.equal(la, lc)


def test_workspace_is_left_zero_and_serves_many_calls(mla):
    """The workspace's completion counters start at zero and every call leaves them zero,
    so one zero-filled workspace serves calls of different shapes in a row."""
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    cases = [(2010, [5, 333, 2047], 12, 2, "fp8", 7), (2011, [4000, 1, 900], 16, 4, "bf16", 0),
             (2012, [64] * 9, 8, 1, "fp8", 5), (2013, [5, 333, 2047], 12, 2, "fp8", 7)]
    for seed, lens, H, P, kvd, splits in cases:
        q, cache = small_case(seed, lens, H, P, kvd)
        kv, bt, sl = cache_to_device(cache, DEV)
        B = len(lens)
        need = mla.decode_workspace_size(B, P, H, max(lens), splits)
        assert 0 < need <= ws.numel()
        out, lse = mla.verify(bf16_tensor(q, DEV), kv, bt, sl, softmax_scale=SIGMA,
                              kv_scale=cache.kv_scale, num_splits=splits, max_kv_len=max(lens),
                              workspace=ws)
        torch.cuda.synchronize()
        ref_o, ref_l = run_oracle(q, cache)
        check_out(out, ref_o)
        check_lse(lse, ref_l)
        assert torch.all(ws[:65536 * 4].view(torch.int32) == 0)


def test_workspace_too_small_is_rejected(mla):
    q, cache = small_case(2009, [5000], 12, 1, "bf16")
    kv, bt, sl = cache_to_device(cache, DEV)
    need = mla.decode_workspace_size(1, 1, 12, 5000, 0)
    assert need > 0
    ws = torch.empty(need - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(mla.MlaError) as e:
        mla.verify(bf16_tensor(q, DEV), kv, bt, sl, softmax_scale=SIGMA, max_kv_len=5000,
                   workspace=ws)
    assert e.value.status == -3


# ---------------------------------------------------------------------------
# full-size workloads, automatic piece plan (the bench's launch configuration)
# ---------------------------------------------------------------------------

def full_case(name):
    w = mi.WORKLOADS[name]
    d = mi.decode_inputs(w)
    return w, d["q"], d["cache"]


def test_full_decode_b1_h12_l1024_bf16(mla):
    w, q, cache = full_case("decode_b1_h12_l1024_bf16")
    print("full", w.name, flush=True)
    out, lse = run_gpu(mla, q, cache, max_kv_len=1024)
    ref_o, ref_l = run_oracle(q, cache)
    check_out(out, ref_o)
    check_lse(lse, ref_l)


def test_full_decode_b32_h12_fp8_paged(mla):
    w, q, cache = full_case("decode_b32_h12_fp8_paged")
    print("full", w.name, flush=True)
    out, lse = run_gpu(mla, q, cache, max_kv_len=16384)
    ref_o, ref_l = run_oracle(q, cache)
    check_out(out, ref_o)
    check_lse(lse, ref_l)


@pytest.mark.parametrize("name", ["verify_b4_p4_h12_l32768_bf16", "verify_b4_p4_h8_l32768_bf16",
                                  "verify_b4_p4_h16_l32768_bf16",
                                  "verify_b4_p4_h12pad16_l32768_bf16"])
def test_full_verify(mla, name):
    w, q, cache = full_case(name)
    print("full", name, flush=True)
    out, lse = run_gpu(mla, q, cache, max_kv_len=32768)
    B, P, H = q.shape[:3]
    ref_o, ref_l = run_oracle(q, cache)  # every row
    check_out(out, ref_o)
    check_lse(lse, ref_l)
    if w.pad_heads_to:
        q12 = np.ascontiguousarray(q[:, :, :w.heads])
        S = mla.decode_num_splits(B, P, H, 32768)
        o12, l12 = run_gpu(mla, q12, cache, num_splits=S)
        assert torch.equal(out[:, :, :w.heads], o12) and torch.equal(lse[:, :, :w.heads], l12)


def test_full_verify_heads_repeated_8_to_16(mla):
    """The 8-head verify workload with each head repeated (8 -> 16 heads), at the piece
    count the automatic plan gives 16 heads: both copies bitwise equal to the 8-head call
    at that piece count, and the 8-head result matches the oracle on every row."""
    w, q8, cache = full_case("verify_b4_p4_h8_l32768_bf16")
    print("full repetition", w.name, flush=True)
    B, P, H = q8.shape[:3]
    S = mla.decode_num_splits(B, P, 2 * H, 32768)
    o16, l16 = run_gpu(mla, np.repeat(q8, 2, axis=2), cache, num_splits=S, max_kv_len=32768)
    o8, l8 = run_gpu(mla, q8, cache, num_splits=S, max_kv_len=32768)
    for c in range(2):
        assert torch.equal(o16[:, :, c::2], o8) and torch.equal(l16[:, :, c::2], l8)
    ref_o, ref_l = run_oracle(q8, cache)
    check_out(o8, ref_o)
    check_lse(l8, ref_l)


def test_full_verify_b1_p4_h12_l32768_fp8(mla):
    """The pages' short verify shape (one sequence, 4 positions, 12 heads, 32K context):
    more pieces than 16 per sequence, so the shares are merged by the separate launch;
    also run with the in-launch merge (16 pieces) and compare both to the oracle."""
    w, q, cache = full_case("verify_b1_p4_h12_l32768_fp8")
    print("full", w.name, flush=True)
    B, P, H = q.shape[:3]
    assert mla.decode_num_splits(B, P, H, 32768) > 16
    ref_o, ref_l = run_oracle(q, cache)  # every row
    for splits in [0, 16]:
        out, lse = run_gpu(mla, q, cache, max_kv_len=32768, num_splits=splits)
        check_out(out, ref_o)
        check_lse(lse, ref_l)


def test_full_decode_b8_h12_l142000_fp8_8parts(mla):
    """8 contiguous key partitions (one per call, as a position shard would compute its
    share), merged by mla_merge_lse, against the unsplit call and the oracle."""
    w, q, cache = full_case("decode_b8_h12_l142000_fp8_8parts")
    print("full", w.name, flush=True)
    B, H = w.batch, w.heads
    bounds = mi.partition_bounds(142000, w.partitions)
    parts_o, parts_l = [], []
    for lo, hi in bounds:
        o, l = run_gpu(mla, q, cache, kv_begin=np.full(B, lo, np.int32),
                       kv_end=np.full(B, hi, np.int32), max_kv_len=hi - lo)
        parts_o.append(o.reshape(-1, 512))
        parts_l.append(l.reshape(-1))
    mo, ml = mla.merge_lse(torch.stack(parts_o), torch.stack(parts_l))
    whole_o, whole_l = run_gpu(mla, q, cache, max_kv_len=142000)
    torch.cuda.synchronize()
    assert (mo - whole_o.reshape(-1, 512)).abs().max().item() < 2e-3
    assert (ml - whole_l.reshape(-1)).abs().max().item() < 2e-5
    rows = np.arange(B * H, dtype=np.int64)  # every row
    ref_o, ref_l = run_oracle(q, cache, rows=rows)
    idx = torch.from_numpy(rows).to(DEV)
    check_out(mo[idx], ref_o, "merged out")
    check_lse(ml[idx], ref_l, "merged lse")
    check_out(whole_o.reshape(-1, 512)[idx], ref_o, "unsplit out")
    check_lse(whole_l.reshape(-1)[idx], ref_l, "unsplit lse")
    # each partition against the oracle on its own range
    lo, hi = bounds[3]
    po, pl = run_oracle(q, cache, np.full(B, lo, np.int32), np.full(B, hi, np.int32), rows=rows)
    check_out(parts_o[3][idx], po, "partition 3 out")
    check_lse(parts_l[3][idx], pl, "partition 3 lse")

    # All partitions in one call, as the bench times them: the S x B (partition,
    # sequence) ranges are S * B sequences of one batch (query and block-table row
    # repeated, range from kv_begin / kv_end).  Each range's result matches its own
    # call's; the merge matches the oracle.
    S = len(bounds)
    qb = np.tile(q, (S, 1, 1, 1))
    bc = mi.PagedCache(kv=cache.kv, kv_dtype=cache.kv_dtype, kv_scale=cache.kv_scale,
                       block_table=np.tile(cache.block_table, (S, 1)),
                       seq_lens=np.tile(cache.seq_lens, S), block_size=cache.block_size)
    kb = np.repeat([lo for lo, _ in bounds], B).astype(np.int32)
    ke = np.repeat([hi for _, hi in bounds], B).astype(np.int32)
    span = max(hi - lo for lo, hi in bounds)
    bo, bl = run_gpu(mla, qb, bc, kv_begin=kb, kv_end=ke, max_kv_len=span)
    bo = bo.reshape(S, B * H, 512)
    bl = bl.reshape(S, B * H)
    for j in range(S):
        assert (bo[j] - parts_o[j]).abs().max().item() < 2e-3
        assert (bl[j] - parts_l[j]).abs().max().item() < 2e-5
    bmo, bml = mla.merge_lse(bo, bl)
    torch.cuda.synchronize()
    check_out(bmo[idx], ref_o, "batched merged out")
    check_lse(bml[idx], ref_l, "batched merged lse")
