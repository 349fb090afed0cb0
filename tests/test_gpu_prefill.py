"""GPU parity of causal prefill against the FP64 oracle, through the C-ABI.

Small packed batches (every row checked) cover ragged sequence lengths around the
32-token key tile and the 128-row work-group block, an empty sequence, 1 / 5 / 8 / 12 /
16 heads, BF16 and FP8 latent rows, FP32 and BF16 outputs.  The full-size workload
(one 32,768-token sequence, 12 heads, BF16 output) runs in the bench's launch
configuration, over a BF16 and an FP8 cache, and is checked on one token of every
128-row work-group block.  Invariants: prefill row i equals
decode on the prefix of length i + 1, future keys do not matter, runs are bitwise
repeatable, power-of-two scalings of q, the softmax scale and the FP8 scale move the
results exactly, and repeated heads, zero-padded heads and reordered sequences leave every
row unchanged (all bitwise).
"""
import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle
from parity import bf16_tensor, check_lse, check_out, i32

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SIGMA = mi.softmax_scale_for()


@pytest.fixture(scope="module")
def mla():
    import mla_latent_kv_attention_amd as m
    m.library()
    assert torch.cuda.is_available()
    return m


def kv_tensor(kv, kv_dtype):
    if kv_dtype == "bf16":
        return bf16_tensor(kv, DEV)
    return torch.from_numpy(np.ascontiguousarray(kv)).to(DEV)


def run_gpu(mla, d, kv_dtype, out_dtype=torch.float32, max_seqlen=None):
    out, lse = mla.prefill(bf16_tensor(d["q"], DEV), kv_tensor(d["kv"], kv_dtype),
                           i32(d["cu_seqlens"], DEV), softmax_scale=SIGMA,
                           kv_scale=d["kv_scale"], out_dtype=out_dtype, max_seqlen=max_seqlen)
    torch.cuda.synchronize()
    return out, lse


def run_oracle(d, kv_dtype, tokens=None):
    return oracle.prefill(d["q"], d["kv"], kv_dtype == "fp8", d["kv_scale"], d["cu_seqlens"],
                          SIGMA, tokens=tokens)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("H", [12, 8, 16, 1, 5])
def test_small_parity(mla, kv_dtype, H):
    lens = [1, 31, 32, 33, 0, 100, 257]
    d = mi.prefill_inputs(mi.PrefillWorkload("small", lens, H, kv_dtype, seed=3000 + H))
    print("case", kv_dtype, H, flush=True)
    out, lse = run_gpu(mla, d, kv_dtype)
    ref_o, ref_l = run_oracle(d, kv_dtype)
    check_out(out, ref_o)
    check_lse(lse, ref_l)


def test_bf16_output_and_single_key_rows(mla):
    lens = [300, 77]
    d = mi.prefill_inputs(mi.PrefillWorkload("small", lens, 12, "bf16", seed=3101))
    out, lse = run_gpu(mla, d, "bf16", out_dtype=torch.bfloat16)
    ref_o, ref_l = run_oracle(d, "bf16")
    check_out(out, ref_o)
    check_lse(lse, ref_l)
    # the first token of each sequence sees one key: its output is that row's value part
    for start in d["cu_seqlens"][:-1]:
        v = torch.from_numpy(d["kv"][start, :512].view(np.int16)).view(torch.bfloat16)
        assert torch.equal(out[start].cpu(), v.expand(12, 512))


def test_prefill_row_equals_decode_on_prefix(mla):
    T, H = 512, 12  # one contiguous 512-token block for the decode side
    d = mi.prefill_inputs(mi.PrefillWorkload("small", [T], H, "bf16", seed=3102))
    out, lse = run_gpu(mla, d, "bf16")
    kv = bf16_tensor(d["kv"], DEV).reshape(1, T, 576)
    toks = [0, 1, 63, 64, 127, 255, 511]
    ref_o, ref_l = run_oracle(d, "bf16", tokens=np.array(toks, np.int64))
    for k, i in enumerate(toks):
        q = bf16_tensor(d["q"][i], DEV).reshape(1, H, 576)
        o, l = mla.decode(q, kv, torch.zeros((1, 1), dtype=torch.int32, device=DEV),
                          torch.tensor([i + 1], dtype=torch.int32, device=DEV),
                          softmax_scale=SIGMA, max_kv_len=i + 1)
        torch.cuda.synchronize()
        # Both paths meet the parity bar but are not bitwise equal: each rounds its
        # weights P = exp(s - m_ref) to bf16 against its own reference maximum m_ref
        # (decode: a row's first visible score maximum; prefill: the row's maximum over
        # the first key tile), so the rounded weights differ; the pages leave the
        # precision of P open.  Each is within the bar of the oracle, so they are within
        # twice the bar of each other; the test asks for the bar itself.
        check_out(o[0], ref_o[k], "decode on prefix %d" % i)
        check_out(out[i], ref_o[k], "prefill row %d" % i)
        check_lse(l[0], ref_l[k])
        check_lse(lse[i], ref_l[k])
        assert (o[0] - out[i]).abs().max().item() <= 1e-2


def scaled_bf16_bits(bits: np.ndarray, c: float) -> np.ndarray:
    """BF16 bit patterns multiplied by a power of two c (exact for these magnitudes)."""
    f = (bits.astype(np.uint32) << 16).view(np.float32) * np.float32(c)
    out = mi.to_bf16_bits(f)
    assert np.array_equal((out.astype(np.uint32) << 16).view(np.float32), f)
    return out


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_power_of_two_scale_invariants(mla, kv_dtype):
    """The scores depend on q and the softmax scale only through their product, and an
    FP8 cache's values through code x kv_scale: (q * c, scale / c) gives bitwise the same
    out and lse for a power of two c, and (kv_scale * c, scale / c) gives out * c and the
    same lse."""
    d = mi.prefill_inputs(mi.PrefillWorkload("scale", [300, 45, 129], 12, kv_dtype, seed=3210))
    q, kv, cu = d["q"], kv_tensor(d["kv"], kv_dtype), i32(d["cu_seqlens"], DEV)

    def run(q_bits, scale, kv_scale):
        o, l = mla.prefill(bf16_tensor(q_bits, DEV), kv, cu, softmax_scale=scale,
                           kv_scale=kv_scale, out_dtype=torch.float32, max_seqlen=300)
        torch.cuda.synchronize()
        return o, l
    base_o, base_l = run(q, SIGMA, d["kv_scale"])
    for c in (2.0, 0.25):
        print("case q x", c, kv_dtype, flush=True)
        o, l = run(scaled_bf16_bits(q, c), SIGMA / c, d["kv_scale"])
        assert torch.equal(o, base_o) and torch.equal(l, base_l)
    if kv_dtype == "fp8":
        for c in (4.0, 0.5):
            print("case kv_scale x", c, flush=True)
            o, l = run(q, SIGMA / c, d["kv_scale"] * c)
            assert torch.equal(o, base_o * c) and torch.equal(l, base_l)
    ref_o, ref_l = run_oracle(d, kv_dtype)
    check_out(base_o, ref_o)
    check_lse(base_l, ref_l)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_heads_repeated_padded_and_sequences_reordered_are_bitwise_invariant(mla, kv_dtype):
    """Each (token, head) row is computed on its own whatever rows share its
    work-group, and key tiles start at the sequence's first token: 8 heads repeated
    into 16 (both copies of every head), 12 heads zero-padded to 16 (K2.5 blog, section
    "PR #35850 修复了什么": head counts per rank of 8, 12 and 16), and the packed
    sequences in another order all give the same rows, bitwise."""
    lens = [130, 1, 77, 256]
    T = sum(lens)

    def run(q_bits, kv_rows, cu, H, kv_scale):
        o, l = mla.prefill(bf16_tensor(q_bits, DEV), kv_tensor(kv_rows, kv_dtype), i32(cu, DEV),
                           softmax_scale=SIGMA, kv_scale=kv_scale, out_dtype=torch.float32,
                           max_seqlen=max(lens))
        torch.cuda.synchronize()
        assert o.shape == (T, H, 512)
        return o, l
    d = mi.prefill_inputs(mi.PrefillWorkload("inv", lens, 8, kv_dtype, seed=3220))
    base_o, base_l = run(d["q"], d["kv"], d["cu_seqlens"], 8, d["kv_scale"])
    print("case repeated heads", kv_dtype, flush=True)
    q16 = np.repeat(d["q"], 2, axis=1)  # heads h, h, h + 1, h + 1, ...
    o16, l16 = run(q16, d["kv"], d["cu_seqlens"], 16, d["kv_scale"])
    for c in range(2):
        assert torch.equal(o16[:, c::2], base_o) and torch.equal(l16[:, c::2], base_l)
    print("case reordered sequences", kv_dtype, flush=True)
    order = [3, 0, 2, 1]
    starts = np.asarray(d["cu_seqlens"][:-1])
    tok = np.concatenate([np.arange(starts[b], starts[b] + lens[b]) for b in order])
    cu_r = np.zeros(len(lens) + 1, np.int32)
    cu_r[1:] = np.cumsum([lens[b] for b in order])
    o_r, l_r = run(np.ascontiguousarray(d["q"][tok]), np.ascontiguousarray(d["kv"][tok]), cu_r,
                   8, d["kv_scale"])
    inv = torch.from_numpy(np.argsort(tok)).to(DEV)
    assert torch.equal(o_r[inv], base_o) and torch.equal(l_r[inv], base_l)
    print("case zero-padded heads", kv_dtype, flush=True)
    d12 = mi.prefill_inputs(mi.PrefillWorkload("inv12", lens, 12, kv_dtype, seed=3221))
    o12, l12 = run(d12["q"], d12["kv"], d12["cu_seqlens"], 12, d12["kv_scale"])
    qpad = np.zeros((T, 16, 576), d12["q"].dtype)
    qpad[:, :12] = d12["q"]
    op, lp = run(qpad, d12["kv"], d12["cu_seqlens"], 16, d12["kv_scale"])
    assert torch.equal(op[:, :12], o12) and torch.equal(lp[:, :12], l12)
    ref_o, ref_l = run_oracle(d, kv_dtype)
    check_out(base_o, ref_o)
    check_lse(base_l, ref_l)


def test_future_keys_do_not_matter_and_runs_repeat(mla):
    T, H = 400, 12
    d = mi.prefill_inputs(mi.PrefillWorkload("small", [T], H, "bf16", seed=3103))
    a, la = run_gpu(mla, d, "bf16")
    a2, la2 = run_gpu(mla, d, "bf16")
    assert torch.equal(a, a2) and torch.equal(la, la2)
    d2 = dict(d)
    d2["kv"] = d["kv"].copy()
    d2["kv"][150:] ^= 0x1234
    b, lb = run_gpu(mla, d2, "bf16")
    assert torch.equal(a[:150], b[:150]) and torch.equal(la[:150], lb[:150])


@pytest.mark.parametrize("gain", [0.9, 2.0])
def test_late_score_jump(mla, gain):
    """A key planted at token 300 parallel to the query of token 350, head 4: its score is
    ~54 (gain 0.9) or ~120 (gain 2) log2 units above the first tile's maximum of that row,
    below and above the kernel's cap of 64.  Above the cap the work-group runs its key loop
    again; rows that stayed under their cap (every row before token 300 in particular) must
    come out bit-identical to a run without the planted key, and every row must match the
    oracle."""
    T, H = 400, 12
    d = mi.prefill_inputs(mi.PrefillWorkload("small", [T], H, "bf16", seed=3105))
    base, lbase = run_gpu(mla, d, "bf16")
    d2 = dict(d)
    d2["kv"] = d["kv"].copy()
    qf = (d["q"][350, 4].astype(np.uint32) << 16).view(np.float32)
    d2["kv"][300] = mi.to_bf16_bits(gain * qf)
    out, lse = run_gpu(mla, d2, "bf16")
    ref_o, ref_l = run_oracle(d2, "bf16")
    check_out(out, ref_o)
    check_lse(lse, ref_l)
    assert torch.equal(out[:300], base[:300]) and torch.equal(lse[:300], lbase[:300])


def test_max_seqlen_hint_does_not_limit_the_work(mla):
    d = mi.prefill_inputs(mi.PrefillWorkload("small", [200, 90], 12, "fp8", seed=3104))
    out, lse = run_gpu(mla, d, "fp8", max_seqlen=8)
    ref_o, ref_l = run_oracle(d, "fp8")
    check_out(out, ref_o)
    check_lse(lse, ref_l)


# ---------------------------------------------------------------------------
# full size: one 32,768-token sequence, 12 heads, in the bench's launch configuration.
# A work-group holds 128 query rows (token x head, rows of a sequence in order), so the
# 32,768 x 12 rows are 3,072 work-group blocks.  One token inside every block is checked
# (all 12 heads), split over four tests by block number mod 4 so that each test's
# oracle work (about a quarter of 1.3e12 FP64 flops) stays well inside a test time limit.
# ---------------------------------------------------------------------------

FULL_BLOCKS = 32768 * 12 // 128


def block_tokens(residue):
    """The middle token of every 128-row block k with k % 4 == residue, plus the edges."""
    toks = [(128 * k + 64) // 12 for k in range(residue, FULL_BLOCKS, 4)]
    edges = [0, 1, 31, 32, 127, 32767] if residue == 0 else []
    return np.unique(np.array(toks + edges, np.int64))


@pytest.fixture(scope="module", params=["bf16", "fp8"])
def full_prefill(request, mla):
    kvd = request.param
    w = (mi.WORKLOADS["prefill_t32768_h12_bf16"] if kvd == "bf16" else
         mi.PrefillWorkload("prefill_t32768_h12_fp8", [32768], 12, "fp8", seed=404))
    d = mi.prefill_inputs(w)
    print("full", w.name, flush=True)
    out, lse = run_gpu(mla, d, kvd, out_dtype=torch.bfloat16, max_seqlen=32768)
    return kvd, d, out, lse


@pytest.mark.slow
@pytest.mark.parametrize("residue", [0, 1, 2, 3])
def test_full_prefill_t32768_h12(full_prefill, residue):
    kvd, d, out, lse = full_prefill
    toks = block_tokens(residue)
    print("oracle on %d tokens (%s, blocks = %d mod 4)" % (len(toks), kvd, residue), flush=True)
    ref_o, ref_l = run_oracle(d, kvd, tokens=toks)
    idx = torch.from_numpy(toks).to(DEV)
    check_out(out[idx], ref_o)
    check_lse(lse[idx], ref_l)
