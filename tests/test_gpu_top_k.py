"""GPU parity of mla_top_k_renorm_prob against the oracle, through the C-ABI.

The kept set is an integer decision taken on exact fp32 comparisons on both
sides, so it must match exactly; inputs are positive, so an entry is kept iff its
output is non-zero.  Kept values agree to the bound of the fp32 sum the kernel
takes (each of 1,024 threads adds at most ceil(n / 1,024) terms in order, then a
fixed tree over 1,024 partial sums; non-negative terms): relative error at most
(ceil(n / 1024) + 12) * 2^-24, one more ulp for the division.

Cases span several 8,192-entry chunks and a ragged last chunk, the vectorised
(vocab % 4 == 0) and scalar loads, k around the 2,048 list limit (above it the
second stage reads the row itself), ties at the k-th value inside a chunk and
across chunks, keep-all values of k, zero rows, vocab 1, in-place calls,
run-to-run determinism, and the full 128 x 163,840 workload.
"""
import math

import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle
from test_oracle_top_k import tied_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def mla():
    import mla_latent_kv_attention_amd as m
    m.library()
    assert torch.cuda.is_available()
    return m


def run(mla, p, ks, inplace=False):
    pt = torch.from_numpy(np.ascontiguousarray(p)).to(DEV)
    kt = torch.from_numpy(np.asarray(ks, np.int32)).to(DEV)
    out = mla.top_k_renorm_prob(pt, kt, out=pt if inplace else None)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(got, p, ks):
    want = oracle.top_k_renorm_prob(p, np.asarray(ks, np.int32))
    V = p.shape[1]
    for r, k in enumerate(ks):
        keff = V if (k <= 0 or k >= V) else k
        kept_g, kept_w = got[r] != 0, want[r] != 0
        bad = np.flatnonzero(kept_g != kept_w)
        assert bad.size == 0, "row %d k %d: kept sets differ at %s" % (r, k, bad[:8].tolist())
        tol = (math.ceil(keff / 1024) + 13) * 2.0 ** -24
        rel = np.abs(got[r][kept_w] - want[r][kept_w]) / want[r][kept_w]
        assert rel.size == 0 or rel.max() <= tol, (r, k, float(rel.max()), tol)


KS = [1, 2, 7, 100, 400, 512, 513, 2047, 2048, 2049, 8191, 8192, 8193, 16384, 30000, 0, -3]


@pytest.mark.parametrize("vocab", [3 * 16384 + 1234, 3 * 16384 + 1236, 40000, 100, 16384])
def test_random_rows(mla, vocab):
    ks = [k for k in KS if k < vocab + 5] + [vocab - 1, vocab, vocab + 7]
    p = mi.probability_rows(61, len(ks), vocab)
    check(run(mla, p, ks), p, ks)


@pytest.mark.parametrize("levels", [2, 5, 300])
def test_ties_at_the_threshold(mla, levels):
    vocab = 2 * 16384 + 999 * 4
    ks = [1, 3, 50, 700, 2048, 2049, 5000, 16384, 20000, vocab - 2, vocab]
    p = tied_rows(71 + levels, len(ks), vocab, levels)
    check(run(mla, p, ks), p, ks)


def test_tie_straddles_chunks(mla):
    """The k-th value occurs in every chunk: the lowest-index ties win, across chunks."""
    vocab = 4 * 16384
    p = np.full((4, vocab), 0.5, np.float32)
    rng = np.random.default_rng(5)
    for r in range(4):
        big = rng.choice(vocab, 40, replace=False)
        p[r, big] = 0.9
    ks = [41, 100, 2048, 17000]
    check(run(mla, p, ks), p, ks)


def test_edge_rows(mla):
    z = np.zeros((3, 5000), np.float32)
    assert not run(mla, z, [5, 0, 4999]).any()
    one = np.array([[0.25]], np.float32)
    assert run(mla, one, [1])[0, 0] == 1.0
    assert run(mla, one, [0])[0, 0] == 1.0
    # a row with zeros among the entries: zeros rank below every positive value
    x = np.zeros((1, 9000), np.float32)
    x[0, [17, 4000, 8999]] = [0.5, 0.25, 0.25]
    got = run(mla, x, [2])
    assert got[0, 17] == np.float32(0.5) / np.float32(0.75) and got[0, 4000] == np.float32(0.25) / np.float32(0.75)
    assert np.count_nonzero(got) == 2


def test_in_place_and_deterministic(mla):
    vocab = 3 * 16384 + 4
    ks = [1, 64, 3000, 0]
    p = mi.probability_rows(83, 4, vocab)
    a = run(mla, p, ks)
    b = run(mla, p, ks)
    c = run(mla, p, ks, inplace=True)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))
    check(a, p, ks)


def test_full_workload(mla):
    w = mi.TOP_K_WORKLOADS["top_k_renorm_r128_v163840"]
    p, ks = w.probs(), w.top_k()
    check(run(mla, p, ks), p, ks)
