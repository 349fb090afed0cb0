"""Pins for the oracle's top-k renormalisation of probability rows (CPU only).

What pins it, other than itself:
  * a library formulation: torch's stable descending sort picks the kept entries
    (stable, so equal values keep index order), the kept values are divided by
    their sum with numpy; the kept sets must be identical and the values agree
    to 1e-12;
  * closed forms: k = 1 is the one-hot row at the first maximum; k <= 0 and
    k >= vocab are the row divided by its sum; an all-equal row keeps its first
    k entries at 1/k each; hand-worked rows with ties at the k-th value;
  * invariants: every row sums to one, exactly k entries are non-zero (positive
    rows), every kept entry is >= every dropped one, and scaling a row by a
    power of two changes nothing;
  * edge cases: a zero row gives zeros, NaN is rejected, vocab 1.
"""
import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle


def torch_reference(p, k):
    """Kept mask and renormalised float64 row from torch.sort(stable, descending)."""
    V = p.shape[0]
    keff = V if (k <= 0 or k >= V) else k
    order = torch.sort(torch.from_numpy(p), descending=True, stable=True).indices.numpy()
    kept = np.zeros(V, bool)
    kept[order[:keff]] = True
    s = p[kept].astype(np.float64).sum()
    out = np.where(kept, p.astype(np.float64) / s, 0.0) if s != 0 else np.zeros(V)
    return kept, out


def tied_rows(seed, rows, vocab, levels):
    """Positive rows whose values come from a few levels, so the k-th value is tied."""
    rng = np.random.default_rng(seed)
    lv = rng.uniform(0.1, 1.0, levels).astype(np.float32)
    return lv[rng.integers(0, levels, size=(rows, vocab))]


@pytest.mark.parametrize("vocab,levels", [(1000, None), (4099, None), (777, 3), (5000, 40)])
def test_matches_stable_sort_formulation(vocab, levels):
    rows = 12
    p = (mi.probability_rows(31, rows, vocab) if levels is None
         else tied_rows(37, rows, vocab, levels))
    ks = [1, 2, 5, 50, vocab // 3, vocab - 1, vocab, vocab + 3, 0, -1, 17, 100]
    out = oracle.top_k_renorm_prob(p, np.array(ks, np.int32))
    for r, k in enumerate(ks):
        kept, ref = torch_reference(p[r], k)
        assert np.array_equal(out[r] != 0, kept), (vocab, levels, k)
        assert np.max(np.abs(out[r] - ref)) < 1e-12


def test_closed_forms():
    p = mi.probability_rows(41, 3, 2000)
    # k = 1: one-hot at the first maximum
    p[1, 7] = p[1, 1500] = p[1].max() * 2  # a tied maximum: the lower index wins
    o1 = oracle.top_k_renorm_prob(p, 1)
    for r in range(3):
        want = np.zeros(2000)
        want[int(np.argmax(p[r]))] = 1.0
        assert np.array_equal(o1[r], want)
    assert o1[1, 7] == 1.0
    # keep-all values of k: the row over its sum
    for k in [0, -5, 2000, 10 ** 6]:
        ok = oracle.top_k_renorm_prob(p, k)
        want = p.astype(np.float64) / p.astype(np.float64).sum(axis=1, keepdims=True)
        assert np.max(np.abs(ok - want)) < 1e-15
    # an all-equal row keeps its first k entries at 1/k
    flat = np.full((1, 300), 0.25, np.float32)
    o = oracle.top_k_renorm_prob(flat, 7)
    assert np.array_equal(o[0, :7], np.full(7, 1 / 7)) and not o[0, 7:].any()


def test_hand_worked_ties():
    x = np.array([[0.1, 0.3, 0.2, 0.3, 0.1]], np.float32)
    v = x.astype(np.float64)[0]
    cases = {
        1: {1: 1.0},                                       # tied maximum: index 1 before 3
        2: {1: 0.5, 3: 0.5},
        3: {1: v[1] / (v[1] + v[2] + v[3]), 2: v[2] / (v[1] + v[2] + v[3]),
            3: v[3] / (v[1] + v[2] + v[3])},
        4: {i: v[i] / (v[:4].sum()) for i in range(4)},    # the 0.1 at index 0, not 4
    }
    for k, kept in cases.items():
        o = oracle.top_k_renorm_prob(x, k)[0]
        want = np.zeros(5)
        for i, val in kept.items():
            want[i] = val
        assert np.max(np.abs(o - want)) < 1e-15, (k, o)


def test_invariants():
    p = mi.probability_rows(43, 8, 3001)
    ks = np.array([1, 3, 10, 64, 500, 1500, 3000, 3001], np.int32)
    o = oracle.top_k_renorm_prob(p, ks)
    for r, k in enumerate(ks):
        kept = o[r] != 0
        assert kept.sum() == min(k, 3001)
        assert abs(o[r].sum() - 1.0) < 1e-12
        if kept.sum() < 3001:
            assert p[r][kept].min() >= p[r][~kept].max()
        # proportional to the input on the kept set
        ratio = o[r][kept] / p[r][kept].astype(np.float64)
        assert np.max(np.abs(ratio / ratio[0] - 1)) < 1e-12
    # a power-of-two scale is exact in fp32 and changes nothing
    o2 = oracle.top_k_renorm_prob(p * np.float32(8.0), ks)
    assert np.max(np.abs(o2 - o)) < 1e-15


def test_edge_cases():
    z = np.zeros((2, 50), np.float32)
    assert not oracle.top_k_renorm_prob(z, 5).any()
    one = np.array([[0.3]], np.float32)
    assert oracle.top_k_renorm_prob(one, 1)[0, 0] == 1.0
    assert oracle.top_k_renorm_prob(one, 0)[0, 0] == 1.0
    bad = np.full((1, 10), 0.1, np.float32)
    bad[0, 3] = np.nan
    with pytest.raises(ValueError):
        oracle.top_k_renorm_prob(bad, 2)
    # zeros rank below every positive value, and -0 below +0
    x = np.array([[0.0, -0.0, 0.5, 0.0]], np.float32)
    o = oracle.top_k_renorm_prob(x, 2)[0]
    assert np.array_equal(o, [0.0, 0.0, 1.0, 0.0])
