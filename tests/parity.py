"""Helpers shared by the GPU parity tests: move seeded inputs to the device, compare with
the oracle to the stated bar.

Bar (floating point, unit-scale inputs): per element |gpu - oracle| <= max(1e-2, one ulp
of the output dtype at |oracle|) -- the ulp term only matters for BF16 outputs with
|out| >= 2, where rounding the exact value already costs up to half an ulp --,
mean |gpu - oracle| <= 1e-3, and |lse_gpu - lse_oracle| <= 1e-4 with -inf exactly where
the oracle has -inf.
"""
from __future__ import annotations

import numpy as np
import torch

import mla_inputs as mi

MAX_ABS = 1e-2
MEAN_ABS = 1e-3
LSE_ABS = 1e-4


def bf16_tensor(bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def cache_to_device(cache: mi.PagedCache, dev):
    if cache.kv_dtype == "bf16":
        kv = bf16_tensor(cache.kv, dev)
    else:
        kv = torch.from_numpy(np.ascontiguousarray(cache.kv)).to(dev)
    bt = torch.from_numpy(np.ascontiguousarray(cache.block_table, dtype=np.int32)).to(dev)
    sl = torch.from_numpy(np.ascontiguousarray(cache.seq_lens, dtype=np.int32)).to(dev)
    return kv, bt, sl


def i32(a, dev):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    _, e = np.frexp(np.abs(x))
    return np.ldexp(1.0, e - 8)


def check_out(gpu: torch.Tensor, ref: np.ndarray, what: str = "out"):
    g = to_f64(gpu).reshape(ref.shape)
    err = np.abs(g - ref)
    tol = np.full(ref.shape, MAX_ABS)
    if gpu.dtype == torch.bfloat16:
        tol = np.maximum(tol, bf16_ulp(ref))
    bad = ~(err <= tol)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d elements over the bound; worst %.3g at %s (gpu %r, oracle %r)"
                             % (what, int(bad.sum()), float(np.nanmax(err)), idx.tolist(),
                                [g[tuple(i)] for i in idx], [ref[tuple(i)] for i in idx]))
    assert err.mean() <= MEAN_ABS, "%s: mean abs error %.3g" % (what, err.mean())
    return float(err.max()), float(err.mean())


def check_lse(gpu: torch.Tensor, ref: np.ndarray, what: str = "lse"):
    g = to_f64(gpu).reshape(ref.shape)
    assert np.array_equal(np.isneginf(g), np.isneginf(ref)), "%s: -inf pattern differs" % what
    fin = np.isfinite(ref)
    assert np.all(np.isfinite(g[fin])), "%s: non-finite values" % what
    d = np.abs(g[fin] - ref[fin])
    assert d.size == 0 or d.max() <= LSE_ABS, "%s: max abs diff %.3g" % (what, d.max())
    return float(d.max()) if d.size else 0.0
