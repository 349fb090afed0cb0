"""Pins for the oracle's latent-row cache write (quantise and scatter), CPU only.

The FP8 encoder is the nearest-finite-code definition; it is pinned against the
decoder (every code round-trips), against the midpoints between neighbouring
codes (ties to the even mantissa, one ulp either side to the nearer code),
against saturation and NaN, and against torch's float8_e4m3fn cast (a library
routine with round-to-nearest-even) on values inside the finite range.  The
scatter is pinned against an independent numpy/torch formulation of the same
write.
"""
import math

import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle

FINITE = [c for c in range(256) if (c & 0x7F) != 0x7F]


def value(c):
    return oracle.fp8_e4m3fn_value(c)


def test_every_finite_code_round_trips():
    for c in FINITE:
        assert oracle.fp8_e4m3fn_encode(value(c)) == c, hex(c)


def test_midpoints_tie_to_even_and_neighbours_round_to_nearest():
    pos = sorted(c for c in FINITE if c < 0x80)
    for a, b in zip(pos[:-1], pos[1:]):
        va, vb = value(a), value(b)
        mid = np.float32((va + vb) / 2)  # at most 5 significant bits: exact in fp32
        assert float(mid) == (va + vb) / 2
        even = a if (a & 1) == 0 else b
        assert oracle.fp8_e4m3fn_encode(float(mid)) == even, (hex(a), hex(b))
        assert oracle.fp8_e4m3fn_encode(float(np.nextafter(mid, np.float32(-1)))) == a
        assert oracle.fp8_e4m3fn_encode(float(np.nextafter(mid, np.float32(1e30)))) == b
        # the same on the negative side
        assert oracle.fp8_e4m3fn_encode(-float(mid)) == (even | 0x80)


def test_saturation_nan_and_signed_zero():
    for y in [448.0, 448.0001, 464.0, 480.0, 1e30, math.inf]:
        assert oracle.fp8_e4m3fn_encode(y) == 0x7E
        assert oracle.fp8_e4m3fn_encode(-y) == 0xFE
    assert oracle.fp8_e4m3fn_encode(math.nan) == 0x7F
    assert oracle.fp8_e4m3fn_encode(0.0) == 0x00
    assert oracle.fp8_e4m3fn_encode(-0.0) == 0x80
    # below half the smallest subnormal (2^-10) rounds to zero; exactly half ties to 0
    assert oracle.fp8_e4m3fn_encode(2.0 ** -10) == 0x00
    assert oracle.fp8_e4m3fn_encode(float(np.nextafter(np.float32(2.0 ** -10), 1))) == 0x01


def test_matches_torch_float8_cast_inside_the_finite_range():
    rng = np.random.default_rng(5)
    y = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 50,
        rng.uniform(-448, 448, 20000).astype(np.float32),
        (rng.standard_normal(5000) * 2.0 ** -8).astype(np.float32),  # subnormal range
    ])
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.fp8_e4m3fn_encode(float(v)) for v in y], np.uint8)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("kv_dtype", ["fp8", "bf16"])
def test_cache_write_scatter(kv_dtype):
    rng = np.random.default_rng(11)
    num_blocks, bs, N = 6, 16, 40
    num_slots = num_blocks * bs
    if kv_dtype == "fp8":
        kv = rng.integers(0, 0x7E, size=(num_blocks, bs, 576), dtype=np.uint8)
    else:
        kv = mi.normal_bf16_bits(11, 9, (num_blocks, bs, 576))
    latent = mi.normal_bf16_bits(11, 10, (N, 576))
    # a large value and an infinity saturate, and a NaN is carried through
    latent[3, 0] = mi.to_bf16_bits(np.array([300.0], np.float32))[0]
    latent[3, 1] = 0x7F80  # +inf
    latent[3, 2] = 0x7FC0  # NaN
    slot = rng.permutation(num_slots)[:N].astype(np.int32)
    slot[5] = -1            # padding: skipped
    slot[7] = num_slots     # out of range: skipped
    scale = 0.0123
    out = oracle.cache_write(latent, slot, kv, kv_dtype == "fp8", scale)

    # independent formulation: fp32 division, clamp, torch's RNE cast; NaN -> 0x7F
    want = kv.reshape(num_slots, 576).copy()
    x = torch.from_numpy(latent.view(np.int16)).view(torch.bfloat16).float()
    for n in range(N):
        s = slot[n]
        if s < 0 or s >= num_slots:
            continue
        if kv_dtype == "fp8":
            y = x[n] / torch.tensor(scale, dtype=torch.float32)
            nan = torch.isnan(y)
            y = torch.clamp(torch.nan_to_num(y, posinf=448.0, neginf=-448.0), -448, 448)
            codes = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
            codes[nan.numpy()] = 0x7F
            want[s] = codes
        else:
            want[s] = latent[n]
    assert np.array_equal(out.reshape(num_slots, 576), want)
    # untouched slots are untouched
    written = set(int(v) for v in slot if 0 <= v < num_slots)
    for s in range(num_slots):
        if s not in written:
            assert np.array_equal(out.reshape(num_slots, 576)[s], kv.reshape(num_slots, 576)[s])
