"""GPU parity of the latent-row cache write against the oracle, through the C-ABI.

Codes and copied rows must be bit-exact: random rows at several magnitudes and
scales, every edge class of the FP8 encoder (signed zeros, subnormals, exact
midpoints between neighbouring codes, saturation, infinities, NaN), padding and
out-of-range slots, BF16 caches; then a write followed by a decode over the
written cache, against the oracle's decode over the oracle-written cache.
"""
import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle
from parity import bf16_tensor, cache_to_device, check_lse, check_out

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def mla():
    import mla_latent_kv_attention_amd as m
    m.library()
    assert torch.cuda.is_available()
    return m


def gpu_write(mla, latent_bits, slot, kv, scale):
    kv_t = torch.from_numpy(np.ascontiguousarray(kv).copy()).to(DEV)
    if kv.dtype == np.uint16:
        kv_t = kv_t.view(torch.bfloat16)
    mla.cache_write(bf16_tensor(latent_bits, DEV), kv_t,
                    torch.from_numpy(slot.astype(np.int32)).to(DEV), kv_scale=scale)
    torch.cuda.synchronize()
    out = kv_t.cpu()
    return (out.view(torch.int16).numpy().view(np.uint16) if kv.dtype == np.uint16
            else out.numpy())


def edge_rows():
    """BF16 rows holding every edge class of the encoder (at scale 1)."""
    finite = [c for c in range(128) if c != 0x7F]
    vals = [oracle.fp8_e4m3fn_value(c) for c in finite]
    mids = [(a + b) / 2 for a, b in zip(vals[:-1], vals[1:])]  # exact in bf16 (<= 5 bits)
    special = [0.0, -0.0, 2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11, 448.0, 449.0, 1000.0, 1e30,
               np.inf, -np.inf, np.nan, -1e-30]
    x = np.array(vals + [-v for v in vals] + mids + [-m for m in mids] + special, np.float32)
    x = np.resize(x, ((x.size + 575) // 576) * 576)
    return mi.to_bf16_bits(x).reshape(-1, 576)


@pytest.mark.parametrize("scale", [1.0, 0.0123, 2.0 ** -4, 3.7e-3])
def test_fp8_codes_are_bit_exact(mla, scale):
    rng = np.random.default_rng(int(scale * 1e6) % 1000)
    rand = np.concatenate([mi.normal_bf16_bits(41, k, (50, 576)) for k in range(3)])
    mag = mi.to_bf16_bits((mi_bf16_f32(rand) * np.float32(scale * 300)).astype(np.float32))
    latent = np.concatenate([rand, mag, edge_rows()])
    N = latent.shape[0]
    num_slots = N + 37
    slot = rng.permutation(num_slots)[:N].astype(np.int32)
    slot[::17] = -1
    slot[5] = num_slots + 3
    kv = rng.integers(0, 0x7E, size=(num_slots, 576), dtype=np.uint8)
    got = gpu_write(mla, latent, slot, kv, scale)
    want = oracle.cache_write(latent, slot, kv, True, scale)
    bad = np.argwhere(got != want)
    assert bad.size == 0, "first mismatches %s: gpu %s oracle %s" % (
        bad[:5].tolist(), got[tuple(bad[:5].T)], want[tuple(bad[:5].T)])


def mi_bf16_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def test_bf16_rows_are_copied(mla):
    rng = np.random.default_rng(43)
    latent = np.concatenate([mi.normal_bf16_bits(43, 1, (70, 576)), edge_rows()])
    N = latent.shape[0]
    num_slots = 3 * 64
    slot = rng.permutation(num_slots)[:N].astype(np.int32)
    slot[3] = -5
    kv = mi.normal_bf16_bits(43, 2, (num_slots, 576))
    got = gpu_write(mla, latent, slot, kv, 1.0)
    want = oracle.cache_write(latent, slot, kv, False, 1.0)
    assert np.array_equal(got, want)


def test_write_then_decode(mla):
    """Append 3 new positions to each of 4 sequences of an FP8 paged cache, then decode
    over the grown sequences: the written cache and the decode both match the oracle."""
    lens0 = [61, 300, 64, 1000]
    grow = 3
    lens = [L + grow for L in lens0]
    cache = mi.paged_cache(47, lens, 64, "fp8")
    rng = np.random.default_rng(47)
    B = len(lens)
    new = mi.normal_bf16_bits(47, 5, (B * grow, 576))
    slot = np.array([cache.block_table[b, t // 64] * 64 + t % 64
                     for b in range(B) for t in range(lens0[b], lens[b])], np.int32)
    kv_flat = cache.kv.reshape(-1, 576)
    want_kv = oracle.cache_write(new, slot, kv_flat, True, cache.kv_scale)
    got_kv = gpu_write(mla, new, slot, kv_flat, cache.kv_scale)
    assert np.array_equal(got_kv, want_kv)
    cache.kv = want_kv.reshape(cache.kv.shape)
    q = mi.normal_bf16_bits(47, 6, (B, 1, 12, 576))
    kv, bt, sl = cache_to_device(cache, DEV)
    sigma = mi.softmax_scale_for()
    out, lse = mla.verify(bf16_tensor(q, DEV), kv, bt, sl, softmax_scale=sigma,
                          kv_scale=cache.kv_scale)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(q, cache.kv, True, cache.kv_scale, cache.block_table,
                           cache.seq_lens, sigma)
    check_out(out, ro)
    check_lse(lse, rl)


@pytest.mark.parametrize("scale", [5.0 / 448.0, 1.0, 3.7e-3, 0.0123, float(np.nextafter(np.float32(2), np.float32(0))),
                                   float(np.float32(1) + np.float32(2.0 ** -23)), 2.0 ** -20, 3e-30, 7e29,
                                   1e-39, 3e38])
def test_every_bf16_value_codes_exactly(mla, scale):
    """All 65,536 BF16 bit patterns (zeros, subnormals, every exponent, infinities, NaNs)
    through the FP8 write at scales with awkward reciprocals: the kernel's quotient
    (reciprocal, product and one fused correction) must code exactly as fp32(x / scale).
    A scale whose reciprocal is not a normal number (1e-39, 3e38) takes the divisions."""
    scale = float(np.float32(scale))
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    latent = np.resize(bits, ((bits.size + 575) // 576) * 576).reshape(-1, 576)
    N = latent.shape[0]
    slot = np.arange(N, dtype=np.int32)
    kv = np.zeros((N, 576), np.uint8)
    got = gpu_write(mla, latent, slot, kv, scale)
    want = oracle.cache_write(latent, slot, kv, True, scale)
    bad = np.argwhere(got != want)
    assert bad.size == 0, "scale %r: %d codes differ, first at %s (x bits 0x%04x: gpu 0x%02x, oracle 0x%02x)" % (
        scale, len(bad), bad[0].tolist(), latent[tuple(bad[0])], got[tuple(bad[0])], want[tuple(bad[0])])
