"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies ``oracle/mla_oracle.c``, plants one plausible mistake (a dropped
term, a wrong sign, a wrong index, a transposed operand, an off-by-one bound),
builds the copy with gcc into a temporary directory and runs a battery of the
pins from ``test_oracle_pins``.  A mutant that passes every pin would mean the
pins cannot tell it from the real oracle, so each one must fail at least one.
Every mutant keeps all memory accesses inside the tiny inputs used here.
"""
import math
import os

import numpy as np
import pytest

import mla_inputs as mi
import oracle
from test_oracle_pins import (SIGMA, bf16_to_f64, brute_decode, brute_rows, cache_rows_f64,
                              fp8_to_f64, run_decode, tiny_decode)

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "mla_oracle.c")

MUTANTS = [
    ("max subtracted with the wrong sign", "w = exp(scores[t - begin] - m)", "w = exp(m - scores[t - begin])"),
    ("rotary dims dropped from the score", "for (int d = 0; d < ORACLE_DK; ++d) dot +=", "for (int d = 0; d < ORACLE_DV; ++d) dot +="),
    ("value read from the wrong end of the row", "out[e] += w * kv_elem(kv, row, e)", "out[e] += w * kv_elem(kv, row, e + 64)"),
    ("block table not consulted per block", "v->table[t / v->block_size]", "v->table[0]"),
    ("slot offset inside a block", "* v->block_size + t % v->block_size", "* v->block_size + t / v->block_size"),
    ("lse without the running max", "*lse = m + log(l);", "*lse = log(l);"),
    ("verify causal bound off by one", "(long)seq_lens[b] - P + j + 1", "(long)seq_lens[b] - P + j"),
    ("query positions reversed", "int j = (int)((flat / H) % P);", "int j = P - 1 - (int)((flat / H) % P);"),
    ("key range start ignored", "long begin = kv_begin ? kv_begin[b] : 0;", "long begin = 0;"),
    ("key range end ignored", "if (kv_end && kv_end[b] < end) end = kv_end[b];", ""),
    ("merge weight taken against the max", "double w = exp(x - L);", "double w = exp(x - M);"),
    ("merge normaliser dropped", "double L = M + log(sum);", "double L = M;"),
    ("FP8 exponent bias", "ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    ("FP8 subnormal step", "ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    ("FP8 per-tensor scale dropped", "v->fp8_lut[((const uint8_t*)row)[d]] * v->scale", "v->fp8_lut[((const uint8_t*)row)[d]]"),
    ("softmax scale dropped", "double s = sigma * dot;", "double s = dot;"),
    ("prefill diagonal excluded", "cu_seqlens[b], g + 1, sigma", "cu_seqlens[b], g, sigma"),
    ("prefill drops the first key of a sequence", "&v, cu_seqlens[b], g + 1", "&v, cu_seqlens[b] + 1, g + 1"),
    ("sequence index from the wrong stride", "int b = (int)(flat / ((long)H * P));", "int b = (int)(flat % B);"),
    ("BF16 decoded with the wrong shift", "(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    ("FP8 encoder ties away from zero", "(err == best_err && (c & 1) == 0 && (best & 1) == 1)",
     "(err == best_err && c > best)"),
    ("FP8 encoder drops the sign", "return (uint8_t)(best | (neg << 7));", "return (uint8_t)best;"),
    ("FP8 encoder maps NaN to zero", "if (isnan(y)) return 0x7F;", "if (isnan(y)) return 0x00;"),
    ("cache write multiplies by the scale", "mla_oracle_fp8_e4m3fn_encode(xf / kv_scale)",
     "mla_oracle_fp8_e4m3fn_encode(xf * kv_scale)"),
    ("top-k ties ranked toward the higher index", "return (a->i < b->i) ? -1 : (a->i > b->i);",
     "return (a->i > b->i) ? -1 : (a->i < b->i);"),
    ("top-k keeps the smallest entries", "if (a->v > b->v) return -1;", "if (a->v < b->v) return -1;"),
    ("top-k keeps one entry too many", "for (long j = 0; j < k; ++j) o[e[j].i]",
     "for (long j = 0; j <= k && j < vocab; ++j) o[e[j].i]"),
    ("top-k normalises by the whole row", "for (long j = 0; j < k; ++j) sum +=",
     "for (long j = 0; j < vocab; ++j) sum +="),
    ("top-k treats k = 0 as keep none", "(top_k[r] <= 0 || top_k[r] >= vocab)",
     "(top_k[r] < 0 || top_k[r] >= vocab)"),
    ("BF16 cache write to the row index instead of the slot",
     "memcpy((uint16_t*)kv + (size_t)s * ORACLE_DK", "memcpy((uint16_t*)kv + (size_t)n * ORACLE_DK"),
]


def pin_decode_bruteforce(orc):
    P = 3
    q, cache = tiny_decode(211, [5, 16, 33, 64], H=3, P=P, kv_dtype="bf16")
    kb = np.array([0, 2, 0, 9], np.int32)
    ke = np.array([5, 16, 20, 64], np.int32)
    o, l = run_decode(orc, q, cache, kv_begin=kb, kv_end=ke)
    ro, rl = brute_decode(q, cache, SIGMA, P, kb, ke)
    assert np.max(np.abs(o - ro)) < 1e-12 and np.max(np.abs(l - rl)) < 1e-12


def pin_decode_fp8_bruteforce(orc):
    q, cache = tiny_decode(223, [7, 40], H=2, P=1, kv_dtype="fp8")
    o, l = run_decode(orc, q, cache)
    ro, rl = brute_decode(q, cache, SIGMA, 1)
    assert np.max(np.abs(o - ro)) < 1e-12 and np.max(np.abs(l - rl)) < 1e-12


def pin_prefill_bruteforce(orc):
    w = mi.PrefillWorkload("tiny", [6, 20], 2, "bf16", seed=227)
    d = mi.prefill_inputs(w)
    out, lse = orc.prefill(d["q"], d["kv"], False, 1.0, d["cu_seqlens"], SIGMA)
    kvv = bf16_to_f64(d["kv"])
    cu = d["cu_seqlens"]
    for b in range(2):
        for g in range(cu[b], cu[b + 1]):
            o, s = brute_rows(bf16_to_f64(d["q"][g]), kvv[cu[b]:g + 1], SIGMA)
            assert np.max(np.abs(out[g] - o)) < 1e-12 and np.max(np.abs(lse[g] - s)) < 1e-12


def pin_merge_equals_whole(orc):
    q, cache = tiny_decode(229, [60, 33], H=2, P=1)
    wo, wl = run_decode(orc, q, cache)
    po, pl = [], []
    for a, c in [(0, 10), (10, 10), (10, 41), (41, 100)]:
        o, l = run_decode(orc, q, cache, kv_begin=np.full(2, a, np.int32),
                          kv_end=np.full(2, c, np.int32))
        po.append(o.reshape(-1, 512))
        pl.append(l.reshape(-1))
    mo, ml = orc.merge(np.stack(po), np.stack(pl))
    assert np.max(np.abs(mo - wo.reshape(-1, 512))) < 1e-12
    assert np.max(np.abs(ml - wl.reshape(-1))) < 1e-12


def pin_fp8_codec(orc):
    ref = fp8_to_f64(np.arange(256, dtype=np.uint8))
    got = np.array([orc.fp8_e4m3fn_value(c) for c in range(256)])
    m = ~np.isnan(ref)
    assert np.array_equal(np.isnan(ref), np.isnan(got)) and np.array_equal(ref[m], got[m])


def pin_zero_query(orc):
    q, cache = tiny_decode(233, [9, 64], H=1, P=1, kv_dtype="fp8")
    q[:] = 0
    out, lse = run_decode(orc, q, cache)
    for b, L in enumerate([9, 64]):
        V = cache_rows_f64(cache, b, 0, L)[:, :512]
        assert np.max(np.abs(out[b, 0, 0] - V.mean(axis=0))) < 1e-13
        assert lse[b, 0, 0] == math.log(L)


def pin_fp8_encoder(orc):
    finite = [c for c in range(256) if (c & 0x7F) != 0x7F]
    for c in finite:  # every code round-trips
        assert orc.fp8_e4m3fn_encode(orc.fp8_e4m3fn_value(c)) == c
    pos = sorted(c for c in finite if c < 0x80)
    for a, b in zip(pos[:-1], pos[1:]):  # midpoints tie to the even mantissa
        mid = (orc.fp8_e4m3fn_value(a) + orc.fp8_e4m3fn_value(b)) / 2
        assert orc.fp8_e4m3fn_encode(mid) == (a if a % 2 == 0 else b)
    assert orc.fp8_e4m3fn_encode(math.nan) == 0x7F
    assert orc.fp8_e4m3fn_encode(-1e9) == 0xFE


def pin_cache_write(orc):
    import torch
    rng = np.random.default_rng(239)
    N, num_slots = 24, 64
    latent = mi.normal_bf16_bits(239, 1, (N, 576))
    slot = rng.permutation(num_slots)[:N].astype(np.int32)
    kv8 = np.zeros((num_slots, 576), np.uint8)
    out8 = orc.cache_write(latent, slot, kv8, True, 0.0123)
    x = torch.from_numpy(latent.view(np.int16)).view(torch.bfloat16).float()
    y = torch.clamp(x / torch.tensor(0.0123, dtype=torch.float32), -448, 448)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(out8[slot], codes)
    kv16 = np.zeros((num_slots, 576), np.uint16)
    out16 = orc.cache_write(latent, slot, kv16, False, 1.0)
    assert np.array_equal(out16[slot], latent)


def pin_top_k(orc):
    from test_oracle_top_k import torch_reference, tied_rows
    p = np.concatenate([mi.probability_rows(241, 4, 500), tied_rows(243, 4, 500, 5)])
    ks = np.array([1, 7, 0, 250, 3, 60, 499, 500], np.int32)
    out = orc.top_k_renorm_prob(p, ks)
    for r, k in enumerate(ks):
        kept, ref = torch_reference(p[r], k)
        assert np.array_equal(out[r] != 0, kept)
        assert np.max(np.abs(out[r] - ref)) < 1e-12


BATTERY = [pin_decode_bruteforce, pin_decode_fp8_bruteforce, pin_prefill_bruteforce,
           pin_merge_equals_whole, pin_fp8_codec, pin_zero_query, pin_fp8_encoder,
           pin_cache_write, pin_top_k]


def _failures(orc):
    failed = []
    for pin in BATTERY:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    return failed


def test_battery_passes_on_the_real_oracle():
    assert _failures(oracle.get()) == []


@pytest.mark.parametrize("name,before,after", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, before, after):
    src = open(SRC).read()
    assert src.count(before) == 1, "mutation anchor must occur exactly once: %r" % before
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(before, after))
    lib = oracle.build(force=True, src=str(mutated), out=str(tmp_path / "libmutant.so"))
    failed = _failures(oracle.OracleLib(lib))
    assert failed, "planted mistake '%s' passed every pin" % name
