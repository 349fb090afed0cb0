#!/usr/bin/env python3
"""Benchmark of MLA latent-KV decode on one MI355X, with roofline and CPU-oracle figures.

A step is one pass of the decode hot path over one batch of the headline workload:
32 sequences, 12 heads, one query each, per-sequence contexts uniform in [4096, 16384],
FP8 E4M3 latent rows with a per-tensor scale in 64-token pages behind a shuffled block
table (synthetic, seeded).  One step = one mla_verify call through the C-ABI: a single
persistent kernel that streams the batch's latent rows and merges split sequences in the
same launch; the inputs are resident in HBM before timing starts.  KV pools rotate
over several copies so the 256 MB last-level cache cannot hold the one being read.

Printed: ONE JSON line (metric, value = algorithmic KV-read GB/s of the whole step,
roofline of the dominant kernel from HIP events on its stream around the back-to-back
timed steps, CPU oracle baseline, and the causal prefill figures the same metric names).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
METRIC = "MLA decode KV GB/s (% of HBM peak) + prefill tokens/s (% MFMA peak), 12 heads"
DECODE_WORKLOAD = "decode_b32_h12_fp8_paged"
PREFILL_WORKLOAD = "prefill_t32768_h12_bf16"
PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(name: str) -> str:
    """Hash of a kernel source with its // comments and blank lines removed, so that
    counters taken on a kernel stay attached to it through comment-only edits."""
    import re
    p = os.path.join(ROOT, "mla_latent_kv_attention_amd", "csrc", name)
    text = open(p, encoding="utf-8").read()
    code = [re.sub(r"//.*$", "", l).rstrip() for l in text.splitlines()]
    return hashlib.sha256("\n".join(l for l in code if l).encode()).hexdigest()[:16]


def traffic_from_profile(kernel_file: str, workload: str):
    """Counter-derived HBM bytes per launch, if a summary for the current kernel source exists."""
    path = os.path.join(PROFILE_DIR, "%s_pmc.json" % workload)
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except ValueError:
        return None
    if d.get("source_sha256_16") != source_hash(kernel_file):
        return None  # the kernel changed since the counters were taken
    return d.get("hbm_bytes_per_launch")


def host_cores() -> int:
    """CPU cores this process may run on (its affinity mask), the oracle's thread count."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def cpu_baseline(q, cache, alg_bytes, min_seconds=10.0, max_reps=400):
    """The FP64 oracle on the whole batch (every row), repeated until >= min_seconds."""
    import oracle
    import mla_inputs as mi
    threads = host_cores()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.decode(q, cache.kv, cache.kv_dtype == "fp8", cache.kv_scale, cache.block_table,
                      cache.seq_lens, mi.softmax_scale_for(), threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or reps >= max_reps:
            break
    return {"value": alg_bytes * reps / el / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": "the whole %s batch (all 384 query rows), %d pass(es), %.1f s of FP64 "
                      "oracle time on %d threads (the process's CPU affinity)"
                      % (DECODE_WORKLOAD, reps, el, threads)}


def prefill_cpu_baseline(pd, pw, min_seconds=10.0, chunk=64, max_chunks=64):
    """The FP64 oracle on a stratified sample of the prefill's tokens, all heads: chunk c
    takes the tokens floor((k + (c * 0.618) mod 1) * T / chunk), k = 0 .. chunk - 1, one per
    equal slice of the sequence.  A token's work grows with its position (token i sees i + 1
    keys), and each chunk has one token in every slice, so the sample's mean work per token
    is the whole prefill's to within one slice; tokens/s of the sample is reported as the
    whole job's rate, with the flop rate of the tokens actually computed beside it."""
    import oracle
    T = pw.total_tokens
    threads = host_cores()
    fp8 = pw.kv_dtype == "fp8"
    done, flops, c, t0 = 0, 0, 0, time.perf_counter()
    while True:
        off = (c * 0.6180339887) % 1.0
        toks = np.minimum(((np.arange(chunk) + off) * T / chunk).astype(np.int64), T - 1)
        oracle.prefill(pd["q"], pd["kv"], fp8, float(pd["kv_scale"]) if fp8 else 1.0,
                       pd["cu_seqlens"], pw.softmax_scale, tokens=toks, threads=threads)
        done += len(toks)
        flops += int(np.sum(toks + 1)) * pw.heads * 2176
        c += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or c >= max_chunks:
            break
    return {"value": round(done / el, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "gflops": round(flops / el / 1e9, 2),
            "sample": "%d of the %d tokens (all %d heads) of %s, %d stratified chunks of %d (one "
                      "token per 1/%d of the sequence), %.1f s of FP64 oracle time on %d threads "
                      "(the process's CPU affinity); rate = sampled tokens / time"
                      % (done, T, pw.heads, pw.name, c, chunk, chunk, el, threads)}


def gpu_clocks():
    """Current shader / memory clock levels from the amdgpu sysfs files (the level
    marked '*'), or None.  Plain file reads: this process has the GPU open, so it must
    not start other programs."""
    import glob
    found = []
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        for name in ("pp_dpm_sclk", "pp_dpm_mclk"):
            try:
                with open(os.path.join(dev, name)) as f:
                    cur = [l.strip() for l in f if "*" in l]
            except OSError:
                continue
            if cur:
                found.append("%s %s: %s" % (os.path.basename(os.path.dirname(dev)), name,
                                            cur[0]))
    return " | ".join(found[:8]) or None


def event_times(torch, stream, fn, n):
    """HIP-event duration (ms) of each of n calls of fn on `stream`."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        fn(i)
        b.record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev])


def back_to_back_us(torch, stream, fn, n):
    """Microseconds per call of n calls of fn launched back to back between two HIP
    events on `stream`."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(n):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / n


def graph_replay_us(torch, fns, out, calls=100, replays=5):
    """Capture `calls` launches (cycling through fns) into one HIP graph; check that
    every replay reproduces the eager result bitwise (eager work and a synchronisation
    between replays), then time replays.  Returns microseconds per call."""
    fns[0]()
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            fns[i % len(fns)]()
    for _ in range(3):
        out.zero_()
        fns[0]()                       # eager work between replays
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(out, ref):
            raise AssertionError("graph replay differs from the eager call")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s = torch.cuda.current_stream()
    torch.cuda.synchronize()
    a.record(s)
    for _ in range(replays):
        g.replay()
    b.record(s)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (replays * calls)


def read_ceiling_gbs(torch, stream, nbytes, copies, calls=30):
    """Rate of a kernel that only reads nbytes (the headline's algorithmic bytes) once,
    over `copies` rotating buffers like the KV pools: back-to-back HIP-event time per
    call, best over a few grid sizes."""
    from mla_latent_kv_attention_amd.read_probe import hbm_read_probe
    n = (nbytes + 15) // 16 * 16
    bufs = [torch.ones(n, dtype=torch.uint8, device="cuda:0") for _ in range(copies)]
    sink = torch.empty(65536 * 256, dtype=torch.int32, device="cuda:0")
    best, grids = None, [512, 1024, 2048]
    for g in grids:
        us = back_to_back_us(torch, stream, lambda i: hbm_read_probe(
            bufs[i % copies], sink, grid=g), calls)
        best = us if best is None else min(best, us)
    del bufs
    return {"us": best, "gbs": nbytes / (best * 1e-6) / 1e9, "grids": grids}


def secondary_configs(torch, mi, mla, acc, oracle, bf16_tensor, cache_to_device, check_out,
                      check_lse, dev, stream, only=None):
    """The other decode / verify configurations: parity on sampled rows, then per-call
    HIP-event times (p10 / p50 / p90) and, for the launch-bound ones, HIP-graph replays."""
    res = {}
    want = lambda n: only is None or n in only
    for name, rotate in (("decode_b1_h12_l1024_bf16", 1), ("verify_b4_p4_h12_l32768_bf16", 4),
                         ("verify_b1_p4_h12_l32768_fp8", 28)):
        if not want(name):
            continue
        w = mi.WORKLOADS[name]
        log("generating", name)
        d = mi.decode_inputs(w)
        q_np, cache = d["q"], d["cache"]
        B, P, H = q_np.shape[:3]
        L = [int(x) for x in cache.seq_lens]
        kv0, bt, sl = cache_to_device(cache, dev)
        pools = [kv0] + [kv0.clone() for _ in range(rotate - 1)]
        q = bf16_tensor(q_np, dev).reshape(B, P, H, 576)
        out = torch.empty((B, P, H, 512), dtype=torch.float32, device=dev)
        lse = torch.empty((B, P, H), dtype=torch.float32, device=dev)
        ws = torch.zeros(max(1, mla.decode_workspace_size(B, P, H, max(L))), dtype=torch.uint8,
                         device=dev)
        fns = [mla.verify_launcher(q, kv, bt, sl, softmax_scale=w.softmax_scale,
                                   kv_scale=cache.kv_scale, max_kv_len=max(L), out=out, lse=lse,
                                   workspace=ws) for kv in pools]
        N = B * P * H
        rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(9).choice(
            N, min(N, 24), replace=False)])).astype(np.int64)
        ro, rl = oracle.decode(q_np, cache.kv, cache.kv_dtype == "fp8", cache.kv_scale,
                               cache.block_table, cache.seq_lens, w.softmax_scale, rows=rows)
        for f in fns:
            f()
            torch.cuda.synchronize()
            idx = torch.from_numpy(rows).to(dev)
            check_out(out.reshape(N, 512)[idx], ro, name + " out")
            check_lse(lse.reshape(N)[idx], rl, name + " lse")
        ms = event_times(torch, stream, lambda i: fns[i % len(fns)](), 100)
        ab = acc.decode_bytes(L, P, H, w.kv_dtype, out_bytes=4, block_size=cache.block_size)
        us = [float(np.percentile(ms, p_)) * 1e3 for p_ in (10, 50, 90)]
        b2b = back_to_back_us(torch, stream, lambda i: fns[i % len(fns)](), 100)
        g_us = graph_replay_us(torch, fns, out)
        res[name] = {"us_p10_p50_p90": [round(x, 2) for x in us],
                     "us_back_to_back": round(b2b, 2),
                     "graph_replay_us": round(g_us, 2), "algorithmic_bytes": ab,
                     "gbs_back_to_back": round(ab / (b2b * 1e-6) / 1e9, 1),
                     "hbm_frac_back_to_back": round(ab / (b2b * 1e-6) / 8e12, 4),
                     "pieces": mla.decode_num_splits(B, P, H, max(L)), "kv_pool_copies": rotate}
        if P > 1:  # verify: time per sequence and layer (graph replay), as the pages quote it
            res[name]["graph_us_per_sequence"] = round(g_us / B, 2)
        log("%s: %.1f us back to back, p50 %.1f us per call, graph %.1f us, %.0f GB/s"
            % (name, b2b, us[1], g_us, res[name]["gbs_back_to_back"]))
        del pools, kv0, fns

    if want("decode_b8_h12_l142000_fp8_8parts"):
        # 142,000-token contexts in 8 contiguous partitions (one call each, as a position shard
        # would compute its share) merged by mla_merge_lse
        name = "decode_b8_h12_l142000_fp8_8parts"
        w = mi.WORKLOADS[name]
        log("generating", name)
        d = mi.decode_inputs(w)
        q_np, cache = d["q"], d["cache"]
        B, P, H = q_np.shape[:3]
        N = B * P * H
        kv, bt, sl = cache_to_device(cache, dev)
        q = bf16_tensor(q_np, dev).reshape(B, P, H, 576)
        bounds = mi.partition_bounds(int(cache.seq_lens[0]), w.partitions)
        S = len(bounds)
        part_out = torch.empty((S, B, P, H, 512), dtype=torch.float32, device=dev)
        part_lse = torch.empty((S, B, P, H), dtype=torch.float32, device=dev)
        out = torch.empty((N, 512), dtype=torch.float32, device=dev)
        lse = torch.empty((N,), dtype=torch.float32, device=dev)
        span = max(hi - lo for lo, hi in bounds)
        wss = [torch.zeros(max(1, mla.decode_workspace_size(B, P, H, span)), dtype=torch.uint8,
                           device=dev) for _ in bounds]
        kbs = [torch.full((B,), lo, dtype=torch.int32, device=dev) for lo, _ in bounds]
        kes = [torch.full((B,), hi, dtype=torch.int32, device=dev) for _, hi in bounds]
        fns = [mla.verify_launcher(q, kv, bt, sl, softmax_scale=w.softmax_scale,
                                   kv_scale=cache.kv_scale, max_kv_len=span, out=part_out[j],
                                   lse=part_lse[j], workspace=wss[j], kv_begin=kbs[j], kv_end=kes[j])
               for j in range(S)]

        def call(_):
            for f in fns:
                f()
            mla.merge_lse(part_out.reshape(S, N, 512), part_lse.reshape(S, N), out=out, lse=lse)

        # The same partitions as one call: the S x B (partition, sequence) ranges as
        # S * B sequences of one batch (query and block-table row repeated per
        # partition, each range given by kv_begin / kv_end), so the pieces of all
        # partitions share the chip; then the same merge.
        qb = q.repeat(S, 1, 1, 1).contiguous()
        btb = bt.repeat(S, 1).contiguous()
        slb = sl.repeat(S).contiguous()
        kbb = torch.tensor(np.repeat([lo for lo, _ in bounds], B).astype(np.int32), device=dev)
        keb = torch.tensor(np.repeat([hi for _, hi in bounds], B).astype(np.int32), device=dev)
        wsb = torch.zeros(max(1, mla.decode_workspace_size(S * B, P, H, span)),
                          dtype=torch.uint8, device=dev)
        fb = mla.verify_launcher(qb, kv, btb, slb, softmax_scale=w.softmax_scale,
                                 kv_scale=cache.kv_scale, max_kv_len=span,
                                 out=part_out.reshape(S * B, P, H, 512),
                                 lse=part_lse.reshape(S * B, P, H), workspace=wsb,
                                 kv_begin=kbb, kv_end=keb)

        def call_batched(_):
            fb()
            mla.merge_lse(part_out.reshape(S, N, 512), part_lse.reshape(S, N), out=out, lse=lse)

        rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(10).choice(
            N, 16, replace=False)])).astype(np.int64)
        ro, rl = oracle.decode(q_np, cache.kv, True, cache.kv_scale, cache.block_table,
                               cache.seq_lens, w.softmax_scale, rows=rows)
        idx = torch.from_numpy(rows).to(dev)
        for form, f in (("batched", call_batched), ("per-partition", call)):
            out.fill_(float("nan"))
            f(0)
            torch.cuda.synchronize()
            check_out(out[idx], ro, "%s %s out" % (name, form))
            check_lse(lse[idx], rl, "%s %s lse" % (name, form))
        ms = event_times(torch, stream, call_batched, 30)
        b2b = back_to_back_us(torch, stream, call_batched, 30)
        b2b_calls = back_to_back_us(torch, stream, call, 30)
        L = [int(x) for x in cache.seq_lens]
        ab = sum(acc.decode_bytes(L, P, H, "fp8", out_bytes=4, block_size=cache.block_size,
                                  kv_begin=[lo] * B, kv_end=[hi] * B) for lo, hi in bounds)
        us = [float(np.percentile(ms, p_)) * 1e3 for p_ in (10, 50, 90)]
        res[name] = {"us_p10_p50_p90": [round(x, 2) for x in us], "algorithmic_bytes": ab,
                     "gbs_p50": round(ab / (us[1] * 1e-6) / 1e9, 1),
                     "hbm_frac_p50": round(ab / (us[1] * 1e-6) / 8e12, 4),
                     "us_back_to_back": round(b2b, 2),
                     "gbs_back_to_back": round(ab / (b2b * 1e-6) / 1e9, 1),
                     "hbm_frac_back_to_back": round(ab / (b2b * 1e-6) / 8e12, 4),
                     "pieces": mla.decode_num_splits(S * B, P, H, span),
                     "launches": 2,
                     "note": "the 8 partitions' 64 ranges in one mla_verify call + mla_merge_lse",
                     "per_partition_calls_us_back_to_back": round(b2b_calls, 2),
                     "per_partition_calls_pieces": mla.decode_num_splits(B, P, H, span)}
        log("%s: %.1f us back to back (batched), %.1f us as 8 calls, p50 %.1f us, %.0f GB/s"
            % (name, b2b, b2b_calls, us[1], res[name]["gbs_back_to_back"]))
        del kv, part_out, fns, fb

    if want("prefill_t32768_h12_fp8"):
        # the same causal prefill over an FP8 latent cache (per-tensor scale): the same
        # seed and shape as the BF16 workload, its rows quantised to E4M3FN
        pw = mi.PrefillWorkload("prefill_t32768_h12_fp8", [32768], 12, "fp8", seed=404)
        res[pw.name] = time_prefill(torch, mi, mla, acc, oracle, bf16_tensor, check_out,
                                    check_lse, dev, stream, pw, 5)

    if want("cache_write_t32768_fp8_paged"):
        # cache write: the 32,768 new rows of the prefill workload quantised into a
        # shuffled FP8 paged cache (64-token blocks)
        name = "cache_write_t32768_fp8_paged"
        T = 32768
        log("generating", name)
        latent_np = mi.normal_bf16_bits(606, 1, (T, 576))
        blocks = np.random.default_rng(606).permutation(T // 64 + 8).astype(np.int64)
        slot_np = (blocks[np.arange(T) // 64] * 64 + np.arange(T) % 64).astype(np.int32)
        scale = float(np.float32(5.0 / 448.0))
        latent = bf16_tensor(latent_np, dev).reshape(T, 576)
        slot_t = torch.from_numpy(slot_np).to(dev)
        kvc = torch.zeros(((T // 64 + 8) * 64, 576), dtype=torch.uint8, device=dev)
        mla.cache_write(latent, kvc, slot_t, kv_scale=scale)
        torch.cuda.synchronize()
        rows = np.random.default_rng(607).choice(T, 64, replace=False)
        sub = oracle.cache_write(latent_np[rows], np.arange(64, dtype=np.int32),
                                 np.zeros((64, 576), np.uint8), True, scale)
        if not np.array_equal(kvc[torch.from_numpy(slot_np[rows]).to(dev)].cpu().numpy(), sub):
            raise AssertionError(name + ": codes differ from the oracle")
        ms = event_times(torch, stream, lambda i: mla.cache_write(latent, kvc, slot_t,
                                                                  kv_scale=scale), 50)
        ab = T * (2 * 576 + 576 + 4)
        us = [float(np.percentile(ms, p_)) * 1e3 for p_ in (10, 50, 90)]
        res[name] = {"us_p10_p50_p90": [round(x, 2) for x in us], "algorithmic_bytes": ab,
                     "gbs_p50": round(ab / (us[1] * 1e-6) / 1e9, 1),
                     "hbm_frac_p50": round(ab / (us[1] * 1e-6) / 8e12, 4)}
        log("%s: p50 %.1f us, %.0f GB/s" % (name, us[1], res[name]["gbs_p50"]))
        del latent, kvc

    if want("top_k_renorm_r128_v163840"):
        # top-k renormalisation of the target probabilities after a verify step: 128 rows
        # (32 sequences x 4 positions) over a 163,840-entry vocabulary, k per row in [1, 100];
        # 7 rotating copies of the 84 MB input so every call reads HBM
        name = "top_k_renorm_r128_v163840"
        w = mi.TOP_K_WORKLOADS[name]
        log("generating", name)
        p_np, k_np = w.probs(), w.top_k()
        copies = 7
        pin = [torch.from_numpy(p_np).to(dev) for _ in range(copies)]
        pout = [torch.empty_like(pin[0]) for _ in range(copies)]
        kt = torch.from_numpy(k_np).to(dev)
        lib = mla.library()
        need = mla.top_k_renorm_workspace_size(w.rows, w.vocab)
        tws = torch.empty(need, dtype=torch.uint8, device=dev)
        import ctypes
        sptr = ctypes.c_void_p(stream.cuda_stream)
        targs = [(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(kt.data_ptr()), w.rows, w.vocab,
                  ctypes.c_void_p(b.data_ptr()), ctypes.c_void_p(tws.data_ptr()), need, sptr)
                 for a, b in zip(pin, pout)]

        def tcall(i):
            st = lib.mla_top_k_renorm_prob(*targs[i % copies])
            if st != 0:
                raise RuntimeError("mla_top_k_renorm_prob failed: %d" % st)
        for i in range(copies):
            tcall(i)
        torch.cuda.synchronize()
        chk = np.array([0, 1, 63, w.rows - 1])
        want = oracle.top_k_renorm_prob(p_np[chk], k_np[chk])
        for j in range(copies):
            got = pout[j][torch.from_numpy(chk).to(dev)].cpu().numpy()
            if not np.array_equal(got != 0, want != 0):
                raise AssertionError(name + ": kept sets differ from the oracle")
            m = want != 0
            if np.max(np.abs(got[m] - want[m]) / want[m]) > 2e-6:
                raise AssertionError(name + ": values differ from the oracle")
        ms = event_times(torch, stream, tcall, 50)
        b2b = back_to_back_us(torch, stream, tcall, 50)
        ab = w.rows * w.vocab * 8 + w.rows * 4
        us = [float(np.percentile(ms, p_)) * 1e3 for p_ in (10, 50, 90)]
        res[name] = {"us_p10_p50_p90": [round(x, 2) for x in us], "algorithmic_bytes": ab,
                     "gbs_p50": round(ab / (us[1] * 1e-6) / 1e9, 1),
                     "hbm_frac_p50": round(ab / (us[1] * 1e-6) / 8e12, 4), "input_copies": copies,
                     "us_back_to_back": round(b2b, 2),
                     "gbs_back_to_back": round(ab / (b2b * 1e-6) / 1e9, 1),
                     "hbm_frac_back_to_back": round(ab / (b2b * 1e-6) / 8e12, 4),
                     "launches": 2}
        log("%s: %.1f us back to back, p50 %.1f us per call, %.0f GB/s"
            % (name, b2b, us[1], res[name]["gbs_back_to_back"]))
    return res


def time_prefill(torch, mi, mla, acc, oracle, bf16_tensor, check_out, check_lse, dev, stream,
                 pw, steps, warmup=4):
    """One causal prefill workload: parity on sampled tokens against the oracle, `warmup`
    untimed calls (the GPU idles while the oracle runs, and its clocks take about three
    11 ms calls to come back up), then the mean of `steps` HIP-event-timed calls."""
    log("generating", pw.name)
    pd = mi.prefill_inputs(pw)
    T = pw.total_tokens
    fp8 = pw.kv_dtype == "fp8"
    pq = bf16_tensor(pd["q"], dev).reshape(T, pw.heads, 576)
    if fp8:
        pkv = torch.from_numpy(np.ascontiguousarray(pd["kv"])).to(dev).reshape(T, 576)
    else:
        pkv = bf16_tensor(pd["kv"], dev).reshape(T, 576)
    kv_scale = float(pd["kv_scale"]) if fp8 else 1.0
    cu = torch.from_numpy(pd["cu_seqlens"]).to(dev)
    pout = torch.empty((T, pw.heads, 512), dtype=torch.bfloat16, device=dev)
    plse = torch.empty((T, pw.heads), dtype=torch.float32, device=dev)

    def pstep():
        mla.prefill(pq, pkv, cu, softmax_scale=pw.softmax_scale, kv_scale=kv_scale,
                    max_seqlen=T, out_dtype=torch.bfloat16, out=pout, lse=plse)
    pstep()
    torch.cuda.synchronize()
    toks = np.array([0, 1, 4095, T - 1], np.int64)
    ro, rl = oracle.prefill(pd["q"], pd["kv"], fp8, kv_scale, pd["cu_seqlens"],
                            pw.softmax_scale, tokens=toks)
    ti = torch.from_numpy(toks).to(dev)
    check_out(pout[ti], ro, pw.name + " out")
    check_lse(plse[ti], rl, pw.name + " lse")
    for _ in range(max(1, warmup)):
        pstep()
    pe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in pe:
        a.record(stream)
        pstep()
        b.record(stream)
    torch.cuda.synchronize()
    pms = np.array([a.elapsed_time(b) for a, b in pe])
    pflops = acc.prefill_flops(pw.seq_lens, pw.heads)
    tflops = pflops / (pms.mean() * 1e-3) / 1e12
    log("%s: %.2f ms, %.0f tok/s, %.1f TFLOP/s" % (pw.name, pms.mean(),
                                                  T / (pms.mean() * 1e-3), tflops))
    return {
        "workload": pw.name, "tokens_per_s": round(T / (pms.mean() * 1e-3), 1),
        "ms": round(float(pms.mean()), 3), "tflops": round(tflops, 1),
        "mfma_frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
        "peak_tflops": BF16_MFMA_PEAK_TFLOPS, "algorithmic_flops": pflops,
        "kernel": "prefill_kernel<%s>" % pw.kv_dtype}


def run_prefill(args, torch, mi, mla, acc, oracle, bf16_tensor, check_out, check_lse, dev,
                stream, result):
    """Causal prefill of the 32K x 12-head workload: parity on sampled tokens, timing, and
    the oracle's rate on a bounded sample of the same workload."""
    pw = mi.WORKLOADS[PREFILL_WORKLOAD]
    res = time_prefill(torch, mi, mla, acc, oracle, bf16_tensor, check_out, check_lse, dev,
                       stream, pw, args.prefill_steps, args.prefill_warmup)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on prefill tokens")
        res["cpu_baseline"] = prefill_cpu_baseline(mi.prefill_inputs(pw), pw)
    result["prefill"] = res


TIMELINE_PHASES = {
    "decode": ["work-group starts", "step-list scan done", "streaming loop ends",
               "wave merge done", "result written / share published", "last piece's merge done"],
    "verify": ["work-group starts", "step-list scan done", "queries and tile 0 in",
               "first tile-loop barrier", "tile loop ends", "normalisers shared",
               "result written / share published"],
}


def run_timeline(args, torch, mi, mla, bf16_tensor, cache_to_device, dev):
    """Per-work-group phase stamps (libmla_timeline.so: the attention library with stamps of
    the 100 MHz real-time counter compiled in): for each workload, `samples` calls each
    following another call on the stream, the stamps of the later one read; per phase the
    median / p90 / max over work-groups of the time from the call's first work-group start,
    averaged over the samples.  Stamps a call did not write (its own phase was not reached,
    e.g. a merge by another piece) are older than its start and left out."""
    import ctypes
    lib = mla.library()
    for fn in ("mla_timeline_read_decode", "mla_timeline_read_verify"):
        getattr(lib, fn).argtypes = [ctypes.c_void_p, ctypes.c_size_t]
        getattr(lib, fn).restype = ctypes.c_int
    groups, slots = 4096, 8
    res = {}
    for name, kind in ((DECODE_WORKLOAD, "decode"), ("verify_b4_p4_h12_l32768_bf16", "verify")):
        w = mi.WORKLOADS[name]
        log("timeline:", name)
        d = mi.decode_inputs(w)
        q_np, cache = d["q"], d["cache"]
        B, P, H = q_np.shape[:3]
        L = [int(x) for x in cache.seq_lens]
        kv0, bt, sl = cache_to_device(cache, dev)
        pools = [kv0] + [kv0.clone() for _ in range(2)]
        q = bf16_tensor(q_np, dev).reshape(B, P, H, 576)
        out = torch.empty((B, P, H, 512), dtype=torch.float32, device=dev)
        lse = torch.empty((B, P, H), dtype=torch.float32, device=dev)
        ws = torch.zeros(max(1, mla.decode_workspace_size(B, P, H, max(L))), dtype=torch.uint8,
                         device=dev)
        fns = [mla.verify_launcher(q, kv, bt, sl, softmax_scale=w.softmax_scale,
                                   kv_scale=cache.kv_scale, max_kv_len=max(L), out=out, lse=lse,
                                   workspace=ws) for kv in pools]
        G = mla.decode_num_splits(B, P, H, max(L))
        if kind == "decode":
            G *= (P * H + 15) // 16  # one work-group per (piece, row block)
        read = getattr(lib, "mla_timeline_read_" + kind)
        buf = np.zeros(groups * slots, np.uint64)
        for i in range(10):
            fns[i % 3]()
        per = []
        for sample in range(args.timeline_samples):
            fns[sample % 3]()
            if read(buf.ctypes.data, buf.nbytes) != 0:  # read and clear
                raise RuntimeError("timeline stamps could not be read")
            fns[(sample + 1) % 3]()
            fns[(sample + 2) % 3]()
            if read(buf.ctypes.data, buf.nbytes) != 0:
                raise RuntimeError("timeline stamps could not be read")
            t = buf.reshape(groups, slots)[:G].astype(np.float64)
            t0 = t[:, 0].min()  # the later call's start: every work-group stamps slot 0
            rows = []
            for k in range(len(TIMELINE_PHASES[kind])):
                v = t[:, k]
                v = (v[v >= t0] - t0) / 100.0  # 100 MHz ticks -> us
                rows.append((np.median(v), np.percentile(v, 90), v.max()) if len(v) else
                            (float("nan"),) * 3)
            per.append(rows)
        a = np.array(per)  # samples x phases x 3
        tab = {ph: [round(float(x), 2) for x in np.nanmean(a[:, k, :], axis=0)]
               for k, ph in enumerate(TIMELINE_PHASES[kind])}
        res[name] = {"work_groups": G, "us_median_p90_max": tab,
                     "samples": args.timeline_samples}
        log("%s (%d work-groups; us from the first work-group's start: median / p90 / max)"
            % (name, G))
        for ph, v in tab.items():
            log("  %-36s %8.2f %8.2f %8.2f" % (ph, v[0], v[1], v[2]))
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # ~10 ms of decode steps: after the parity check's CPU work the GPU's clocks take a
    # few milliseconds of sustained work to come back up
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--rotate", type=int, default=3, help="KV pool copies cycled over")
    ap.add_argument("--num-splits", type=int, default=0, help="pieces; 0 = automatic plan")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the other decode / verify configurations")
    ap.add_argument("--no-decode", action="store_true",
                    help="prefill figures only (for profiling the prefill kernel)")
    ap.add_argument("--prefill-steps", type=int, default=5)
    ap.add_argument("--prefill-warmup", type=int, default=4)
    ap.add_argument("--secondary", default="",
                    help="comma-separated secondary workloads to run (default: all)")
    ap.add_argument("--timeline", action="store_true",
                    help="only print per-work-group phase timelines of the headline decode and "
                         "the 4 x 4 x 32K verify (loads libmla_timeline.so) and exit")
    ap.add_argument("--timeline-samples", type=int, default=8)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device copies of MIB MiB (the reference kernel "
                         "for scaling HBM byte counters) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (position or head "
              "sharding is a design note only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "dispatches": 5}), flush=True)
        return
    import mla_inputs as mi
    import mla_latent_kv_attention_amd as mla
    from mla_latent_kv_attention_amd import accounting as acc
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import bf16_tensor, cache_to_device, check_lse, check_out

    if args.timeline:
        mla.LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(mla.__file__)),
                                    "libmla_timeline.so")
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        res = run_timeline(args, torch, mi, mla, bf16_tensor, cache_to_device, dev)
        print(json.dumps({"timeline": res}), flush=True)
        return
    mla.library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    if args.no_decode:
        result = {"metric": METRIC, "value": None, "unit": "GB/s", "n_gpus": 1, "steps": 0,
                  "warmup": 0, "ms_per_step": None, "higher_is_better": True,
                  "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                  "data": "synthetic", "config": {"workload": PREFILL_WORKLOAD}}
        import oracle
        if not args.no_prefill:
            run_prefill(args, torch, mi, mla, acc, oracle, bf16_tensor, check_out, check_lse, dev,
                        stream, result)
        if args.secondary:
            result["secondary"] = secondary_configs(torch, mi, mla, acc, oracle, bf16_tensor,
                                                    cache_to_device, check_out, check_lse, dev,
                                                    stream, only=set(args.secondary.split(",")))
        print(json.dumps(result), flush=True)
        return

    # ---------------- decode workload ----------------
    w = mi.WORKLOADS[DECODE_WORKLOAD]
    log("generating", w.name)
    d = mi.decode_inputs(w)
    q_np, cache = d["q"], d["cache"]
    B, P, H = q_np.shape[:3]
    L = [int(x) for x in cache.seq_lens]
    max_len = max(L)
    kv0, bt, sl = cache_to_device(cache, dev)
    pools = [kv0] + [kv0.clone() for _ in range(max(0, args.rotate - 1))]
    q = bf16_tensor(q_np, dev).reshape(B, P, H, 576)
    W = mla.decode_num_splits(B, P, H, max_len, args.num_splits)
    N = B * P * H
    out = torch.empty((B, P, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((B, P, H), dtype=torch.float32, device=dev)
    # one zero-filled workspace for every call: each call leaves its counters zero
    workspace = torch.zeros(max(1, mla.decode_workspace_size(B, P, H, max_len, args.num_splits)),
                            dtype=torch.uint8, device=dev)
    sigma = w.softmax_scale
    launches = [mla.verify_launcher(q, kv, bt, sl, softmax_scale=sigma, kv_scale=cache.kv_scale,
                                    max_kv_len=max_len, out=out, lse=lse, workspace=workspace,
                                    num_splits=args.num_splits) for kv in pools]

    def step(i):
        launches[i % len(launches)]()

    # parity on the timed buffers (every pool) before timing
    import oracle
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(5).choice(N, 30, False)]))
    ref_o, ref_l = oracle.decode(q_np, cache.kv, True, cache.kv_scale, cache.block_table,
                                 cache.seq_lens, sigma, rows=rows.astype(np.int64))
    idx = torch.from_numpy(rows).to(dev)
    for i in range(len(pools)):
        step(i)
        torch.cuda.synchronize()
        check_out(out.reshape(N, 512)[idx], ref_o, "decode out (pool %d)" % i)
        check_lse(lse.reshape(N)[idx], ref_l, "decode lse (pool %d)" % i)
    log("parity ok on %d sampled rows, %d pools, %d pieces" % (len(rows), len(pools), W))

    alg_bytes = acc.decode_bytes(L, P, H, "fp8", out_bytes=4, block_size=cache.block_size)
    alg_flops = acc.decode_flops(L, P, H)

    for i in range(args.warmup):
        step(i)
    # Timed region: the K steps back to back between two events on the stream the
    # library launches on (torch's current stream), bracketed by synchronisations;
    # the kernel's average launch duration is the region over K (inter-launch gaps
    # included).
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    r0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    r1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_avg_ms = r0.elapsed_time(r1) / args.steps
    # per-call spread from a second pass with an event pair around every call (each
    # pair adds its own few microseconds)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for i in range(args.steps):
        e0, e1 = ev[i]
        e0.record(stream)
        step(i)
        e1.record(stream)
    torch.cuda.synchronize()
    kern_ms = np.array([a.elapsed_time(b) for a, b in ev])
    ms_per_step = wall * 1e3 / args.steps
    value = alg_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = alg_bytes / (kern_avg_ms * 1e-3) / 1e9
    traffic = traffic_from_profile("mla_decode.hip", DECODE_WORKLOAD)
    log("decode: %.1f us/step wall, kernel %.1f us back to back (per call with events: p10 %.1f,"
        " p90 %.1f)" % (ms_per_step * 1e3, kern_avg_ms * 1e3, np.percentile(kern_ms, 10) * 1e3,
                        np.percentile(kern_ms, 90) * 1e3))

    ceiling = read_ceiling_gbs(torch, stream, alg_bytes, len(pools))
    log("plain read of the same %d bytes: %.0f GB/s (best of grids %s)"
        % (alg_bytes, ceiling["gbs"], ceiling["grids"]))

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 kv / bf16 q / fp32 accumulate",
        "data": "synthetic (seeded N(0,1), FP8 E4M3 per-tensor scale, shuffled 64-token pages)",
        "config": {"workload": DECODE_WORKLOAD, "batch": B, "heads": H, "query_positions": P,
                   "context": "uniform [4096, 16384]", "total_keys": int(sum(L)),
                   "kv_dtype": "fp8_e4m3", "block_size": cache.block_size, "pieces": W,
                   "kv_pool_copies": len(pools), "algorithmic_bytes": alg_bytes,
                   "algorithmic_flops": alg_flops},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "decode_kernel<fp8>",
                     "kernel_us": round(float(kern_avg_ms) * 1e3, 2),
                     "kernel_us_per_call_p10_p50_p90":
                         [round(float(np.percentile(kern_ms, q)) * 1e3, 2)
                                               for q in (10, 50, 90)],
                     # context, not the peak: a kernel that only reads the same bytes
                     "read_ceiling": {"gbs": round(ceiling["gbs"], 1),
                                      "us": round(ceiling["us"], 2),
                                      "frac_of_peak": round(ceiling["gbs"] / HBM_PEAK_GBS, 4),
                                      "achieved_over_ceiling":
                                          round(achieved / ceiling["gbs"], 4),
                                      "kernel": "read_probe_kernel (libmla_read_probe.so)"}},
    }

    # ---------------- prefill (the metric's second half) ----------------
    if not args.no_prefill:
        run_prefill(args, torch, mi, mla, acc, oracle, bf16_tensor, check_out, check_lse, dev,
                    stream, result)

    if not args.no_secondary:
        result["secondary"] = secondary_configs(torch, mi, mla, acc, oracle, bf16_tensor,
                                                cache_to_device, check_out, check_lse, dev,
                                                stream, only=set(args.secondary.split(","))
                                                if args.secondary else None)
    result["clocks"] = gpu_clocks()

    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(q_np, cache, alg_bytes)
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
