"""HIP-graph capture and replay of the entry points, through the Python binding.

The pages measured the short verify as a graph-replayed kernel test (one sequence, four
verify positions: "Scaling Kimi K3 on AMD Instinct MI355X", section
"并行度必须适配真正的形状").  Every entry point here is asynchronous on the caller's
stream and never synchronises, so it can be captured: mla_verify with the shares merged in
the launch and with the separate merge launch, mla_prefill and mla_merge_lse are captured
into one graph (the binding's own calls, with the host hints given so that nothing reads
device memory back during capture).  The graph is replayed several times with eager
library work and a synchronisation between replays, and every replay is compared with
the oracle and bitwise with the eager call.
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


@pytest.fixture(scope="module")
def mla():
    import mla_latent_kv_attention_amd as m
    m.library()
    assert torch.cuda.is_available()
    return m


def test_graph_replay_of_every_entry_point(mla):
    # verify: 3 sequences x 4 positions x 12 heads over an FP8 paged cache
    lens = [37, 700, 2100]
    cache = mi.paged_cache(7101, lens, 64, "fp8")
    q_np = mi.normal_bf16_bits(7101, 3, (3, 4, 12, 576))
    kv, bt, sl = cache_to_device(cache, DEV)
    q = bf16_tensor(q_np, DEV)
    in_launch, separate = 20, 100  # <= 16 and > 16 pieces per sequence
    ws = {s: torch.zeros(mla.decode_workspace_size(3, 4, 12, 2100, s), dtype=torch.uint8,
                         device=DEV) for s in (in_launch, separate)}
    ref_vo, ref_vl = oracle.decode(q_np, cache.kv, True, cache.kv_scale, cache.block_table,
                                   cache.seq_lens, SIGMA)
    # prefill: two packed sequences, BF16 out
    pd = mi.prefill_inputs(mi.PrefillWorkload("graph", [150, 41], 12, "bf16", seed=7102))
    pq, pkv, pcu = bf16_tensor(pd["q"], DEV), bf16_tensor(pd["kv"], DEV), i32(pd["cu_seqlens"], DEV)
    ref_po, ref_pl = oracle.prefill(pd["q"], pd["kv"], False, 1.0, pd["cu_seqlens"], SIGMA)
    # the same prefill over an FP8 cache (its tiles staged in LDS as codes)
    pd8 = mi.prefill_inputs(mi.PrefillWorkload("graph8", [150, 41], 12, "fp8", seed=7105))
    pq8, pkv8, pcu8 = bf16_tensor(pd8["q"], DEV), torch.from_numpy(pd8["kv"]).to(DEV), i32(pd8["cu_seqlens"], DEV)
    ref_po8, ref_pl8 = oracle.prefill(pd8["q"], pd8["kv"], True, pd8["kv_scale"], pd8["cu_seqlens"], SIGMA)
    # merge: 6 partials of 40 rows, one row with no keys anywhere
    rng = np.random.default_rng(7103)
    po_np = rng.standard_normal((6, 40, 512)).astype(np.float32)
    pl_np = (rng.standard_normal((6, 40)) * 3).astype(np.float32)
    pl_np[:, 7] = -np.inf
    po, pl = torch.from_numpy(po_np).to(DEV), torch.from_numpy(pl_np).to(DEV)
    ref_mo, ref_ml = oracle.merge(po_np.astype(np.float64), pl_np.astype(np.float64))

    def calls():
        r = {}
        for s in (in_launch, separate):
            r["verify%d" % s] = mla.verify(q, kv, bt, sl, softmax_scale=SIGMA,
                                           kv_scale=cache.kv_scale, max_kv_len=2100,
                                           num_splits=s, workspace=ws[s])
        r["prefill"] = mla.prefill(pq, pkv, pcu, softmax_scale=SIGMA, max_seqlen=150)
        r["prefill8"] = mla.prefill(pq8, pkv8, pcu8, softmax_scale=SIGMA, kv_scale=pd8["kv_scale"],
                                    max_seqlen=150)
        r["merge"] = mla.merge_lse(po, pl)
        return r

    def check(r, what):
        for s in (in_launch, separate):
            o, l = r["verify%d" % s]
            check_out(o, ref_vo, "%s verify (%d pieces) out" % (what, s))
            check_lse(l, ref_vl, "%s verify (%d pieces) lse" % (what, s))
        check_out(r["prefill"][0], ref_po, what + " prefill out")
        check_lse(r["prefill"][1], ref_pl, what + " prefill lse")
        check_out(r["prefill8"][0], ref_po8, what + " fp8 prefill out")
        check_lse(r["prefill8"][1], ref_pl8, what + " fp8 prefill lse")
        check_out(r["merge"][0], ref_mo, what + " merge out")
        check_lse(r["merge"][1], ref_ml, what + " merge lse")

    eager = calls()
    torch.cuda.synchronize()
    check(eager, "eager")
    eager = {k: (o.clone(), l.clone()) for k, (o, l) in eager.items()}

    side = torch.cuda.Stream(DEV)  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the stream the capture uses
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        captured = calls()

    other_cache = mi.paged_cache(7104, [300, 5], 64, "bf16")
    okv, obt, osl = cache_to_device(other_cache, DEV)
    oq = bf16_tensor(mi.normal_bf16_bits(7104, 3, (2, 1, 8, 576)), DEV)
    for rep in range(4):
        print("replay", rep, flush=True)
        for o, l in captured.values():
            o.fill_(float("nan"))
            l.fill_(float("nan"))
        # eager library work between replays (its own workspace, same kernels)
        mla.verify(oq, okv, obt, osl, softmax_scale=SIGMA, max_kv_len=300)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(captured, "replay %d" % rep)
        for k, (o, l) in captured.items():
            assert torch.equal(o, eager[k][0]) and torch.equal(l, eager[k][1]), k
    # every call left the workspace counters zero
    for s in (in_launch, separate):
        assert torch.all(ws[s][:65536 * 4].view(torch.int32) == 0)
