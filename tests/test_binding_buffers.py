"""The Python binding rejects caller-supplied buffers the kernels would write past or
misread, before anything reaches the library: wrong shape, dtype, device or layout of
out / lse / workspace, and batch arrays whose length is not the batch.  CPU tensors stand
in for device tensors here; every call below raises before the C-ABI is called."""
import pytest
import torch

import mla_latent_kv_attention_amd as mla

CPU = torch.device("cpu")


def verify_inputs(B=2, P=4, H=12, kv_dtype=torch.bfloat16):
    q = torch.zeros((B, P, H, 576), dtype=torch.bfloat16)
    kv = torch.zeros((8, 64, 576), dtype=kv_dtype)
    bt = torch.zeros((B, 4), dtype=torch.int32)
    sl = torch.full((B,), 100, dtype=torch.int32)
    return q, kv, bt, sl


@pytest.fixture(scope="module", autouse=True)
def lib():
    import os
    if not os.path.exists(mla.LIB_PATH):
        from mla_latent_kv_attention_amd import build
        build.build()
    return mla.library()


@pytest.mark.parametrize("out", [
    torch.zeros((2, 4, 12, 512), dtype=torch.bfloat16),       # bf16 buffer, fp32 requested
    torch.zeros((2, 4, 12, 256), dtype=torch.float32),        # half the width
    torch.zeros((2, 4, 11, 512), dtype=torch.float32),        # one head short
    torch.zeros((2, 4, 12, 1024), dtype=torch.float32)[..., ::2],  # strided view
])
def test_verify_rejects_mismatched_out(out):
    q, kv, bt, sl = verify_inputs()
    with pytest.raises(TypeError, match="out"):
        mla.verify(q, kv, bt, sl, softmax_scale=0.07, max_kv_len=100, out=out)


@pytest.mark.parametrize("lse", [
    torch.zeros((2, 4, 12), dtype=torch.bfloat16),
    torch.zeros((2, 4, 6), dtype=torch.float32),
    torch.zeros((2, 4, 24), dtype=torch.float32)[..., ::2],
])
def test_verify_rejects_mismatched_lse(lse):
    q, kv, bt, sl = verify_inputs()
    with pytest.raises(TypeError, match="lse"):
        mla.verify(q, kv, bt, sl, softmax_scale=0.07, max_kv_len=100, lse=lse)


def test_verify_rejects_bf16_out_with_fp32_out_dtype_and_the_reverse():
    q, kv, bt, sl = verify_inputs()
    with pytest.raises(TypeError, match="out"):
        mla.verify(q, kv, bt, sl, softmax_scale=0.07, max_kv_len=100, out_dtype=torch.bfloat16,
                   out=torch.zeros((2, 4, 12, 512), dtype=torch.float32))


def test_verify_rejects_short_batch_arrays_and_bad_workspace():
    q, kv, bt, sl = verify_inputs()
    with pytest.raises(TypeError, match="seq_lens"):
        mla.verify(q, kv, bt, sl[:1], softmax_scale=0.07, max_kv_len=100)
    with pytest.raises(TypeError, match="block_table"):
        mla.verify(q, kv, bt[:1], sl, softmax_scale=0.07, max_kv_len=100)
    with pytest.raises(TypeError, match="kv_end"):
        mla.verify(q, kv, bt, sl, softmax_scale=0.07, max_kv_len=100,
                   kv_end=torch.zeros((3,), dtype=torch.int32))
    with pytest.raises(TypeError, match="workspace"):
        mla.verify(q, kv, bt, sl, softmax_scale=0.07, max_kv_len=100,
                   workspace=torch.zeros(1 << 20, dtype=torch.int32))


def test_verify_launcher_checks_out_and_lse():
    q, kv, bt, sl = verify_inputs()
    with pytest.raises(TypeError, match="out"):
        mla.verify_launcher(q, kv, bt, sl, softmax_scale=0.07, max_kv_len=100,
                            out=torch.zeros((2, 4, 12, 500), dtype=torch.float32), lse=None,
                            workspace=None)
    with pytest.raises(TypeError, match="lse"):
        mla.verify_launcher(q, kv, bt, sl, softmax_scale=0.07, max_kv_len=100,
                            out=torch.zeros((2, 4, 12, 512), dtype=torch.float32),
                            lse=torch.zeros((2, 4, 12), dtype=torch.float64), workspace=None)


def test_decode_rejects_mismatched_out_and_lse():
    q = torch.zeros((3, 12, 576), dtype=torch.bfloat16)
    kv = torch.zeros((8, 64, 576), dtype=torch.uint8)
    bt = torch.zeros((3, 4), dtype=torch.int32)
    sl = torch.full((3,), 100, dtype=torch.int32)
    with pytest.raises(TypeError, match="out"):
        mla.decode(q, kv, bt, sl, softmax_scale=0.07, max_kv_len=100,
                   out=torch.zeros((3, 12, 512), dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="lse"):
        mla.decode(q, kv, bt, sl, softmax_scale=0.07, max_kv_len=100,
                   lse=torch.zeros((3, 11), dtype=torch.float32))


def test_prefill_rejects_mismatched_out_and_lse():
    q = torch.zeros((40, 12, 576), dtype=torch.bfloat16)
    kv = torch.zeros((40, 576), dtype=torch.bfloat16)
    cu = torch.tensor([0, 40], dtype=torch.int32)
    with pytest.raises(TypeError, match="out"):   # prefill's default out dtype is bf16
        mla.prefill(q, kv, cu, softmax_scale=0.07, out=torch.zeros((40, 12, 512)))
    with pytest.raises(TypeError, match="out"):
        mla.prefill(q, kv, cu, softmax_scale=0.07, out_dtype=torch.float32,
                    out=torch.zeros((40, 12, 256)))
    with pytest.raises(TypeError, match="lse"):
        mla.prefill(q, kv, cu, softmax_scale=0.07, lse=torch.zeros((40, 12), dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="kv"):
        mla.prefill(q, kv[:39], cu, softmax_scale=0.07)


def test_merge_lse_rejects_mismatched_out_and_lse():
    po = torch.zeros((3, 10, 512), dtype=torch.float32)
    pl = torch.zeros((3, 10), dtype=torch.float32)
    with pytest.raises(TypeError, match="out"):
        mla.merge_lse(po, pl, out=torch.zeros((10, 512), dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="out"):
        mla.merge_lse(po, pl, out=torch.zeros((9, 512), dtype=torch.float32))
    with pytest.raises(TypeError, match="lse"):
        mla.merge_lse(po, pl, lse=torch.zeros((10, 2), dtype=torch.float32))


def test_workspace_flags_are_read_reported_and_cleared_on_the_host():
    """The binding's side of the error-flags word: a workspace whose flags word is set
    raises WorkspaceError naming the cause, and comes back with its counters and flags
    zeroed; a clean workspace passes."""
    ws = torch.zeros(mla.WORKSPACE_FLAGS_OFFSET + 4096, dtype=torch.uint8)
    mla.check_decode_workspace(ws)  # clean
    ws[:64] = 7                     # stale counters
    ws[mla.WORKSPACE_FLAGS_OFFSET:mla.WORKSPACE_FLAGS_OFFSET + 4].view(torch.int32)[0] = \
        mla.FLAG_STALE_COUNTERS | mla.FLAG_BAD_LENGTHS
    ws[mla.WORKSPACE_FLAGS_OFFSET + 8:] = 9  # partial results: left alone
    with pytest.raises(mla.WorkspaceError) as e:
        mla.check_decode_workspace(ws)
    assert e.value.flags == 3 and "counters" in str(e.value) and "length" in str(e.value)
    assert torch.all(ws[:mla.WORKSPACE_FLAGS_OFFSET + 4] == 0)
    assert torch.all(ws[mla.WORKSPACE_FLAGS_OFFSET + 8:] == 9)
    mla.check_decode_workspace(ws)


def test_flags_offset_matches_the_header():
    import os
    import re
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "include", "mla.h")).read()
    assert re.search(r"#define MLA_WORKSPACE_FLAGS_OFFSET \(4 \* MLA_MAX_COUNTERS\)", hdr)
    assert re.search(r"#define MLA_MAX_COUNTERS 65536", hdr)
    assert re.search(r"#define MLA_FLAG_STALE_COUNTERS 1\b", hdr)
    assert re.search(r"#define MLA_FLAG_BAD_LENGTHS 2\b", hdr)
    assert mla.WORKSPACE_FLAGS_OFFSET == 4 * 65536
