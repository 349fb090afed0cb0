"""The C-ABI library on the CPU: it loads, exports every symbol include/mla.h declares,
and its host-side logic (argument checks, split planner, workspace sizing) behaves as
documented.  No compute call is made here: every call below is rejected, or returns,
before anything is launched."""
import ctypes
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")


@pytest.fixture(scope="module")
def lib():
    import mla_latent_kv_attention_amd as m
    if not os.path.exists(m.LIB_PATH):
        from mla_latent_kv_attention_amd import build
        build.build()
    return m.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["mla_decode", "mla_verify", "mla_prefill", "mla_merge_lse", "mla_cache_write",
              "mla_top_k_renorm_prob", "mla_top_k_renorm_workspace_size",
              "mla_decode_workspace_size", "mla_decode_num_splits", "mla_status_string",
              "mla_version"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert lib.mla_status_string(0) == b"ok"
    assert lib.mla_status_string(-3).startswith(b"workspace")
    assert lib.mla_version() >= 100


NULL = None


def verify_args(**over):
    a = dict(q=1, kv=1, kv_dtype=0, kv_scale=1.0, bt=1, max_blocks=4, block_size=64, sl=1,
             kb=None, ke=None, B=2, P=1, H=12, max_kv_len=100, scale=0.07, out=1, out_dtype=2,
             lse=None, splits=0, ws=None, ws_bytes=0, stream=None)
    a.update(over)
    # non-null pointers are never dereferenced: every call here fails a host check first
    p = lambda v: None if v is None else ctypes.c_void_p(0x1000)
    return [p(a["q"]), p(a["kv"]), a["kv_dtype"], a["kv_scale"], p(a["bt"]), a["max_blocks"],
            a["block_size"], p(a["sl"]), p(a["kb"]), p(a["ke"]), a["B"], a["P"], a["H"],
            a["max_kv_len"], a["scale"], p(a["out"]), a["out_dtype"], p(a["lse"]), a["splits"],
            p(a["ws"]), a["ws_bytes"], a["stream"]]


@pytest.mark.parametrize("over,status", [
    (dict(P=0), -1),
    (dict(H=0), -1),
    (dict(B=-1), -1),
    (dict(splits=-2), -1),
    (dict(max_kv_len=-5), -1),
    (dict(P=257, H=256), -2),       # more query rows per sequence than MLA_MAX_CALL_ROWS
    (dict(kv_dtype=7), -2),
    (dict(out_dtype=1), -2),        # FP8 is a cache format, not an output format
    (dict(block_size=24), -1),
    (dict(block_size=0), -1),
    (dict(max_blocks=0), -1),
    (dict(kv_dtype=1, kv_scale=0.0), -1),
    (dict(kv_dtype=1, kv_scale=float("inf")), -1),
    (dict(scale=float("nan")), -1),
    (dict(q=None), -1),
    (dict(kv=None), -1),
    (dict(bt=None), -1),
    (dict(sl=None), -1),
    (dict(out=None), -1),
])
def test_verify_rejects_bad_arguments_before_launch(lib, over, status):
    assert lib.mla_verify(*verify_args(**over)) == status


@pytest.mark.parametrize("over,status", [
    (dict(P=0), -1), (dict(H=0), -1), (dict(B=-1), -1), (dict(P=257, H=256), -2),
    (dict(kv_dtype=7), -2), (dict(out_dtype=1), -2), (dict(block_size=24), -1),
    (dict(kv_dtype=1, kv_scale=0.0), -1), (dict(out=None), -1),
])
def test_noalloc_verify_rejects_bad_arguments_before_launch(lib, over, status):
    """mla_verify_noalloc takes mla_verify's arguments minus the workspace and checks them
    the same way, before any launch."""
    a = verify_args(**over)
    args = a[:19] + [a[21]]  # drop workspace and workspace_bytes
    lib.mla_verify_noalloc.restype = ctypes.c_int
    assert lib.mla_verify_noalloc(*args) == status


def test_empty_batch_is_a_no_op(lib):
    assert lib.mla_verify(*verify_args(B=0, q=None, kv=None, bt=None, sl=None, out=None)) == 0


def test_merge_rejects_bad_arguments(lib):
    P = ctypes.c_void_p(0x1000)
    assert lib.mla_merge_lse(P, P, 0, 4, P, 2, None, None) == -1
    assert lib.mla_merge_lse(P, P, 2, -1, P, 2, None, None) == -1
    assert lib.mla_merge_lse(P, P, 2, 4, P, 1, None, None) == -2
    assert lib.mla_merge_lse(None, P, 2, 4, P, 2, None, None) == -1
    assert lib.mla_merge_lse(None, None, 2, 0, None, 2, None, None) == 0


def test_cache_write_rejects_bad_arguments(lib):
    P = ctypes.c_void_p(0x1000)
    lib.mla_cache_write.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_long,
                                    ctypes.c_void_p]
    assert lib.mla_cache_write(P, -1, P, P, 1, 0.01, 64, None) == -1
    assert lib.mla_cache_write(P, 4, P, P, 2, 0.01, 64, None) == -2   # FP32 is no cache dtype
    assert lib.mla_cache_write(P, 4, P, P, 1, 0.0, 64, None) == -1    # FP8 needs a scale > 0
    assert lib.mla_cache_write(None, 4, P, P, 1, 0.01, 64, None) == -1
    assert lib.mla_cache_write(P, 4, None, P, 0, 1.0, 64, None) == -1
    assert lib.mla_cache_write(None, 0, None, None, 0, 1.0, 0, None) == 0


def test_top_k_renorm_rejects_bad_arguments_and_sizes_its_workspace(lib):
    P = ctypes.c_void_p(0x1000)
    ws = lib.mla_top_k_renorm_workspace_size
    # 8,192-entry chunks, 2,048 candidates of 8 bytes each per chunk, then one float
    # per chunk; both parts 256-byte aligned
    up = lambda x: (x + 255) // 256 * 256
    assert ws(128, 163840) == up(128 * 20 * 2048 * 8) + up(128 * 20 * 4)
    assert ws(3, 16385) == up(3 * 3 * 2048 * 8) + up(3 * 3 * 4)
    assert ws(0, 1000) == 0 and ws(4, 0) == 0
    f = lib.mla_top_k_renorm_prob
    need = ws(4, 1000)
    assert f(P, P, -1, 1000, P, P, need, None) == -1
    assert f(P, P, 4, 0, P, P, need, None) == -1
    assert f(None, P, 4, 1000, P, P, need, None) == -1
    assert f(P, None, 4, 1000, P, P, need, None) == -1
    assert f(P, P, 4, 1000, None, P, need, None) == -1
    assert f(P, P, 4, 1000, P, None, need, None) == -3
    assert f(P, P, 4, 1000, P, P, need - 1, None) == -3
    assert f(P, P, 4, 1000, P, ctypes.c_void_p(0x1004), need, None) == -3  # not 8-byte aligned
    assert f(None, None, 0, 0, None, None, 0, None) == 0


def test_prefill_rejects_bad_arguments(lib):
    P = ctypes.c_void_p(0x1000)
    assert lib.mla_prefill(P, P, 0, 1.0, P, 1, 16, 16, 0, 0.07, P, 0, None, None) == -1
    assert lib.mla_prefill(P, P, 0, 1.0, P, 1, 16, 16, 1 << 28, 0.07, P, 0, None, None) == -2
    assert lib.mla_prefill(P, P, 3, 1.0, P, 1, 16, 16, 12, 0.07, P, 0, None, None) == -2
    assert lib.mla_prefill(P, P, 1, -1.0, P, 1, 16, 16, 12, 0.07, P, 0, None, None) == -1
    assert lib.mla_prefill(None, P, 0, 1.0, P, 1, 16, 16, 12, 0.07, P, 0, None, None) == -1
    assert lib.mla_prefill(None, None, 0, 1.0, None, 0, 0, 0, 12, 0.07, None, 0, None, None) == 0


def test_planner_fills_the_chip_for_the_short_verify_shape(lib):
    """The pages' short verify: one sequence, 4 positions, 12 heads; 48 work-groups were
    too few for the chip.  The persistent plan launches more than that, never more than
    one per CU, once the history is long enough.  One work-group serves all of a piece's
    row blocks, so the grid is the piece count."""
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_closed_forms.json")))
    sv = g["short_verify_workgroups"]
    heads = sv["heads"]
    assert heads * sv["tiled_width"] // sv["wide_tile_columns"] == sv["wide_tile_workgroups"]
    assert heads * sv["tiled_width"] // sv["narrow_tile_columns"] == sv["narrow_tile_workgroups"]
    rows = 4 * heads
    row_blocks = -(-rows // 16)
    for cus in [256, 304]:
        for ctx in [16384, 32768, 142000]:
            W = lib.mla_decode_num_splits(1, 4, heads, ctx, 0, cus)
            grid = W if ctx >= 65536 else W * row_blocks  # one work-group per piece / per row block
            assert grid <= cus
            assert grid > sv["wide_tile_workgroups"]


@pytest.mark.parametrize("B,P,H,L", [(1, 1, 12, 1024), (32, 1, 12, 16384), (4, 4, 12, 32768),
                                     (4, 4, 16, 32768), (8, 1, 12, 17750), (3, 2, 8, 64),
                                     (1, 1, 12, 16), (0, 1, 12, 0), (1, 4, 12, 32768),
                                     (2, 4, 12, 32768), (1, 4, 12, 65536)])
def test_planner_pieces_fit_the_chip_and_the_work(lib, B, P, H, L):
    """At most one work-group per CU, at least two 16-token steps per piece (as far as the
    max_kv_len hint tells), and as many pieces as both allow.  The grid is one work-group
    per (piece, 16-row block), or one per piece for sequences of several row blocks over
    a batch key range of at least 65,536 tokens (one work-group serves all row blocks)."""
    RB = -(-(P * H) // 16)
    shared = RB >= 2 and max(B, 1) * L >= 65536
    for cus in [80, 256, 304]:
        W = lib.mla_decode_num_splits(B, P, H, L, 0, cus)
        steps = max(B, 1) * (-(-L // 16))
        per_piece = 1 if shared else RB
        want = max(1, min(cus // per_piece, -(-steps // 2)))
        assert W == want
        assert W * per_piece <= cus


@pytest.mark.parametrize("B,P,H,L,S", [(32, 1, 12, 16384, 0), (4, 4, 12, 32768, 0),
                                       (2, 3, 5, 100, 7), (1, 1, 12, 16, 0)])
def test_workspace_holds_slots_and_counters(lib, B, P, H, L, S):
    """A fixed block of 65536 counters and a 256-byte error-flags block first (the same
    bytes for every shape), then (W + B) x rows partial outputs and lse, then each
    sequence's piece range, each part 256-byte aligned; nothing for a single piece."""
    W = lib.mla_decode_num_splits(B, P, H, L, S, 0)  # the plan the workspace query uses
    R = P * H
    al = lambda x: -(-x // 256) * 256
    want = 0 if W <= 1 else (65536 * 4 + 256 + al((W + B) * R * 512 * 4) + al((W + B) * R * 4)
                             + al(2 * B * 4))
    assert lib.mla_decode_workspace_size(B, P, H, L, S) == want


def test_counter_capacity_is_enforced(lib):
    """B x ceil(P*H/16) above the counter block's 65536 entries needs the single-piece
    plan; any other piece count is rejected before the device is queried."""
    assert lib.mla_verify(*verify_args(B=65537, H=12, splits=0)) == -2
    assert lib.mla_verify(*verify_args(B=32769, H=17, splits=3)) == -2
    assert lib.mla_verify(*verify_args(B=32768, H=17, splits=3, ws=None)) != -2


def test_explicit_split_count_is_honoured(lib):
    assert lib.mla_decode_num_splits(2, 1, 12, 1000, 7, 256) == 7
    assert lib.mla_decode_num_splits(2, 1, 12, 10, 3, 256) == 3
    assert lib.mla_decode_num_splits(2, 5, 16, 10, 3, 256) == 3  # each row group's plan
    assert lib.mla_decode_num_splits(2, 257, 256, 10, 3, 256) == -2


@pytest.mark.parametrize("B,P,H,L,S,groups", [
    (2, 5, 16, 1000, 0, [(4, 16), (1, 16)]),     # whole positions: 4 per group
    (3, 1, 128, 5000, 0, [(1, 64)]),             # 64-head slices of one position
    (1, 3, 100, 40000, 0, [(1, 64), (1, 36)]),   # slices of 64 and 36 heads, per position
    (4, 9, 8, 20000, 12, [(8, 8), (1, 8)]),
    (2, 65, 1, 300, 0, [(64, 1), (1, 1)])])
def test_row_groups_share_one_workspace(lib, B, P, H, L, S, groups):
    """More than 64 query rows per sequence run as groups of at most 64 rows, one launch
    each over the same workspace: the call needs what its largest group shape needs,
    and its piece count is the first group's."""
    want = max(lib.mla_decode_workspace_size(B, gp, gh, L, S) for gp, gh in groups)
    assert lib.mla_decode_workspace_size(B, P, H, L, S) == want
    gp, gh = groups[0]
    assert lib.mla_decode_num_splits(B, P, H, L, S, 256) == \
        lib.mla_decode_num_splits(B, gp, gh, L, S, 256)


def test_read_probe_rejects_bad_arguments_before_launch():
    """The benchmark's measurement helper (its own library, not the attention boundary):
    null pointers, a size or address not a multiple of 16 and grids outside 1 .. 65536
    are refused; an empty read launches nothing."""
    from mla_latent_kv_attention_amd import read_probe
    if not os.path.exists(read_probe.LIB_PATH):
        from mla_latent_kv_attention_amd import build
        build.build()
    lib = read_probe.library()
    P = ctypes.c_void_p(0x1000)
    assert lib.mla_hbm_read_probe(None, 16, P, 1, None) == -1
    assert lib.mla_hbm_read_probe(P, 16, None, 1, None) == -1
    assert lib.mla_hbm_read_probe(P, 17, P, 1, None) == -1
    assert lib.mla_hbm_read_probe(ctypes.c_void_p(0x1008), 16, P, 1, None) == -1
    assert lib.mla_hbm_read_probe(P, 16, P, 0, None) == -1
    assert lib.mla_hbm_read_probe(P, 16, P, 65537, None) == -1
    assert lib.mla_hbm_read_probe(P, 0, P, 4, None) == 0


def test_attention_library_does_not_export_the_probe(lib):
    assert not hasattr(lib, "mla_hbm_read_probe")


def test_phase_stamps_only_in_the_timeline_library(lib):
    """The attention library has the stamps compiled out; libmla_timeline.so (the same
    sources built with MLA_TIMELINE, loaded only by `bench.py --timeline`) exports their
    readers and every entry point of the attention library."""
    import mla_latent_kv_attention_amd as m
    for fn in ("mla_timeline_read_decode", "mla_timeline_read_verify"):
        assert not hasattr(lib, fn)
    path = os.path.join(os.path.dirname(m.LIB_PATH), "libmla_timeline.so")
    if not os.path.exists(path):
        pytest.skip("libmla_timeline.so is not built")
    tl = ctypes.CDLL(path)
    for fn in ("mla_timeline_read_decode", "mla_timeline_read_verify", "mla_verify",
               "mla_verify_noalloc", "mla_prefill", "mla_decode_workspace_size"):
        assert hasattr(tl, fn), fn
