"""MLA over a compressed latent KV cache on MI355X (gfx950): Python binding.

A thin ctypes layer over ``libmla.so`` (the C-ABI declared in ``include/mla.h``).
It only marshals arguments: PyTorch supplies device memory and the current HIP
stream; every step of the attention runs in the library's HIP kernels.  There is
no other implementation behind these functions: if the library is missing they
raise instead of computing anything.

Entry points (same names as the C-ABI):
  decode(q, kv_cache, block_table, seq_lens, ...)   one query position per sequence
  verify(q, kv_cache, block_table, seq_lens, ...)   P query positions, causal among them
  prefill(q, kv, cu_seqlens, ...)                   causal attention of packed sequences
  merge_lse(part_out, part_lse, ...)                merge partials by log-sum-exp
  cache_write(latent, kv_cache, slot_mapping, ...)  quantise / copy new rows into cache slots
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

HEAD_DIM_K = 576
HEAD_DIM_V = 512
MAX_ROWS = 64  # query rows per sequence one kernel launch takes; calls group larger P x H
MAX_CALL_ROWS = 65536  # query rows (P x H) per sequence a decode / verify call accepts

DTYPE_BF16 = 0
DTYPE_FP8_E4M3 = 1
DTYPE_FP32 = 2

_STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported shape or dtype",
           -3: "workspace missing or too small", -4: "HIP launch or query failed",
           -5: "needs more than the no-allocation entry point's scratch"}


class MlaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s failed: %s (status %d)" % (fn, _STATUS.get(status, "?"), status))
        self.status = status


_lib = None


def library() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                "libmla.so is not built (%s); run mla_latent_kv_attention_amd/build.py" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.mla_verify.restype = I
        lib.mla_verify.argtypes = [P, P, I, F, P, I, I, P, P, P, I, I, I, I, F, P, I, P, I, P, Z, P]
        lib.mla_verify_noalloc.restype = I
        lib.mla_verify_noalloc.argtypes = [P, P, I, F, P, I, I, P, P, P, I, I, I, I, F, P, I, P, I,
                                           P]
        lib.mla_decode.restype = I
        lib.mla_decode.argtypes = [P, P, I, F, P, I, I, P, P, P, I, I, I, F, P, I, P, I, P, Z, P]
        lib.mla_prefill.restype = I
        lib.mla_prefill.argtypes = [P, P, I, F, P, I, I, I, I, F, P, I, P, P]
        lib.mla_cache_write.restype = I
        lib.mla_cache_write.argtypes = [P, ctypes.c_long, P, P, I, F, ctypes.c_long, P]
        lib.mla_merge_lse.restype = I
        lib.mla_merge_lse.argtypes = [P, P, I, I, P, I, P, P]
        lib.mla_decode_workspace_size.restype = Z
        lib.mla_decode_workspace_size.argtypes = [I, I, I, I, I]
        lib.mla_decode_num_splits.restype = I
        lib.mla_decode_num_splits.argtypes = [I, I, I, I, I, I]
        lib.mla_top_k_renorm_prob.restype = I
        lib.mla_top_k_renorm_prob.argtypes = [P, P, I, I, P, P, Z, P]
        lib.mla_top_k_renorm_workspace_size.restype = Z
        lib.mla_top_k_renorm_workspace_size.argtypes = [I, I]
        lib.mla_status_string.restype = ctypes.c_char_p
        lib.mla_status_string.argtypes = [I]
        lib.mla_version.restype = I
        lib.mla_version.argtypes = []
        _lib = lib
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _check(fn: str, status: int):
    if status != 0:
        raise MlaError(fn, status)


def _kv_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return DTYPE_FP8_E4M3
    raise TypeError("kv cache must be bfloat16, uint8 or float8_e4m3fn (FP8 E4M3FN codes)")


def _out_dtype(d: torch.dtype) -> int:
    if d == torch.float32:
        return DTYPE_FP32
    if d == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")


def _dev_i32(t: Optional[torch.Tensor], name: str, dev: torch.device):
    if t is None:
        return None
    if t.dtype != torch.int32 or t.device != dev or not t.is_contiguous():
        raise TypeError("%s must be a contiguous int32 tensor on %s" % (name, dev))
    return t


def _out_buffer(t: Optional[torch.Tensor], name: str, shape, dtype: torch.dtype,
                dev: torch.device) -> Optional[torch.Tensor]:
    """A caller-supplied output buffer must be exactly what the kernels write: contiguous,
    on the inputs' device, of the stated shape and dtype (a smaller or narrower buffer
    would be written past its end)."""
    if t is None:
        return None
    if (tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != dev
            or not t.is_contiguous()):
        raise TypeError("%s must be a contiguous %s tensor of shape %s on %s (got %s %s on %s%s)"
                        % (name, dtype, tuple(shape), dev, t.dtype, tuple(t.shape), t.device,
                           "" if t.is_contiguous() else ", not contiguous"))
    return t


def _workspace_buffer(t: Optional[torch.Tensor], dev: torch.device) -> Optional[torch.Tensor]:
    if t is None:
        return None
    if t.dtype != torch.uint8 or t.device != dev or not t.is_contiguous():
        raise TypeError("workspace must be a contiguous uint8 tensor on %s" % dev)
    return t


def _check_batch_arrays(B: int, block_table, seq_lens, kv_begin, kv_end):
    if block_table.dim() != 2 or block_table.shape[0] != B or block_table.shape[1] < 1:
        raise TypeError("block_table must be [B, max_blocks_per_seq] with B = %d" % B)
    for name, t in (("seq_lens", seq_lens), ("kv_begin", kv_begin), ("kv_end", kv_end)):
        if t is not None and tuple(t.shape) != (B,):
            raise TypeError("%s must be [B] with B = %d" % (name, B))


def decode_num_splits(B: int, P: int, H: int, max_kv_len: int, num_splits: int = 0,
                      num_cus: int = 0) -> int:
    """Pieces the batch's key steps are divided into (num_cus = 0: the current device)."""
    return library().mla_decode_num_splits(B, P, H, max_kv_len, num_splits, num_cus)


def decode_workspace_size(B: int, P: int, H: int, max_kv_len: int, num_splits: int = 0) -> int:
    return library().mla_decode_workspace_size(B, P, H, max_kv_len, num_splits)


# The decode workspace's error-flags word (after its 65,536 completion counters) and its
# bits (include/mla.h: MLA_WORKSPACE_FLAGS_OFFSET, MLA_FLAG_*).
WORKSPACE_FLAGS_OFFSET = 4 * 65536
FLAG_STALE_COUNTERS = 1
FLAG_BAD_LENGTHS = 2
FLAG_BAD_BLOCKS = 4


class WorkspaceError(RuntimeError):
    """A decode workspace reported error flags (its calls' results are not to be trusted)."""

    def __init__(self, flags: int):
        what = []
        if flags & FLAG_STALE_COUNTERS:
            what.append("completion counters were not zero when a call started (a call did not "
                        "complete, or calls overlapped on this workspace)")
        if flags & FLAG_BAD_LENGTHS:
            what.append("a sequence length or kv_begin outside the contract")
        if flags & FLAG_BAD_BLOCKS:
            what.append("a negative block-table entry (block 0 was read in its place)")
        super().__init__("decode workspace flags 0x%x: %s" % (flags, "; ".join(what) or "?"))
        self.flags = flags


def decode_workspace_flags(workspace: torch.Tensor) -> int:
    """The error flags the kernels ORed into a decode workspace (reads device memory:
    waits for the calls queued on the tensor's stream)."""
    w = workspace[WORKSPACE_FLAGS_OFFSET:WORKSPACE_FLAGS_OFFSET + 4]
    return int(w.view(torch.int32).item()) if w.numel() == 4 else 0


def reset_decode_workspace(workspace: torch.Tensor) -> None:
    """Zero a decode workspace's completion counters and error flags."""
    workspace[:WORKSPACE_FLAGS_OFFSET + 4].zero_()


def check_decode_workspace(workspace: torch.Tensor) -> None:
    """Raise WorkspaceError if the calls on this workspace reported error flags, after
    zeroing its counters and flags so that the next call starts clean."""
    flags = decode_workspace_flags(workspace)
    if flags:
        reset_decode_workspace(workspace)
        raise WorkspaceError(flags)


# Zero-filled decode workspaces, one per (device, stream): every call leaves the
# workspace's counters zero, so calls ordered on one stream can share it.
_workspaces = {}


def decode_workspace(nbytes: int, dev: torch.device) -> torch.Tensor:
    """A zero-filled workspace of at least nbytes for calls on dev's current stream."""
    key = (dev, torch.cuda.current_stream(dev).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def verify(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
           seq_lens: torch.Tensor, *, softmax_scale: float, kv_scale: float = 1.0,
           kv_begin: Optional[torch.Tensor] = None, kv_end: Optional[torch.Tensor] = None,
           max_kv_len: Optional[int] = None, out_dtype: torch.dtype = torch.float32,
           num_splits: int = 0, out: Optional[torch.Tensor] = None,
           lse: Optional[torch.Tensor] = None, return_lse: bool = True,
           workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Speculative verify: q [B, P, H, 576] bf16 over a paged cache [blocks, block_size, 576].

    Query j of sequence b is position seq_lens[b] - P + j and sees keys
    kv_begin <= t < min(kv_end, seq_lens[b] - P + j + 1).  Returns (out [B, P, H, 512],
    lse [B, P, H] fp32 or None).  ``max_kv_len`` (host int) bounds any sequence's key
    range; when omitted it is read back from the device (a synchronisation).  A
    caller-supplied ``workspace`` (uint8) must be zero-filled before its first use; the
    calls keep it that way.
    """
    lib = library()
    if q.dim() != 4 or q.shape[-1] != HEAD_DIM_K or q.dtype != torch.bfloat16:
        raise TypeError("q must be [B, P, H, 576] bfloat16")
    dev = q.device
    B, P, H, _ = q.shape
    q = q.contiguous()
    if kv_cache.dim() != 3 or kv_cache.shape[-1] != HEAD_DIM_K or kv_cache.device != dev:
        raise TypeError("kv_cache must be [num_blocks, block_size, 576] on the query's device")
    kv_cache = kv_cache.contiguous()
    kvd = _kv_dtype(kv_cache)
    block_table = _dev_i32(block_table, "block_table", dev)
    seq_lens = _dev_i32(seq_lens, "seq_lens", dev)
    kv_begin = _dev_i32(kv_begin, "kv_begin", dev)
    kv_end = _dev_i32(kv_end, "kv_end", dev)
    _check_batch_arrays(B, block_table, seq_lens, kv_begin, kv_end)
    od = _out_dtype(out_dtype)
    out = _out_buffer(out, "out", (B, P, H, HEAD_DIM_V), out_dtype, dev)
    lse = _out_buffer(lse, "lse", (B, P, H), torch.float32, dev)
    workspace = _workspace_buffer(workspace, dev)
    if max_kv_len is None:
        hi = seq_lens if kv_end is None else torch.minimum(seq_lens, kv_end)
        lo = torch.zeros_like(hi) if kv_begin is None else kv_begin.clamp(min=0)
        max_kv_len = int((hi - lo).clamp(min=0).max().item()) if B > 0 else 0
    if out is None:
        out = torch.empty((B, P, H, HEAD_DIM_V), dtype=out_dtype, device=dev)
    if lse is None and return_lse:
        lse = torch.empty((B, P, H), dtype=torch.float32, device=dev)
    ws_need = lib.mla_decode_workspace_size(B, P, H, max_kv_len, num_splits)
    if workspace is None and ws_need > 0:
        workspace = decode_workspace(ws_need, dev)
    st = lib.mla_verify(
        _ptr(q), _ptr(kv_cache), kvd, float(kv_scale), _ptr(block_table),
        block_table.shape[1], kv_cache.shape[1], _ptr(seq_lens), _ptr(kv_begin), _ptr(kv_end),
        B, P, H, int(max_kv_len), float(softmax_scale), _ptr(out), od, _ptr(lse),
        int(num_splits), _ptr(workspace), 0 if workspace is None else workspace.numel(),
        _stream(dev))
    _check("mla_verify", st)
    return out, lse


def verify_noalloc(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                   seq_lens: torch.Tensor, *, softmax_scale: float, max_kv_len: int,
                   out: torch.Tensor, lse: Optional[torch.Tensor] = None, kv_scale: float = 1.0,
                   kv_begin: Optional[torch.Tensor] = None, kv_end: Optional[torch.Tensor] = None,
                   num_splits: int = 0) -> None:
    """mla_verify_noalloc: verify into caller-allocated out [B, P, H, 512] (fp32 or bf16) and
    lse [B, P, H] fp32 (or None), with the library's own per-GPU scratch instead of a
    workspace.  Allocates nothing on the device.  Calls that overlap on one GPU race."""
    lib = library()
    if q.dim() != 4 or q.shape[-1] != HEAD_DIM_K or q.dtype != torch.bfloat16 or \
            not q.is_contiguous():
        raise TypeError("q must be a contiguous [B, P, H, 576] bfloat16 tensor")
    dev = q.device
    B, P, H, _ = q.shape
    if (kv_cache.dim() != 3 or kv_cache.shape[-1] != HEAD_DIM_K or kv_cache.device != dev
            or not kv_cache.is_contiguous()):
        raise TypeError("kv_cache must be a contiguous [num_blocks, block_size, 576] tensor on "
                        "the query's device")
    bt = _dev_i32(block_table, "block_table", dev)
    sl = _dev_i32(seq_lens, "seq_lens", dev)
    kb = _dev_i32(kv_begin, "kv_begin", dev)
    ke = _dev_i32(kv_end, "kv_end", dev)
    _check_batch_arrays(B, bt, sl, kb, ke)
    _out_buffer(out, "out", (B, P, H, HEAD_DIM_V), out.dtype, dev)
    od = _out_dtype(out.dtype)
    _out_buffer(lse, "lse", (B, P, H), torch.float32, dev)
    _check("mla_verify_noalloc", lib.mla_verify_noalloc(
        _ptr(q), _ptr(kv_cache), _kv_dtype(kv_cache), float(kv_scale), _ptr(bt), bt.shape[1],
        kv_cache.shape[1], _ptr(sl), _ptr(kb), _ptr(ke), B, P, H, int(max_kv_len),
        float(softmax_scale), _ptr(out), od, _ptr(lse), int(num_splits), _stream(dev)))


def verify_launcher(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                    seq_lens: torch.Tensor, *, softmax_scale: float, kv_scale: float = 1.0,
                    max_kv_len: int, out: torch.Tensor, lse: Optional[torch.Tensor],
                    workspace: Optional[torch.Tensor], num_splits: int = 0,
                    kv_begin: Optional[torch.Tensor] = None,
                    kv_end: Optional[torch.Tensor] = None):
    """verify's C call with every argument marshalled once: returns a function that
    launches it on torch's current stream of q's device at call time (so the call can be
    captured into a HIP graph).  For loops that launch the same call many times (the
    tensors must stay alive and keep their storage)."""
    lib = library()
    if q.dim() != 4 or q.shape[-1] != HEAD_DIM_K or q.dtype != torch.bfloat16 or \
            not q.is_contiguous():
        raise TypeError("q must be a contiguous [B, P, H, 576] bfloat16 tensor")
    dev = q.device
    B, P, H, _ = q.shape
    if (kv_cache.dim() != 3 or kv_cache.shape[-1] != HEAD_DIM_K or kv_cache.device != dev
            or not kv_cache.is_contiguous()):
        raise TypeError("kv_cache must be a contiguous [num_blocks, block_size, 576] tensor on "
                        "the query's device")
    bt = _dev_i32(block_table, "block_table", dev)
    sl = _dev_i32(seq_lens, "seq_lens", dev)
    kb = _dev_i32(kv_begin, "kv_begin", dev)
    ke = _dev_i32(kv_end, "kv_end", dev)
    _check_batch_arrays(B, bt, sl, kb, ke)
    if out is None:
        raise TypeError("out is required")
    _out_buffer(out, "out", (B, P, H, HEAD_DIM_V), out.dtype, dev)
    od = _out_dtype(out.dtype)
    _out_buffer(lse, "lse", (B, P, H), torch.float32, dev)
    _workspace_buffer(workspace, dev)
    need = lib.mla_decode_workspace_size(B, P, H, int(max_kv_len), int(num_splits))
    if need > 0 and (workspace is None or workspace.numel() < need):
        raise MlaError("mla_verify", -3)
    args = (_ptr(q), _ptr(kv_cache), _kv_dtype(kv_cache), float(kv_scale), _ptr(bt),
            bt.shape[1], kv_cache.shape[1], _ptr(sl), _ptr(kb), _ptr(ke),
            B, P, H, int(max_kv_len), float(softmax_scale), _ptr(out), od,
            _ptr(lse), int(num_splits), _ptr(workspace),
            0 if workspace is None else workspace.numel())
    fn = lib.mla_verify

    def launch():
        st = fn(*args, _stream(dev))
        if st != 0:
            raise MlaError("mla_verify", st)
    return launch


def decode(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
           seq_lens: torch.Tensor, **kw) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Decode: q [B, H, 576] bf16; returns (out [B, H, 512], lse [B, H] or None)."""
    if q.dim() != 3:
        raise TypeError("q must be [B, H, 576]")
    out = kw.pop("out", None)
    lse = kw.pop("lse", None)
    B, H = q.shape[0], q.shape[1]
    od = kw.get("out_dtype", torch.float32)
    _out_buffer(out, "out", (B, H, HEAD_DIM_V), od, q.device)
    _out_buffer(lse, "lse", (B, H), torch.float32, q.device)
    o, l = verify(q.unsqueeze(1), kv_cache, block_table, seq_lens,
                  out=None if out is None else out.unsqueeze(1),
                  lse=None if lse is None else lse.unsqueeze(1), **kw)
    return o.squeeze(1), (None if l is None else l.squeeze(1))


def prefill(q: torch.Tensor, kv: torch.Tensor, cu_seqlens: torch.Tensor, *,
            softmax_scale: float, kv_scale: float = 1.0, max_seqlen: Optional[int] = None,
            out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None,
            return_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Causal prefill: q [T, H, 576] bf16, kv [T, 576]; cu_seqlens [B + 1] int32 on device."""
    lib = library()
    if q.dim() != 3 or q.shape[-1] != HEAD_DIM_K or q.dtype != torch.bfloat16:
        raise TypeError("q must be [T, H, 576] bfloat16")
    dev = q.device
    T, H, _ = q.shape
    q = q.contiguous()
    if tuple(kv.shape) != (T, HEAD_DIM_K) or kv.device != dev:
        raise TypeError("kv must be [T, 576] on the query's device")
    kv = kv.contiguous()
    cu = _dev_i32(cu_seqlens, "cu_seqlens", dev)
    B = cu.numel() - 1
    if max_seqlen is None:
        max_seqlen = int((cu[1:] - cu[:-1]).max().item()) if B > 0 else 0
    if cu.dim() != 1 or cu.numel() < 1:
        raise TypeError("cu_seqlens must be [B + 1]")
    od = _out_dtype(out_dtype)
    out = _out_buffer(out, "out", (T, H, HEAD_DIM_V), out_dtype, dev)
    lse = _out_buffer(lse, "lse", (T, H), torch.float32, dev)
    if out is None:
        out = torch.empty((T, H, HEAD_DIM_V), dtype=out_dtype, device=dev)
    if lse is None and return_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    st = lib.mla_prefill(_ptr(q), _ptr(kv), _kv_dtype(kv), float(kv_scale), _ptr(cu), B, T,
                         int(max_seqlen), H, float(softmax_scale), _ptr(out), od, _ptr(lse),
                         _stream(dev))
    _check("mla_prefill", st)
    return out, lse


def merge_lse(part_out: torch.Tensor, part_lse: torch.Tensor, *,
              out_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None,
              lse: Optional[torch.Tensor] = None,
              return_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Merge partials part_out [S, N, 512] fp32 / part_lse [S, N] fp32 by log-sum-exp."""
    lib = library()
    if part_out.dim() != 3 or part_out.shape[-1] != HEAD_DIM_V or part_out.dtype != torch.float32:
        raise TypeError("part_out must be [S, N, 512] float32")
    S, N, _ = part_out.shape
    if part_lse.shape != (S, N) or part_lse.dtype != torch.float32:
        raise TypeError("part_lse must be [S, N] float32")
    dev = part_out.device
    part_out = part_out.contiguous()
    part_lse = part_lse.contiguous()
    if part_lse.device != dev:
        raise TypeError("part_lse must be on part_out's device")
    od = _out_dtype(out_dtype)
    out = _out_buffer(out, "out", (N, HEAD_DIM_V), out_dtype, dev)
    lse = _out_buffer(lse, "lse", (N,), torch.float32, dev)
    if out is None:
        out = torch.empty((N, HEAD_DIM_V), dtype=out_dtype, device=dev)
    if lse is None and return_lse:
        lse = torch.empty((N,), dtype=torch.float32, device=dev)
    st = lib.mla_merge_lse(_ptr(part_out), _ptr(part_lse), S, N, _ptr(out), od, _ptr(lse),
                           _stream(dev))
    _check("mla_merge_lse", st)
    return out, lse


def cache_write(latent: torch.Tensor, kv_cache: torch.Tensor, slot_mapping: torch.Tensor, *,
                kv_scale: float = 1.0) -> torch.Tensor:
    """Write latent [N, 576] bf16 rows into kv_cache [num_blocks, block_size, 576] at flat
    slots slot_mapping [N] int32 (negative or out-of-range slots are skipped); FP8 caches
    (uint8 / float8_e4m3fn) receive E4M3FN codes of x / kv_scale.  Returns kv_cache."""
    lib = library()
    if latent.dim() != 2 or latent.shape[1] != HEAD_DIM_K or latent.dtype != torch.bfloat16:
        raise TypeError("latent must be [N, 576] bfloat16")
    dev = latent.device
    if kv_cache.shape[-1] != HEAD_DIM_K or kv_cache.device != dev or not kv_cache.is_contiguous():
        raise TypeError("kv_cache must be a contiguous [..., 576] tensor on the latent's device")
    latent = latent.contiguous()
    sm = _dev_i32(slot_mapping, "slot_mapping", dev)
    if sm.numel() != latent.shape[0]:
        raise TypeError("slot_mapping must have one entry per latent row")
    st = lib.mla_cache_write(_ptr(latent), latent.shape[0], _ptr(sm), _ptr(kv_cache),
                             _kv_dtype(kv_cache), float(kv_scale),
                             kv_cache.numel() // HEAD_DIM_K, _stream(dev))
    _check("mla_cache_write", st)
    return kv_cache


def top_k_renorm_workspace_size(rows: int, vocab: int) -> int:
    return library().mla_top_k_renorm_workspace_size(rows, vocab)


# Scratch for top_k_renorm_prob, one per (device, stream); it needs no initialisation.
_topk_workspaces = {}


def top_k_renorm_prob(probs: torch.Tensor, top_k: torch.Tensor, *,
                      out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Keep the top_k[r] largest entries of each row of probs [rows, vocab] fp32, zero the
    rest and divide the kept ones by their sum (ties: the lower index first; k <= 0 or
    k >= vocab keeps the whole row).  top_k: [rows] int32 on the same device.  ``out`` may
    be ``probs`` (in place).  Returns out."""
    lib = library()
    if probs.dim() != 2 or probs.dtype != torch.float32 or not probs.is_contiguous():
        raise TypeError("probs must be a contiguous [rows, vocab] float32 tensor")
    dev = probs.device
    rows, vocab = probs.shape
    tk = _dev_i32(top_k, "top_k", dev)
    if tk.numel() != rows:
        raise TypeError("top_k must have one entry per row")
    if out is None:
        out = torch.empty_like(probs)
    elif (out.shape != probs.shape or out.dtype != torch.float32 or out.device != dev
          or not out.is_contiguous()):
        raise TypeError("out must be a contiguous float32 tensor shaped like probs")
    need = lib.mla_top_k_renorm_workspace_size(rows, vocab)
    if workspace is None:
        key = (dev, torch.cuda.current_stream(dev).cuda_stream)
        workspace = _topk_workspaces.get(key)
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
            _topk_workspaces[key] = workspace
    st = lib.mla_top_k_renorm_prob(_ptr(probs), _ptr(tk), rows, vocab, _ptr(out),
                                   _ptr(workspace), workspace.numel(), _stream(dev))
    _check("mla_top_k_renorm_prob", st)
    return out


def default_softmax_scale(qk_dim: int = 192) -> float:
    """1 / sqrt(qk_dim); 192 = 128 + 64 is the query-key width before absorption."""
    return 1.0 / math.sqrt(qk_dim)
