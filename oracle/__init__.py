"""FP64 CPU oracle for MLA attention over a latent KV cache (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU-baseline
leg may import this package; the product library never does.  The arithmetic
lives in ``mla_oracle.c`` (plain C, double precision, OpenMP over query rows);
this module only builds it with gcc and marshals numpy arrays.

Functions follow the plain definitions stated in ``mla_oracle.c``: softmax
attention of each query row over its visible latent rows (key = the whole
576-wide row, value = its first 512 entries), the merge of partial results
by their log-sum-exp normalisers, the latent-row cache write (FP8 E4M3FN
quantisation and scatter) and the top-k renormalisation of probability rows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "libmla_oracle.so")

DK = 576
DV = 512


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (double precision, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-Wall",
             "-shared", "-fPIC", src, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


class OracleLib:
    """One loaded copy of the compiled oracle."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        lib.mla_oracle_fp8_e4m3fn_value.restype = ctypes.c_double
        lib.mla_oracle_fp8_e4m3fn_value.argtypes = [ctypes.c_uint8]
        lib.mla_oracle_bf16_value.restype = ctypes.c_double
        lib.mla_oracle_bf16_value.argtypes = [ctypes.c_uint16]
        lib.mla_oracle_decode.restype = ctypes.c_int
        lib.mla_oracle_decode.argtypes = [
            P, P, ctypes.c_int, ctypes.c_float, P, ctypes.c_int, ctypes.c_int, P, P, P,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, P, ctypes.c_long, P, P,
            ctypes.c_int]
        lib.mla_oracle_prefill.restype = ctypes.c_int
        lib.mla_oracle_prefill.argtypes = [
            P, P, ctypes.c_int, ctypes.c_float, P, ctypes.c_int, ctypes.c_int, ctypes.c_float,
            P, ctypes.c_long, P, P, ctypes.c_int]
        lib.mla_oracle_merge.restype = ctypes.c_int
        lib.mla_oracle_merge.argtypes = [P, P, ctypes.c_int, ctypes.c_long, P, P]
        lib.mla_oracle_max_threads.restype = ctypes.c_int
        lib.mla_oracle_max_threads.argtypes = []
        lib.mla_oracle_fp8_e4m3fn_encode.restype = ctypes.c_uint8
        lib.mla_oracle_fp8_e4m3fn_encode.argtypes = [ctypes.c_float]
        lib.mla_oracle_cache_write.restype = ctypes.c_int
        lib.mla_oracle_cache_write.argtypes = [P, ctypes.c_long, P, P, ctypes.c_int,
                                               ctypes.c_float, ctypes.c_long]
        lib.mla_oracle_top_k_renorm.restype = ctypes.c_int
        lib.mla_oracle_top_k_renorm.argtypes = [P, P, ctypes.c_long, ctypes.c_long, P]
        self.lib = lib
        self.path = path

    def fp8_e4m3fn_encode(self, y: float) -> int:
        """E4M3FN code nearest to fp32 y (clamped to +-448, ties to even, NaN -> 0x7F)."""
        return int(self.lib.mla_oracle_fp8_e4m3fn_encode(ctypes.c_float(y)))

    def cache_write(self, latent_bits: np.ndarray, slot: np.ndarray, kv: np.ndarray,
                    kv_fp8: bool, kv_scale: float) -> np.ndarray:
        """Copy of kv [.., 576] (BF16 bits or FP8 codes) with the rows of latent_bits
        [N, 576] (BF16 bits) written, quantised for FP8, at flat slots `slot` [N]."""
        lat = _c(latent_bits, np.uint16)
        sl = _c(slot, np.int32)
        out = np.ascontiguousarray(kv).copy()
        num_slots = out.size // 576
        self.lib.mla_oracle_cache_write(_ptr(lat), lat.shape[0], _ptr(sl), _ptr(out),
                                         1 if kv_fp8 else 0, float(kv_scale), num_slots)
        return out

    def top_k_renorm_prob(self, probs: np.ndarray, top_k) -> np.ndarray:
        """Rows of fp32 probabilities -> float64 rows: the k largest entries of each row
        divided by their sum, every other entry zero (k per row; k <= 0 or k >= vocab
        keeps the whole row; ties rank the lower index first)."""
        p = _c(probs, np.float32)
        if p.ndim != 2:
            raise ValueError("probs must be [rows, vocab]")
        rows, vocab = p.shape
        k = np.ascontiguousarray(np.broadcast_to(np.asarray(top_k, np.int32), (rows,)))
        out = np.empty((rows, vocab), np.float64)
        st = self.lib.mla_oracle_top_k_renorm(_ptr(p), _ptr(k), rows, vocab, _ptr(out))
        if st != 0:
            raise ValueError("oracle top_k_renorm failed (%d): NaN entry or no memory" % st)
        return out

    def max_threads(self) -> int:
        return self.lib.mla_oracle_max_threads()

    def fp8_e4m3fn_value(self, code: int) -> float:
        """Exact value of one OCP FP8 E4M3FN code."""
        return self.lib.mla_oracle_fp8_e4m3fn_value(int(code) & 0xFF)

    def bf16_value(self, bits: int) -> float:
        """Exact value of one BF16 bit pattern."""
        return self.lib.mla_oracle_bf16_value(int(bits) & 0xFFFF)

    def decode(self, q_bits: np.ndarray, kv: np.ndarray, kv_fp8: bool, kv_scale: float,
               block_table: np.ndarray, seq_lens: np.ndarray, softmax_scale: float,
               kv_begin: Optional[np.ndarray] = None, kv_end: Optional[np.ndarray] = None,
               rows: Optional[np.ndarray] = None,
               threads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """Decode / verify attention over a paged latent cache, in float64.

        q_bits [B, P, H, 576] uint16 (BF16 bits); kv [num_blocks, block_size, 576]
        uint16 (BF16 bits) or uint8 (FP8 E4M3FN codes); block_table [B, max_blocks]
        int32; seq_lens [B] int32 (context length including the P queries).
        Query j of sequence b sees keys t with
        max(kv_begin, 0) <= t < min(kv_end, seq_lens - P + j + 1).
        Returns out [B, P, H, 512] and lse [B, P, H] (or [n_rows, 512], [n_rows]
        when ``rows`` lists flat row indices (b * P + j) * H + h).
        """
        q_bits = _c(q_bits, np.uint16)
        B, P, H, dk = q_bits.shape
        assert dk == DK
        kv = np.ascontiguousarray(kv)
        assert kv.dtype == (np.uint8 if kv_fp8 else np.uint16) and kv.shape[-1] == DK
        block_size = kv.shape[1]
        bt = _c(block_table, np.int32)
        sl = _c(seq_lens, np.int32)
        kb = _c(kv_begin, np.int32)
        ke = _c(kv_end, np.int32)
        assert bt.shape[0] == B and sl.shape == (B,)
        rws = _c(rows, np.int64)
        n = B * P * H if rws is None else rws.shape[0]
        out = np.empty((n, DV), np.float64)
        lse = np.empty((n,), np.float64)
        rc = self.lib.mla_oracle_decode(
            _ptr(q_bits), _ptr(kv), 1 if kv_fp8 else 0, float(kv_scale), _ptr(bt), bt.shape[1],
            block_size, _ptr(sl), _ptr(kb), _ptr(ke), B, P, H, float(softmax_scale), _ptr(rws),
            0 if rws is None else n, _ptr(out), _ptr(lse), int(threads))
        if rc != 0:
            raise ValueError("oracle decode rejected its arguments")
        if rws is None:
            return out.reshape(B, P, H, DV), lse.reshape(B, P, H)
        return out, lse

    def prefill(self, q_bits: np.ndarray, kv: np.ndarray, kv_fp8: bool, kv_scale: float,
                cu_seqlens: np.ndarray, softmax_scale: float,
                tokens: Optional[np.ndarray] = None,
                threads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """Causal prefill over packed sequences, in float64.

        q_bits [T, H, 576] uint16; kv [T, 576] uint16 or uint8; cu_seqlens [B + 1].
        Token g of sequence b sees keys cu_seqlens[b] .. g.  Returns out [n, H, 512],
        lse [n, H] for all T tokens or the listed global ``tokens``.
        """
        q_bits = _c(q_bits, np.uint16)
        T, H, dk = q_bits.shape
        assert dk == DK
        kv = np.ascontiguousarray(kv)
        assert kv.dtype == (np.uint8 if kv_fp8 else np.uint16) and kv.shape == (T, DK)
        cu = _c(cu_seqlens, np.int32)
        B = cu.shape[0] - 1
        assert cu[-1] == T
        tk = _c(tokens, np.int64)
        n = T if tk is None else tk.shape[0]
        out = np.empty((n, H, DV), np.float64)
        lse = np.empty((n, H), np.float64)
        rc = self.lib.mla_oracle_prefill(
            _ptr(q_bits), _ptr(kv), 1 if kv_fp8 else 0, float(kv_scale), _ptr(cu), B, H,
            float(softmax_scale), _ptr(tk), 0 if tk is None else n, _ptr(out), _ptr(lse),
            int(threads))
        if rc != 0:
            raise ValueError("oracle prefill rejected its arguments")
        return out, lse

    def merge(self, part_out: np.ndarray, part_lse: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
        """Merge S partial results [S, N, 512] / [S, N] by their log-sum-exp normalisers."""
        po = _c(part_out, np.float64)
        pl = _c(part_lse, np.float64)
        S, N, dv = po.shape
        assert dv == DV and pl.shape == (S, N)
        out = np.empty((N, DV), np.float64)
        lse = np.empty((N,), np.float64)
        rc = self.lib.mla_oracle_merge(_ptr(po), _ptr(pl), S, N, _ptr(out), _ptr(lse))
        if rc != 0:
            raise ValueError("oracle merge rejected its arguments")
        return out, lse


_default: Optional[OracleLib] = None


def get() -> OracleLib:
    """The oracle built from ``mla_oracle.c`` (compiled on first use if missing or stale)."""
    global _default
    if _default is None:
        build(force=False)
        _default = OracleLib(_LIB)
    return _default


def max_threads() -> int:
    return get().max_threads()


def fp8_e4m3fn_value(code: int) -> float:
    return get().fp8_e4m3fn_value(code)


def bf16_value(bits: int) -> float:
    return get().bf16_value(bits)


def decode(*args, **kwargs):
    return get().decode(*args, **kwargs)


def prefill(*args, **kwargs):
    return get().prefill(*args, **kwargs)


def fp8_e4m3fn_encode(y: float) -> int:
    return get().fp8_e4m3fn_encode(y)


def cache_write(*args, **kwargs):
    return get().cache_write(*args, **kwargs)


def merge(*args, **kwargs):
    return get().merge(*args, **kwargs)


def top_k_renorm_prob(*args, **kwargs):
    return get().top_k_renorm_prob(*args, **kwargs)
