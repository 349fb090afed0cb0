"""ctypes wrapper of the benchmark's plain-read probe (``libmla_read_probe.so``, built
from ``csrc/probe/mla_read_probe.hip``): a measurement helper next to the attention
library, not part of it.  The package's own binding never imports this module."""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla_read_probe.so")
_lib = None


def library() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libmla_read_probe.so is not built (%s); run "
                              "mla_latent_kv_attention_amd/build.py" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        lib.mla_hbm_read_probe.restype = ctypes.c_int
        lib.mla_hbm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                           ctypes.c_int, ctypes.c_void_p]
        _lib = lib
    return _lib


def hbm_read_probe(src: torch.Tensor, sink: torch.Tensor, *, grid: int = 1024) -> None:
    """Launch the plain-read probe over src's bytes on torch's current stream (timed by
    the caller, it gives the device's rate for a kernel that only reads those bytes).
    sink: int32 device tensor of at least grid * 256 elements."""
    if not src.is_contiguous() or src.device.type != "cuda":
        raise TypeError("src must be a contiguous device tensor")
    if sink.dtype != torch.int32 or sink.numel() < grid * 256 or sink.device != src.device:
        raise TypeError("sink must be an int32 tensor of grid * 256 elements on src's device")
    nbytes = src.numel() * src.element_size()
    st = library().mla_hbm_read_probe(
        ctypes.c_void_p(src.data_ptr()), nbytes - nbytes % 16, ctypes.c_void_p(sink.data_ptr()),
        int(grid), ctypes.c_void_p(torch.cuda.current_stream(src.device).cuda_stream))
    if st != 0:
        raise RuntimeError("mla_hbm_read_probe failed (status %d)" % st)
