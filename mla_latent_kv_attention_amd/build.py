"""Build the HIP libraries for gfx950 with hipcc (in-tree): libmla.so, the attention
library behind include/mla.h; libmla_read_probe.so, the benchmark's plain-read probe
(a measurement helper kept out of the attention library); and libmla_timeline.so, the
attention library again with per-work-group phase stamps compiled in (MLA_TIMELINE),
which only `bench.py --timeline` loads."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmla.so")
SOURCES = ["mla_api.cpp", "mla_decode.hip", "mla_verify.hip", "mla_prefill.hip", "mla_cache.hip",
           "mla_sampling.hip"]
PROBE_LIB = os.path.join(PKG, "libmla_read_probe.so")
PROBE_SOURCES = [os.path.join("probe", "mla_read_probe.hip")]
TIMELINE_LIB = os.path.join(PKG, "libmla_timeline.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _build_one(sources, lib, verbose: bool, defines=()) -> str:
    srcs = []
    for s in sources:
        path = os.path.join(CSRC, s)
        srcs += (["-x", "hip"] if s.endswith(".cpp") else []) + [path]
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-D" + d for d in defines] + ["-I", os.path.join(CSRC, "probe")] + \
        srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "unknown target feature" not in l and "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile the three libraries; returns the attention library's path."""
    _build_one(PROBE_SOURCES, PROBE_LIB, verbose)
    _build_one(SOURCES, TIMELINE_LIB, verbose, defines=("MLA_TIMELINE",))
    return _build_one(SOURCES, LIB, verbose)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
