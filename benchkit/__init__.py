"""Measurement kit of the benchmark: in-run streaming probes (``probe.hip``,
built into ``libbenchkit.so``) and the reader of rocprofv3 PMC counter runs
(``traffic.py``).  Not part of the library's product path: the benchmark
uses it to set each kernel beside the best time the same HBM traffic takes on
the same device in the same run."""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libbenchkit.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build() -> str:
    """Compile probe.hip for gfx950 into libbenchkit.so (always rebuilds)."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, os.path.join(HERE, "probe.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on benchkit/probe.hip")
    os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise ImportError(f"{LIB} is missing: build it first (python -c 'import benchkit; benchkit.build()')")
        L = ctypes.CDLL(LIB)
        L.benchkit_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        L.benchkit_stream.restype = ctypes.c_int
        _lib = L
    return _lib


class StreamProbe:
    """A probe that reads ``read_bytes`` and writes ``write_bytes`` (rounded
    down to 16-byte vectors) on torch's current stream, in one of the probe
    kernel's shapes: ``u`` vectors per thread, nontemporal loads ``ntl``,
    nontemporal stores ``nts``."""

    SHAPES = [(u, ntl, nts) for u in (1, 2, 4, 8) for ntl in (0, 1) for nts in (0, 1)]

    def __init__(self, torch, read_bytes: int, write_bytes: int, device):
        self.torch = torch
        self.nr = read_bytes // 16 * 16
        self.nw = min(write_bytes // 16 * 16, self.nr)
        self.src = torch.ones(self.nr // 4, dtype=torch.float32, device=device)
        self.dst = torch.empty(max(self.nw // 4, 4), dtype=torch.float32, device=device)
        self.sink = torch.zeros(256, dtype=torch.int32, device=device)
        self.shape = self.SHAPES[0]

    def __call__(self, shape=None):
        u, ntl, nts = shape or self.shape
        rc = lib().benchkit_stream(ctypes.c_void_p(self.src.data_ptr()), self.nr,
                                   ctypes.c_void_p(self.dst.data_ptr()), self.nw,
                                   ctypes.c_void_p(self.sink.data_ptr()), u, ntl, nts,
                                   ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"benchkit_stream failed ({rc})")
