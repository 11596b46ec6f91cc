"""Device fill of the seeded inputs (same definition as synth/__init__.py).

Used where inputs are too large to generate on the host (64-layer stacks,
a 248320 x 5120 embedding table).  Tests check it bit for bit against the
numpy generator on sampled elements.
"""
from __future__ import annotations

import ctypes as C
import os
import shutil
import subprocess

import numpy as np
import torch

from . import GAUSS_TABLE, SCALE_TABLE, stream_key

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fill.hip")
LIB = os.path.join(_HERE, "libsynth.so")


def build() -> str:
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    tmp = LIB + ".tmp"
    subprocess.check_call([hipcc, "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                           "-o", tmp, _SRC], stderr=subprocess.DEVNULL)
    os.replace(tmp, LIB)
    return LIB


_lib = None
_tables: dict = {}


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} missing: run synth.device.build()")
        L = C.CDLL(LIB)
        for fn in ("synth_fill_trits", "synth_fill_table16", "synth_fill_table32"):
            getattr(L, fn).restype = C.c_int
        L.synth_fill_trits.argtypes = [C.c_void_p, C.c_uint64, C.c_int64, C.c_int64, C.c_void_p]
        L.synth_fill_table16.argtypes = [C.c_void_p, C.c_void_p, C.c_uint64, C.c_int64, C.c_int64, C.c_void_p]
        L.synth_fill_table32.argtypes = [C.c_void_p, C.c_void_p, C.c_uint64, C.c_int64, C.c_int64, C.c_void_p]
        _lib = L
    return _lib


def _table(name: str, device):
    key = (name, str(device))
    if key not in _tables:
        src = SCALE_TABLE.view(np.int16) if name == "scale" else GAUSS_TABLE
        _tables[key] = torch.from_numpy(np.ascontiguousarray(src)).to(device)
    return _tables[key]


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ok(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what}: hip error {rc}")


def trits(seed: int, stream: int, n: int, k: int, device="cuda", row0: int = 0, out=None) -> torch.Tensor:
    if out is None:
        out = torch.empty((n, k), dtype=torch.int8, device=device)
    _ok(_L().synth_fill_trits(C.c_void_p(out.data_ptr()), stream_key(seed, stream), row0 * k, n * k,
                              _stream()), "synth_fill_trits")
    return out


def scales(seed: int, stream: int, n: int, nb: int, device="cuda", row0: int = 0, out=None) -> torch.Tensor:
    if out is None:
        out = torch.empty((n, nb), dtype=torch.int16, device=device)
    t = _table("scale", out.device)
    _ok(_L().synth_fill_table16(C.c_void_p(out.data_ptr()), C.c_void_p(t.data_ptr()),
                                stream_key(seed, stream), row0 * nb, n * nb, _stream()), "synth_fill_table16")
    return out


def gauss(seed: int, stream: int, count: int, device="cuda", start: int = 0, out=None) -> torch.Tensor:
    if out is None:
        out = torch.empty(count, dtype=torch.float32, device=device)
    t = _table("gauss", out.device)
    _ok(_L().synth_fill_table32(C.c_void_p(out.data_ptr()), C.c_void_p(t.data_ptr()),
                                stream_key(seed, stream), start, count, _stream()), "synth_fill_table32")
    return out
