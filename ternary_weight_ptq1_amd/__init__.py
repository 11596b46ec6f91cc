"""Python binding of ``libptq1.so`` (the C ABI in ``include/ptq1.h``).

Argument marshalling only: every function passes device pointers of torch
tensors and ``torch.cuda.current_stream()`` to the C entry point of the same
name and raises :class:`Ptq1Error` on a non-OK status.  torch supplies device
memory and streams; every step of the computation runs in the HIP kernels.
There is no fallback: if the library is not built, importing the binding's
functions raises.
"""
from __future__ import annotations

import ctypes as C
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PTQ1_LIB may name another build of the same library (the sanitizer build
# of build.py --sanitize, for host-only test runs)
LIB_PATH = os.environ.get("PTQ1_LIB", os.path.join(_HERE, "libptq1.so"))
HEADER = os.path.join(os.path.dirname(_HERE), "include", "ptq1.h")

BLOCK_WEIGHTS = 128
TRIT_BYTES = 26
BLOCK_BYTES = 28
HADAMARD = 1024
TILE_ROWS = 32
TILE_BLOCKS = 2

STATUS = {0: "PTQ1_OK", 1: "PTQ1_ERR_NULL", 2: "PTQ1_ERR_SHAPE", 3: "PTQ1_ERR_ALIGN",
          4: "PTQ1_ERR_OVERFLOW", 5: "PTQ1_ERR_UNSUPPORTED", 6: "PTQ1_ERR_WORKSPACE",
          7: "PTQ1_ERR_ALIAS", 8: "PTQ1_ERR_HIP"}


class Ptq1Error(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


_lib = None
i64, sz, p = C.c_int64, C.c_size_t, C.c_void_p

_SIGS = {
    "ptq1_status_string": ([C.c_int], C.c_char_p),
    "ptq1_last_error": ([], C.c_char_p),
    "ptq1_geometry": ([p, C.c_int32], C.c_int),
    "ptq1_packed_bytes": ([i64, i64], i64),
    "ptq1_tiled_bytes": ([i64, i64], i64),
    "ptq1_tile": ([p, i64, i64, p, p], C.c_int),
    "ptq1_pack": ([p, p, i64, i64, p, p], C.c_int),
    "ptq1_dequant": ([p, i64, i64, p, p], C.c_int),
    "hadamard_rotate": ([p, p, i64, i64, p, p], C.c_int),
    "hadamard_unrotate_rows": ([p, i64, i64, p, i64, p, p, p], C.c_int),
    "ptq1_matvec_workspace_bytes": ([i64, i64], sz),
    "ptq1_matvec": ([p, i64, i64, p, p, p, p, p, sz, p], C.c_int),
    "ptq1_matvec_float_peel": ([p, i64, i64, p, p, p, p, p, sz, p], C.c_int),
    "ptq1_gate_up_workspace_bytes": ([i64, i64], sz),
    "ptq1_gate_up": ([p, p, i64, i64, p, p, p, p, p, sz, p], C.c_int),
    "ptq1_swiglu": ([p, p, p, i64, p], C.c_int),
    "ptq1_gemm_workspace_bytes": ([i64, i64, i64], sz),
    "ptq1_gemm": ([p, i64, i64, p, i64, p, p, p, sz, p], C.c_int),
    "ptq1_ffn_workspace_bytes": ([i64, i64, i64], sz),
    "ptq1_ffn_block": ([p, p, i64, i64, i64, p, p, p, p, C.c_float, p, p, sz, p], C.c_int),
    "pq2_packed_bytes": ([i64, i64], i64),
    "pq2_pack": ([p, p, i64, i64, p, p], C.c_int),
    "pq2_dequant": ([p, i64, i64, p, p], C.c_int),
    "pq2_tiled_bytes": ([i64, i64], i64),
    "pq2_tile": ([p, i64, i64, p, p], C.c_int),
    "pq2_matvec_workspace_bytes": ([i64, i64], sz),
    "pq2_matvec": ([p, i64, i64, p, p, p, p, p, sz, p], C.c_int),
    "pq2_gemm_workspace_bytes": ([i64, i64, i64], sz),
    "pq2_gemm": ([p, i64, i64, p, i64, p, p, p, sz, p], C.c_int),
    "pq2_ffn_workspace_bytes": ([i64, i64, i64], sz),
    "ptq1_matvec_w2a8_workspace_bytes": ([i64, i64], sz),
    "ptq1_gemm_w2a8_workspace_bytes": ([i64, i64, i64], sz),
    "ptq1_gemm_w2a8": ([p, i64, i64, p, i64, p, p, sz, p], C.c_int),
    "ptq1_matvec_w2a8": ([p, i64, i64, p, p, p, p, sz, p], C.c_int),
    "pq2_ffn_block": ([p, p, i64, i64, i64, p, p, p, p, C.c_float, p, p, sz, p], C.c_int),
    "ptq1_ffn_workspace_offsets": ([i64, i64, i64, p], C.c_int),
    "ptq1_ffn_block_noalloc": ([p, p, i64, i64, i64, p, p, p, p, C.c_float, p, p], C.c_int),
    "pq2_ffn_workspace_offsets": ([i64, i64, i64, p], C.c_int),
    "ptq1_profile_arm": ([C.c_char_p, p, p, C.c_int32], C.c_int),
    "ptq1_profile_count": ([C.c_char_p], C.c_int32),
}


def lib():
    """The loaded C library.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m ternary_weight_ptq1_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions declared in include/ptq1.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"\b([a-z_0-9]+)\s*\(", text.split('extern "C" {', 1)[1])


def _check(fn: str, status: int):
    if status != 0:
        raise Ptq1Error(fn, status, lib().ptq1_last_error().decode())


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


# ------------------------------------------------------------- validation ----
# The C library sees only pointers and sizes, so every tensor is checked here
# against the sizes the call will read or write before anything is enqueued:
# a host tensor or a short one would become an out-of-range device access.

def _on_device(t: torch.Tensor) -> bool:
    return t.is_cuda


def _dev(t: torch.Tensor, name: str, dtype=None, numel: int | None = None, min_numel: int | None = None,
         device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not _on_device(t):
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, the call uses {numel}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} has {t.numel()} elements, the call reads or writes {min_numel}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call runs on {device}")
    return t


def _opt(t, name, dtype, numel=None, device=None):
    return None if t is None else _dev(t, name, dtype, numel=numel, device=device)


def _signs(s, device, required=True):
    if s is None:
        if required:
            raise ValueError("signs1024 is required")
        return None
    return _dev(s, "signs1024", torch.float32, numel=HADAMARD, device=device)


def _rows_of(x: torch.Tensor, k: int, name: str = "x") -> int:
    """Rows of an activation tensor of width k (its element count must be a multiple of k)."""
    if k <= 0:
        raise ValueError(f"k = {k} must be positive")
    if x.numel() % k != 0:
        raise ValueError(f"{name} has {x.numel()} elements, not a multiple of k = {k}")
    return x.numel() // k


def _mat(w: torch.Tensor, name: str, nbytes: int, device):
    """A weight matrix of nbytes bytes (a negative nbytes is a bad shape, refused by the library)."""
    return _dev(w, name, torch.uint8, min_numel=nbytes if nbytes > 0 else None, device=device)


def _ws(nbytes: int, device, ws):
    if nbytes == 0:
        return None, 0
    if ws is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes
    _dev(ws, "ws", torch.uint8, min_numel=nbytes, device=device)
    return ws, ws.numel()


def _out(out, name, shape, device, dtype=torch.float32):
    count = 1
    for s in shape:
        count *= s
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    return _dev(out, name, dtype, numel=count, device=device)


# ------------------------------------------------------------------ codec ----

def ptq1_geometry() -> tuple[int, int, int, int, int, int]:
    """(weights per block, trit bytes, block bytes, Hadamard width, tile rows, tile blocks)."""
    out = (C.c_int32 * 6)()
    _check("ptq1_geometry", lib().ptq1_geometry(C.cast(out, p), 6))
    return tuple(out)


def ptq1_packed_bytes(n: int, k: int) -> int:
    return lib().ptq1_packed_bytes(n, k)


def _trits_scales(trits, scales_f16):
    _dev(trits, "trits", torch.int8)
    if trits.dim() != 2:
        raise ValueError("trits must be [n, k]")
    n, k = trits.shape
    if k % BLOCK_WEIGHTS != 0:
        raise ValueError(f"k = {k} is not a multiple of {BLOCK_WEIGHTS}")
    _dev(scales_f16, "scales_f16", (torch.int16, torch.float16, torch.uint16), numel=n * (k // BLOCK_WEIGHTS),
         device=trits.device)
    return n, k


def ptq1_pack(trits: torch.Tensor, scales_f16: torch.Tensor, out: torch.Tensor | None = None,
              stream=None) -> torch.Tensor:
    """int8 trits [n, k] + binary16 bit patterns [n, k/128] (int16 or float16) -> uint8 [n, k/128*28]."""
    n, k = _trits_scales(trits, scales_f16)
    out = _out(out, "blocks", (n, (k // BLOCK_WEIGHTS) * BLOCK_BYTES), trits.device, torch.uint8)
    _check("ptq1_pack", lib().ptq1_pack(_ptr(trits), _ptr(scales_f16), n, k, _ptr(out), _stream(stream)))
    return out


def ptq1_tiled_bytes(n: int, k: int) -> int:
    return lib().ptq1_tiled_bytes(n, k)


def ptq1_tile(blocks: torch.Tensor, n: int, k: int, out: torch.Tensor | None = None,
              stream=None) -> torch.Tensor:
    """Packed [n, k/128*28] uint8 -> the tiled device layout (flat uint8) the
    matvec, gate/up, GEMM and feed-forward calls read."""
    nbytes = ptq1_tiled_bytes(n, k)
    if nbytes < 0:
        raise ValueError(f"bad shape [{n}][{k}]")
    _mat(blocks, "blocks", ptq1_packed_bytes(n, k), None)
    out = _out(out, "tiled", (nbytes,), blocks.device, torch.uint8)
    _check("ptq1_tile", lib().ptq1_tile(_ptr(blocks), n, k, _ptr(out), _stream(stream)))
    return out


def ptq1_dequant(blocks: torch.Tensor, n: int, k: int, out: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
    _mat(blocks, "blocks", ptq1_packed_bytes(n, k), None)
    out = _out(out, "w", (n, k), blocks.device)
    _check("ptq1_dequant", lib().ptq1_dequant(_ptr(blocks), n, k, _ptr(out), _stream(stream)))
    return out


# --------------------------------------------------------------- rotation ----

def hadamard_rotate(x: torch.Tensor, signs1024: torch.Tensor, out: torch.Tensor | None = None,
                    stream=None) -> torch.Tensor:
    """Rotate the rows of x [m, k] (or [k]); out may be x."""
    _dev(x, "x", torch.float32)
    _signs(signs1024, x.device)
    k = x.shape[-1] if x.dim() > 0 else 0
    m = _rows_of(x, k)
    if out is None:
        out = torch.empty_like(x)
    _dev(out, "y", torch.float32, numel=x.numel(), device=x.device)
    _check("hadamard_rotate", lib().hadamard_rotate(_ptr(x), _ptr(out), m, k, _ptr(signs1024),
                                                    _stream(stream)))
    return out


def hadamard_unrotate_rows(table: torch.Tensor, signs1024: torch.Tensor, ids: torch.Tensor | None = None,
                           n_rows: int | None = None, out: torch.Tensor | None = None,
                           stream=None) -> torch.Tensor:
    _dev(table, "table", torch.float32)
    if table.dim() != 2:
        raise ValueError("table must be [n_table, d]")
    _signs(signs1024, table.device)
    n_table, d = table.shape
    if ids is not None:
        _dev(ids, "ids", torch.int32, device=table.device)
        n_rows = ids.numel()
    elif n_rows is None:
        n_rows = n_table
    out = _out(out, "out", (n_rows, d), table.device)
    _check("hadamard_unrotate_rows",
           lib().hadamard_unrotate_rows(_ptr(table), n_table, d, _ptr(ids), n_rows, _ptr(signs1024),
                                        _ptr(out), _stream(stream)))
    return out


# ----------------------------------------------------------------- decode ----

def ptq1_matvec(blocks: torch.Tensor, n: int, k: int, x: torch.Tensor, signs1024: torch.Tensor | None,
                residual: torch.Tensor | None = None, out: torch.Tensor | None = None,
                ws: torch.Tensor | None = None, stream=None, fn: str = "ptq1_matvec") -> torch.Tensor:
    """y = residual + W R x, W tiled (ptq1_tile).  ws: optional scratch of
    at least workspace_bytes("matvec", n, k) bytes."""
    _dev(x, "x", torch.float32, numel=k)
    dv = x.device
    _mat(blocks, "blocks", ptq1_tiled_bytes(n, k), dv)
    _signs(signs1024, dv, required=False)
    _opt(residual, "residual", torch.float32, numel=n, device=dv)
    out = _out(out, "y", (n,), dv)
    ws, wsb = _ws(lib().ptq1_matvec_workspace_bytes(n, k), dv, ws)
    _check(fn, getattr(lib(), fn)(_ptr(blocks), n, k, _ptr(x), _ptr(signs1024), _ptr(residual),
                                  _ptr(out), _ptr(ws), wsb, _stream(stream)))
    return out


def ptq1_matvec_float_peel(blocks, n, k, x, signs1024, residual=None, out=None, ws=None, stream=None):
    """The same matvec with every trit peeled on the float pipeline, eight lanes per block (tiled layout)."""
    return ptq1_matvec(blocks, n, k, x, signs1024, residual, out, ws, stream, fn="ptq1_matvec_float_peel")


def ptq1_gate_up(w_gate: torch.Tensor, w_up: torch.Tensor, f: int, d: int, x: torch.Tensor,
                 signs1024: torch.Tensor | None, g: torch.Tensor | None = None,
                 u: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None):
    _dev(x, "x", torch.float32, numel=d)
    dv = x.device
    tb = ptq1_tiled_bytes(f, d)
    _mat(w_gate, "w_gate", tb, dv)
    _mat(w_up, "w_up", tb, dv)
    _signs(signs1024, dv, required=False)
    g = _out(g, "g", (f,), dv)
    u = _out(u, "u", (f,), dv)
    ws, wsb = _ws(lib().ptq1_gate_up_workspace_bytes(f, d), dv, ws)
    _check("ptq1_gate_up", lib().ptq1_gate_up(_ptr(w_gate), _ptr(w_up), f, d, _ptr(x), _ptr(signs1024),
                                              _ptr(g), _ptr(u), _ptr(ws), wsb, _stream(stream)))
    return g, u


def ptq1_swiglu(g: torch.Tensor, u: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    _dev(g, "g", torch.float32)
    _dev(u, "u", torch.float32, numel=g.numel(), device=g.device)
    if out is None:
        out = torch.empty_like(g)
    _dev(out, "h", torch.float32, numel=g.numel(), device=g.device)
    _check("ptq1_swiglu", lib().ptq1_swiglu(_ptr(g), _ptr(u), _ptr(out), g.numel(), _stream(stream)))
    return out


# ---------------------------------------------------------------- prefill ----

def ptq1_gemm(blocks: torch.Tensor, n: int, k: int, x: torch.Tensor, signs1024: torch.Tensor | None,
              out: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    _dev(x, "x", torch.float32)
    dv = x.device
    m = _rows_of(x, k)
    _mat(blocks, "blocks", ptq1_tiled_bytes(n, k), dv)
    _signs(signs1024, dv, required=False)
    out = _out(out, "y", (m, n), dv)
    ws, wsb = _ws(lib().ptq1_gemm_workspace_bytes(m, n, k), dv, ws)
    _check("ptq1_gemm", lib().ptq1_gemm(_ptr(blocks), n, k, _ptr(x), m, _ptr(signs1024), _ptr(out),
                                        _ptr(ws), wsb, _stream(stream)))
    return out


def ptq1_ffn_block(x: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                   signs1024: torch.Tensor, d: int, f: int, rms_eps: float = 0.0,
                   out: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                   stream=None, rms_gain: torch.Tensor | None = None, fn: str = "ptq1_ffn_block") -> torch.Tensor:
    """x [m, d] -> x + W_down R(silu(W_gate R xn) * (W_up R xn)), xn = a * rms_gain * x (a = RMS
    scale of x when rms_eps > 0; rms_gain [d] or None); out may be x.  fn = "pq2_ffn_block" takes
    PQ2_0 tiled matrices (pq2_tile)."""
    _dev(x, "x", torch.float32)
    dv = x.device
    m = _rows_of(x, d)
    tiled = pq2_tiled_bytes if fn == "pq2_ffn_block" else ptq1_tiled_bytes
    _mat(w_gate, "w_gate", tiled(f, d), dv)
    _mat(w_up, "w_up", tiled(f, d), dv)
    _mat(w_down, "w_down", tiled(d, f), dv)
    _signs(signs1024, dv)
    _opt(rms_gain, "rms_gain", torch.float32, numel=d, device=dv)
    if out is None:
        out = torch.empty_like(x)
    _dev(out, "x_out", torch.float32, numel=m * d, device=dv)
    wsfn = "pq2_ffn_workspace_bytes" if fn == "pq2_ffn_block" else "ptq1_ffn_workspace_bytes"
    ws, wsb = _ws(getattr(lib(), wsfn)(m, d, f), dv, ws)
    _check(fn, getattr(lib(), fn)(_ptr(x), _ptr(out), m, d, f, _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                  _ptr(signs1024), float(rms_eps), _ptr(rms_gain) if rms_gain is not None else None,
                                  _ptr(ws), wsb, _stream(stream)))
    return out


def ptq1_ffn_block_noalloc(x: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                           signs1024: torch.Tensor, d: int, f: int, rms_eps: float = 0.0,
                           out: torch.Tensor | None = None, stream=None,
                           rms_gain: torch.Tensor | None = None) -> torch.Tensor:
    """ptq1_ffn_block on the library's own static scratch buffer (no workspace argument; calls on one GPU
    must not overlap).  `out` must be given by a caller that cannot allocate."""
    _dev(x, "x", torch.float32)
    dv = x.device
    m = _rows_of(x, d)
    _mat(w_gate, "w_gate", ptq1_tiled_bytes(f, d), dv)
    _mat(w_up, "w_up", ptq1_tiled_bytes(f, d), dv)
    _mat(w_down, "w_down", ptq1_tiled_bytes(d, f), dv)
    _signs(signs1024, dv)
    _opt(rms_gain, "rms_gain", torch.float32, numel=d, device=dv)
    if out is None:
        out = torch.empty_like(x)
    _dev(out, "x_out", torch.float32, numel=m * d, device=dv)
    _check("ptq1_ffn_block_noalloc",
           lib().ptq1_ffn_block_noalloc(_ptr(x), _ptr(out), m, d, f, _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                        _ptr(signs1024), float(rms_eps),
                                        _ptr(rms_gain) if rms_gain is not None else None, _stream(stream)))
    return out


def pq2_ffn_block(x, w_gate, w_up, w_down, signs1024, d, f, rms_eps=0.0, out=None, ws=None, stream=None,
                  rms_gain=None):
    """ptq1_ffn_block over PQ2_0 tiled matrices."""
    return ptq1_ffn_block(x, w_gate, w_up, w_down, signs1024, d, f, rms_eps, out, ws, stream, rms_gain,
                          fn="pq2_ffn_block")


# ------------------------------------------------------------------ PQ2_0 ----

PQ2_BLOCK_BYTES = 34


def pq2_packed_bytes(n: int, k: int) -> int:
    return lib().pq2_packed_bytes(n, k)


def pq2_pack(trits: torch.Tensor, scales_f16: torch.Tensor, out: torch.Tensor | None = None,
             stream=None) -> torch.Tensor:
    """int8 trits [n, k] + binary16 bit patterns [n, k/128] -> uint8 [n, k/128*34]."""
    n, k = _trits_scales(trits, scales_f16)
    out = _out(out, "blocks", (n, (k // BLOCK_WEIGHTS) * PQ2_BLOCK_BYTES), trits.device, torch.uint8)
    _check("pq2_pack", lib().pq2_pack(_ptr(trits), _ptr(scales_f16), n, k, _ptr(out), _stream(stream)))
    return out


def pq2_dequant(blocks: torch.Tensor, n: int, k: int, out: torch.Tensor | None = None,
                stream=None) -> torch.Tensor:
    _mat(blocks, "blocks", pq2_packed_bytes(n, k), None)
    out = _out(out, "w", (n, k), blocks.device)
    _check("pq2_dequant", lib().pq2_dequant(_ptr(blocks), n, k, _ptr(out), _stream(stream)))
    return out


def pq2_tiled_bytes(n: int, k: int) -> int:
    return lib().pq2_tiled_bytes(n, k)


def pq2_tile(blocks: torch.Tensor, n: int, k: int, out: torch.Tensor | None = None,
             stream=None) -> torch.Tensor:
    """Packed PQ2_0 [n, k/128*34] uint8 -> the tiled layout pq2_matvec reads (flat uint8)."""
    nbytes = pq2_tiled_bytes(n, k)
    if nbytes < 0:
        raise ValueError(f"bad shape [{n}][{k}]")
    _mat(blocks, "blocks", pq2_packed_bytes(n, k), None)
    out = _out(out, "tiled", (nbytes,), blocks.device, torch.uint8)
    _check("pq2_tile", lib().pq2_tile(_ptr(blocks), n, k, _ptr(out), _stream(stream)))
    return out


def pq2_matvec(tiled: torch.Tensor, n: int, k: int, x: torch.Tensor, signs1024: torch.Tensor | None,
               residual: torch.Tensor | None = None, out: torch.Tensor | None = None,
               ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y = residual + W R x over a PQ2_0 tiled matrix (pq2_tile)."""
    _dev(x, "x", torch.float32, numel=k)
    dv = x.device
    _mat(tiled, "tiled", pq2_tiled_bytes(n, k), dv)
    _signs(signs1024, dv, required=False)
    _opt(residual, "residual", torch.float32, numel=n, device=dv)
    out = _out(out, "y", (n,), dv)
    ws, wsb = _ws(lib().pq2_matvec_workspace_bytes(n, k), dv, ws)
    _check("pq2_matvec", lib().pq2_matvec(_ptr(tiled), n, k, _ptr(x), _ptr(signs1024), _ptr(residual),
                                          _ptr(out), _ptr(ws), wsb, _stream(stream)))
    return out


def pq2_gemm(tiled: torch.Tensor, n: int, k: int, x: torch.Tensor, signs1024: torch.Tensor | None,
             out: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Y [m, n] = bf16(R X) . W^T over a PQ2_0 tiled matrix (pq2_tile)."""
    _dev(x, "x", torch.float32)
    dv = x.device
    m = _rows_of(x, k)
    _mat(tiled, "tiled", pq2_tiled_bytes(n, k), dv)
    _signs(signs1024, dv, required=False)
    out = _out(out, "y", (m, n), dv)
    ws, wsb = _ws(lib().pq2_gemm_workspace_bytes(m, n, k), dv, ws)
    _check("pq2_gemm", lib().pq2_gemm(_ptr(tiled), n, k, _ptr(x), m, _ptr(signs1024), _ptr(out), _ptr(ws), wsb,
                                      _stream(stream)))
    return out


def ptq1_matvec_w2a8(tiled: torch.Tensor, n: int, k: int, x: torch.Tensor, residual: torch.Tensor | None = None,
                     out: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y = residual + W q * step with x quantised to 8-bit integers (per call, absmax)."""
    _dev(x, "x", torch.float32, numel=k)
    dv = x.device
    _mat(tiled, "tiled", ptq1_tiled_bytes(n, k), dv)
    _opt(residual, "residual", torch.float32, numel=n, device=dv)
    out = _out(out, "y", (n,), dv)
    ws, wsb = _ws(lib().ptq1_matvec_w2a8_workspace_bytes(n, k), dv, ws)
    _check("ptq1_matvec_w2a8", lib().ptq1_matvec_w2a8(_ptr(tiled), n, k, _ptr(x), _ptr(residual), _ptr(out),
                                                      _ptr(ws), wsb, _stream(stream)))
    return out


def ptq1_gemm_w2a8(tiled: torch.Tensor, n: int, k: int, x: torch.Tensor, out: torch.Tensor | None = None,
                   ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Y [m, n] with each row of x quantised to 8-bit integers (its own absmax)."""
    _dev(x, "x", torch.float32)
    dv = x.device
    m = _rows_of(x, k)
    _mat(tiled, "tiled", ptq1_tiled_bytes(n, k), dv)
    out = _out(out, "y", (m, n), dv)
    ws, wsb = _ws(lib().ptq1_gemm_w2a8_workspace_bytes(m, n, k), dv, ws)
    _check("ptq1_gemm_w2a8", lib().ptq1_gemm_w2a8(_ptr(tiled), n, k, _ptr(x), m, _ptr(out), _ptr(ws), wsb,
                                                  _stream(stream)))
    return out


def ffn_workspace_offsets(m: int, d: int, f: int, fmt: str = "ptq1") -> tuple[int, int, int]:
    """Byte offsets of (g, u, h) in an FFN block's workspace (-1: not stored on that path)."""
    out = (C.c_int64 * 3)()
    fn = "pq2_ffn_workspace_offsets" if fmt == "pq2" else "ptq1_ffn_workspace_offsets"
    _check(fn, getattr(lib(), fn)(m, d, f, C.cast(out, p)))
    return tuple(out)


def workspace_bytes(kind: str, *shape) -> int:
    fn = {"matvec": "ptq1_matvec_workspace_bytes", "gate_up": "ptq1_gate_up_workspace_bytes",
          "gemm": "ptq1_gemm_workspace_bytes", "ffn": "ptq1_ffn_workspace_bytes",
          "pq2_matvec": "pq2_matvec_workspace_bytes", "pq2_gemm": "pq2_gemm_workspace_bytes"}[kind]
    return int(getattr(lib(), fn)(*shape))


# -------------------------------------------------------------- profiling ----

_hip = None


def _hiprt():
    """The HIP runtime (already loaded by torch), for raw events."""
    global _hip
    if _hip is None:
        h = C.CDLL("libamdhip64.so")
        h.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        h.hipEventDestroy.argtypes = [C.c_void_p]
        h.hipEventSynchronize.argtypes = [C.c_void_p]
        h.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        _hip = h
    return _hip


class KernelTimer:
    """Times the next `count` launches of one kernel family inside any call
    (ptq1_profile_arm): HIP events recorded by the library on the stream of
    each launch.  Use as a context manager around the timed calls, then read
    `durations_ms()` after a device synchronisation."""

    def __init__(self, kernel: str, count: int):
        self.kernel = kernel.encode()
        self.count = count
        hip = _hiprt()
        self._start = (C.c_void_p * count)()
        self._stop = (C.c_void_p * count)()
        for arr in (self._start, self._stop):
            for i in range(count):
                ev = C.c_void_p()
                if hip.hipEventCreate(C.byref(ev)) != 0:
                    raise RuntimeError("hipEventCreate failed")
                arr[i] = ev

    def __enter__(self):
        _check("ptq1_profile_arm", lib().ptq1_profile_arm(self.kernel, C.cast(self._start, p),
                                                          C.cast(self._stop, p), self.count))
        return self

    def __exit__(self, *exc):
        self.launches = lib().ptq1_profile_count(self.kernel)
        _check("ptq1_profile_arm", lib().ptq1_profile_arm(self.kernel, None, None, 0))
        return False

    def durations_ms(self) -> list[float]:
        hip = _hiprt()
        out = []
        for i in range(self.launches):
            if hip.hipEventSynchronize(self._stop[i]) != 0:
                raise RuntimeError("hipEventSynchronize failed")
            ms = C.c_float()
            if hip.hipEventElapsedTime(C.byref(ms), self._start[i], self._stop[i]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out.append(ms.value)
        return out

    def close(self):
        hip = _hiprt()
        for arr in (self._start, self._stop):
            for i in range(self.count):
                if arr[i]:
                    hip.hipEventDestroy(arr[i])
                    arr[i] = None

