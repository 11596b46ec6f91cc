"""fp64 CPU oracle for the PTQ1_0 ternary linear layer (TEST INFRASTRUCTURE).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does, and
this package never imports the product.  The arithmetic lives in
``ptq1_oracle.c`` (plain C loops, fp64, OpenMP over output rows, no SIMD
intrinsics, no BLAS, no fast-math); this module only marshals numpy arrays.

Every function names the passage it follows in ``ptq1_oracle.c``'s header.
Parity status: every function is pinned by ``tests/test_oracle.py``; byte
layout compatibility with third-party PTQ1_0 files is unpinned (no such file
or layout specification is available).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ptq1_oracle.c")
_LIB = os.path.join(_HERE, "libptq1_oracle.so")

BLOCK_W = 128
TRIT_BYTES = 26
BLOCK_BYTES = 28
HAD = 1024


_LIB_SAN = os.path.join(_HERE, "libptq1_oracle_asan.so")
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math, fp64, OpenMP); with
    sanitize, a second copy instrumented by AddressSanitizer and
    UndefinedBehaviorSanitizer (loaded when PTQ1_ORACLE_LIB names it)."""
    out = _LIB_SAN if sanitize else _LIB
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.check_call(
            ["gcc", "-O1" if sanitize else "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
             "-ffp-contract=off", "-Wall", "-Wextra", *(SANITIZE_FLAGS if sanitize else []), "-o", tmp, _SRC,
             "-lm"])
        os.replace(tmp, out)
    return out


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("PTQ1_ORACLE_LIB")
        if path is None:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
        L = C.CDLL(path)
        i64, p = C.c_int64, C.c_void_p
        L.orc_f16_to_f64.argtypes = [C.c_uint16]
        L.orc_f16_to_f64.restype = C.c_double
        L.orc_byte_digits.argtypes = [C.c_uint8, p]
        L.orc_digits_byte.argtypes = [p]
        L.orc_digits_byte.restype = C.c_uint8
        L.orc_pack.argtypes = [p, p, i64, i64, p]
        L.orc_unpack.argtypes = [p, i64, i64, p, p]
        L.orc_dequant.argtypes = [p, i64, i64, p]
        L.orc_pq2_pack.argtypes = [p, p, i64, i64, p]
        L.orc_pq2_unpack.argtypes = [p, i64, i64, p, p]
        L.orc_pq2_dequant.argtypes = [p, i64, i64, p]
        L.orc_hadamard_entry.argtypes = [C.c_int, C.c_int]
        L.orc_hadamard_entry.restype = C.c_double
        L.orc_rotate.argtypes = [p, i64, i64, p, p]
        L.orc_unrotate.argtypes = [p, i64, i64, p, p]
        L.orc_gemm_rows.argtypes = [p, i64, i64, p, i64, p, i64, p]
        L.orc_gemm.argtypes = [p, i64, i64, p, i64, p]
        L.orc_swiglu.argtypes = [p, p, i64, p]
        L.orc_rms_scale.argtypes = [p, i64, i64, C.c_double, p]
        L.orc_ffn_block.argtypes = [p, i64, i64, i64, p, p, p, p, C.c_double, p, p]
        L.orc_set_threads.argtypes = [C.c_int]
        for fn in ("orc_pack", "orc_unpack", "orc_dequant", "orc_rotate", "orc_unrotate",
                   "orc_gemm_rows", "orc_gemm", "orc_ffn_block", "orc_threads",
                   "orc_block_weights", "orc_block_bytes", "orc_block_trit_bytes",
                   "orc_hadamard_width", "orc_pq2_pack", "orc_pq2_unpack", "orc_pq2_dequant",
                   "orc_pq2_block_bytes"):
            getattr(L, fn).restype = C.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments")


def threads() -> int:
    return lib().orc_threads()


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def f16_to_f64(bits) -> np.ndarray:
    """Own binary16 decoder, element-wise over a uint16 array."""
    bits = np.asarray(bits, dtype=np.uint16)
    f = lib().orc_f16_to_f64
    return np.array([f(int(b)) for b in bits.ravel()], dtype=np.float64).reshape(bits.shape)


def byte_digits(b: int) -> list[int]:
    d = (C.c_int * 5)()
    lib().orc_byte_digits(C.c_uint8(b), C.cast(d, C.c_void_p))
    return list(d)


def digits_byte(d) -> int:
    arr = (C.c_int * 5)(*[int(v) for v in d])
    return int(lib().orc_digits_byte(C.cast(arr, C.c_void_p)))


def pack(trits: np.ndarray, scales_f16_bits: np.ndarray) -> np.ndarray:
    """int8 trits [n, k], uint16 fp16 scale bits [n, k/128] -> uint8 blocks [n, k/128*28]."""
    t = np.ascontiguousarray(trits, dtype=np.int8)
    s = np.ascontiguousarray(scales_f16_bits, dtype=np.uint16)
    n, k = t.shape
    out = np.zeros((n, (k // BLOCK_W) * BLOCK_BYTES), dtype=np.uint8)
    _check(lib().orc_pack(_ptr(t), _ptr(s), n, k, _ptr(out)), "pack")
    return out


def unpack(blocks: np.ndarray, n: int, k: int):
    b = np.ascontiguousarray(blocks, dtype=np.uint8)
    t = np.zeros((n, k), dtype=np.int8)
    s = np.zeros((n, k // BLOCK_W), dtype=np.uint16)
    _check(lib().orc_unpack(_ptr(b), n, k, _ptr(t), _ptr(s)), "unpack")
    return t, s


def dequant(blocks: np.ndarray, n: int, k: int) -> np.ndarray:
    b = np.ascontiguousarray(blocks, dtype=np.uint8)
    w = np.zeros((n, k), dtype=np.float64)
    _check(lib().orc_dequant(_ptr(b), n, k, _ptr(w)), "dequant")
    return w


# ---- PQ2_0: 2-bit codes, 4 per byte, then the fp16 scale (34 bytes per 128 weights)

def pq2_pack(trits: np.ndarray, scales_f16_bits: np.ndarray) -> np.ndarray:
    """int8 trits [n, k], uint16 fp16 scale bits [n, k/128] -> uint8 blocks [n, k/128*34]."""
    t = np.ascontiguousarray(trits, dtype=np.int8)
    s = np.ascontiguousarray(scales_f16_bits, dtype=np.uint16)
    n, k = t.shape
    out = np.zeros((n, (k // BLOCK_W) * lib().orc_pq2_block_bytes()), dtype=np.uint8)
    _check(lib().orc_pq2_pack(_ptr(t), _ptr(s), n, k, _ptr(out)), "pq2_pack")
    return out


def pq2_unpack(blocks: np.ndarray, n: int, k: int):
    b = np.ascontiguousarray(blocks, dtype=np.uint8)
    t = np.zeros((n, k), dtype=np.int8)
    s = np.zeros((n, k // BLOCK_W), dtype=np.uint16)
    _check(lib().orc_pq2_unpack(_ptr(b), n, k, _ptr(t), _ptr(s)), "pq2_unpack")
    return t, s


def pq2_dequant(blocks: np.ndarray, n: int, k: int) -> np.ndarray:
    b = np.ascontiguousarray(blocks, dtype=np.uint8)
    w = np.zeros((n, k), dtype=np.float64)
    _check(lib().orc_pq2_dequant(_ptr(b), n, k, _ptr(w)), "pq2_dequant")
    return w


def pq2_matvec(blocks: np.ndarray, n: int, k: int, xr: np.ndarray, rows=None) -> np.ndarray:
    """W xr for a PQ2_0 matrix: the dequantised rows (fp64) times the already rotated x."""
    w = pq2_dequant(blocks, n, k)
    if rows is not None:
        w = w[np.asarray(rows, dtype=np.int64)]
    return w @ _f64(xr).reshape(k)


def pq2_gemm(blocks: np.ndarray, n: int, k: int, xr: np.ndarray, rows=None) -> np.ndarray:
    """Y [m, len(rows) or n] = xr [m, k] . W^T, W the dequantised PQ2_0 rows (fp64)."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(n, -1)
    if rows is not None:
        b = b[np.asarray(rows, dtype=np.int64)]
    w = pq2_dequant(b, b.shape[0], k)
    return _f64(xr).reshape(-1, k) @ w.T


def hadamard_entry(i: int, j: int) -> float:
    return lib().orc_hadamard_entry(int(i), int(j))


def rotate(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """Rows of x [m, k] (k % 1024 == 0): each 1024-chunk -> (1/32) H (s * chunk)."""
    x2 = _f64(x)
    shp = x2.shape
    x2 = x2.reshape(-1, shp[-1])
    y = np.zeros_like(x2)
    _check(lib().orc_rotate(_ptr(x2), x2.shape[0], x2.shape[1], _ptr(_f64(signs)), _ptr(y)), "rotate")
    return y.reshape(shp)


def unrotate(y: np.ndarray, signs: np.ndarray) -> np.ndarray:
    y2 = _f64(y)
    shp = y2.shape
    y2 = y2.reshape(-1, shp[-1])
    x = np.zeros_like(y2)
    _check(lib().orc_unrotate(_ptr(y2), y2.shape[0], y2.shape[1], _ptr(_f64(signs)), _ptr(x)), "unrotate")
    return x.reshape(shp)


def gemm(blocks: np.ndarray, n: int, k: int, xr: np.ndarray, rows=None) -> np.ndarray:
    """Y [m, len(rows) or n] = xr [m, k] . W^T with W the dequantised packed matrix [n, k]."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8)
    x2 = _f64(xr).reshape(-1, k)
    m = x2.shape[0]
    if rows is None:
        y = np.zeros((m, n), dtype=np.float64)
        _check(lib().orc_gemm_rows(_ptr(b), n, k, _ptr(x2), m, None, n, _ptr(y)), "gemm")
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        y = np.zeros((m, len(r)), dtype=np.float64)
        _check(lib().orc_gemm_rows(_ptr(b), n, k, _ptr(x2), m, _ptr(r), len(r), _ptr(y)), "gemm")
    return y


def matvec(blocks: np.ndarray, n: int, k: int, xr: np.ndarray, rows=None) -> np.ndarray:
    return gemm(blocks, n, k, np.asarray(xr).reshape(1, k), rows)[0]


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g2, u2 = _f64(g), _f64(u)
    h = np.zeros_like(g2)
    lib().orc_swiglu(_ptr(g2), _ptr(u2), g2.size, _ptr(h))
    return h


def rms_scale(x: np.ndarray, eps: float) -> np.ndarray:
    x2 = _f64(x)
    x2 = x2.reshape(-1, x2.shape[-1])
    a = np.zeros(x2.shape[0], dtype=np.float64)
    lib().orc_rms_scale(_ptr(x2), x2.shape[0], x2.shape[1], float(eps), _ptr(a))
    return a


def ffn_block(x: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray,
              signs: np.ndarray, d: int, f: int, rms_eps: float, gain: np.ndarray | None = None) -> np.ndarray:
    """x + Wd R(silu(Wg R(a gain x)) * (Wu R(a gain x))): a = RMS scale of x (1 when rms_eps <= 0),
    gain [d] the norm's per-channel weight (None: all ones)."""
    x2 = _f64(x).reshape(-1, d)
    m = x2.shape[0]
    out = np.zeros_like(x2)
    args = [np.ascontiguousarray(w, dtype=np.uint8) for w in (wg, wu, wd)]
    gv = None if gain is None else _f64(gain).reshape(d)
    _check(lib().orc_ffn_block(_ptr(x2), m, d, f, _ptr(args[0]), _ptr(args[1]), _ptr(args[2]),
                               _ptr(_f64(signs)), float(rms_eps), _ptr(gv) if gv is not None else None,
                               _ptr(out)), "ffn_block")
    return out


def pq2_ffn_block(x: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray, signs: np.ndarray, d: int,
                  f: int, rms_eps: float, gain: np.ndarray | None = None) -> np.ndarray:
    """ffn_block over PQ2_0 matrices, composed step by step from the oracle's
    rotate, PQ2_0 product, SwiGLU and RMS scale (the same definition)."""
    x2 = _f64(x).reshape(-1, d)
    xn = x2 * (rms_scale(x2, rms_eps).reshape(-1, 1) if rms_eps > 0 else 1.0)
    if gain is not None:
        xn = xn * _f64(gain).reshape(1, d)
    xr = rotate(xn, signs)
    g = pq2_gemm(wg, f, d, xr)
    u = pq2_gemm(wu, f, d, xr)
    h = swiglu(g, u)
    return x2 + pq2_gemm(wd, d, f, rotate(h, signs))


def w2a8_quant(x: np.ndarray):
    """8-bit activations ("Why I Am Building Another Inference Engine", Level 5:
    integer kernels pair ternary weights with int8 activations; Level 4: a
    BitNet layer rounds its activations to int8 ahead of its ternary matmuls).
    Reading (the pages name the step, not its formula): one absmax scale per
    call, c = 127 / max|x| rounded once to fp32 (0 for an all-zero x), then
    q = rint(x * c) in fp32 with ties to even; the step back is max|x| / 127.
    The decisions are taken in fp32, as the kernel takes them."""
    x32 = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    g = float(np.max(np.abs(x32))) if x32.size else 0.0
    c = np.float32(127.0 / g) if g > 0.0 else np.float32(0.0)
    q = np.rint(x32 * c).astype(np.int64)
    return q, g / 127.0


def w2a8_matvec(blocks: np.ndarray, n: int, k: int, x: np.ndarray, rows=None) -> np.ndarray:
    """step * sum_b scale_rb * (integer sum over block b of trit * q), the
    per-block sums in exact integer arithmetic (W2A8)."""
    q, step = w2a8_quant(x)
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(n, -1)
    if rows is not None:
        b = b[np.asarray(rows, dtype=np.int64)]
    nr, nb = b.shape[0], k // BLOCK_W
    t, sc = unpack(b, nr, k)
    isum = (t.reshape(nr, nb, BLOCK_W).astype(np.int64) * q.reshape(1, nb, BLOCK_W)).sum(axis=2)
    return step * (f16_to_f64(sc).reshape(nr, nb) * isum).sum(axis=1)


def w2a8_gemm(blocks: np.ndarray, n: int, k: int, x: np.ndarray, rows=None) -> np.ndarray:
    """Y [m, len(rows) or n]: every row of x quantised on its own (one absmax
    per token), then the W2A8 product of w2a8_matvec."""
    x2 = np.asarray(x, dtype=np.float32).reshape(-1, k)
    return np.stack([w2a8_matvec(blocks, n, k, xi, rows=rows) for xi in x2])


def embedding_unrotate(table_rows: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """Restore looked-up rows of a rotated embedding table: unrotate each row."""
    return unrotate(table_rows, signs)
