"""Seeded synthetic inputs for the ternary linear layer (test and bench infrastructure).

This module is shared by both sides of every parity check: it produces the raw
inputs (trits, fp16 scale bit patterns, fp32 activations, sign vectors,
embedding tables) and nothing else. It contains none of the method's
arithmetic: no packing, no decoding, no rotation, no products.

Generator definition (counter-based, so any element can be regenerated alone):

  mix64(z)       SplitMix64 output finaliser (Steele, Lea & Flood, "Fast
                 splittable pseudorandom number generators", OOPSLA 2014):
                   z ^= z >> 30; z *= 0xBF58476D1CE4E5B9
                   z ^= z >> 27; z *= 0x94D049BB133111EB
                   z ^= z >> 31
  key(S, s)      mix64(S * 0x9E3779B97F4A7C15 + s * 0xD1B54A32D192ED03 + 1)
  draw(S, s, i)  mix64(key(S, s) + (i + 1) * 0x9E3779B97F4A7C15)

  all arithmetic modulo 2**64.  Element i of stream s under seed S is draw(S, s, i).

Distributions (all decisions are integer comparisons on the 64-bit draw, so a
device implementation of the same definition reproduces them bit for bit):

  trit       r = draw >> 11 (53 bits); -1 if r < T1, 0 if r < T2, else +1,
             T1 = 0.3 * 2**53, T2 = 0.7 * 2**53  ->  P(0) = 0.4, P(+-1) = 0.3.
  scale      fp16 bit pattern SCALE_TABLE[draw >> 48]; SCALE_TABLE[j] is the
             fp16 (round-to-nearest-even) of exp(ln 0.02 + 0.3 * z_j) with
             z_j = Phi^-1((j + 0.5) / 65536): a log-normal with median 0.02 and
             sigma 0.3 sampled by 16-bit inverse CDF.
  gauss      GAUSS_TABLE[draw >> 48], GAUSS_TABLE[j] = fp32(Phi^-1((j + 0.5) / 65536)).
  sign       -1.0f if draw >> 63 == 1 else +1.0f.
  channel    floor((draw >> 11) * K / 2**53), distinct by rejection in draw order.

Stream ids for each tensor role are fixed below; layer L of a stack offsets
them by 16 * L.
"""
from __future__ import annotations

import numpy as np

M64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
STREAM_MUL = 0xD1B54A32D192ED03
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB

T1 = int(0.3 * (1 << 53))
T2 = int(0.7 * (1 << 53))

# stream roles
S_GATE_TRITS, S_GATE_SCALES = 1, 2
S_UP_TRITS, S_UP_SCALES = 3, 4
S_DOWN_TRITS, S_DOWN_SCALES = 5, 6
S_X, S_OUTLIERS, S_SIGNS = 7, 8, 9
S_TABLE, S_IDS = 10, 11
S_W_TRITS, S_W_SCALES = 12, 13  # a lone matrix (matvec / gemm configs)

N_OUTLIERS = 8
OUTLIER_GAIN = np.float32(50.0)


def layer_stream(role: int, layer: int) -> int:
    return role + 16 * layer


def _mix_np(z: np.ndarray) -> np.ndarray:
    z = z ^ (z >> np.uint64(30))
    z = z * np.uint64(MIX1)
    z = z ^ (z >> np.uint64(27))
    z = z * np.uint64(MIX2)
    return z ^ (z >> np.uint64(31))


def _mix_int(z: int) -> int:
    z &= M64
    z ^= z >> 30
    z = (z * MIX1) & M64
    z ^= z >> 27
    z = (z * MIX2) & M64
    return z ^ (z >> 31)


def stream_key(seed: int, stream: int) -> int:
    return _mix_int((seed * GOLDEN + stream * STREAM_MUL + 1) & M64)


def draws(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """draw(seed, stream, i) for i in [start, start + count) as uint64."""
    key = np.uint64(stream_key(seed, stream))
    with np.errstate(over="ignore"):
        idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        return _mix_np(key + idx * np.uint64(GOLDEN))


def draws_at(seed: int, stream: int, idx: np.ndarray) -> np.ndarray:
    key = np.uint64(stream_key(seed, stream))
    with np.errstate(over="ignore"):
        i = np.asarray(idx, dtype=np.uint64) + np.uint64(1)
        return _mix_np(key + i * np.uint64(GOLDEN))


def _tables():
    from scipy.special import ndtri

    j = np.arange(65536, dtype=np.float64)
    z = ndtri((j + 0.5) / 65536.0)
    gauss = z.astype(np.float32)
    scale = np.exp(np.log(0.02) + 0.3 * z).astype(np.float16).view(np.uint16)
    return gauss, scale


GAUSS_TABLE, SCALE_TABLE = _tables()


def trits_from_draws(d: np.ndarray) -> np.ndarray:
    r = d >> np.uint64(11)
    t = np.full(d.shape, 1, dtype=np.int8)
    t[r < np.uint64(T2)] = 0
    t[r < np.uint64(T1)] = -1
    return t


def trits(seed: int, stream: int, n: int, k: int, row0: int = 0) -> np.ndarray:
    """int8 [n, k] trits of rows row0..row0+n of an [*, k] matrix."""
    d = draws(seed, stream, row0 * k, n * k)
    return trits_from_draws(d).reshape(n, k)


def trits_rows(seed: int, stream: int, rows: np.ndarray, k: int) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.int64)
    idx = (rows[:, None] * k + np.arange(k, dtype=np.int64)[None, :]).ravel()
    return trits_from_draws(draws_at(seed, stream, idx)).reshape(len(rows), k)


def scales(seed: int, stream: int, n: int, nb: int, row0: int = 0) -> np.ndarray:
    """uint16 fp16 bit patterns [n, nb] (one per 128-weight block)."""
    d = draws(seed, stream, row0 * nb, n * nb)
    return SCALE_TABLE[(d >> np.uint64(48)).astype(np.int64)].reshape(n, nb)


def scales_rows(seed: int, stream: int, rows: np.ndarray, nb: int) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.int64)
    idx = (rows[:, None] * nb + np.arange(nb, dtype=np.int64)[None, :]).ravel()
    d = draws_at(seed, stream, idx)
    return SCALE_TABLE[(d >> np.uint64(48)).astype(np.int64)].reshape(len(rows), nb)


def gauss(seed: int, stream: int, count: int, start: int = 0) -> np.ndarray:
    d = draws(seed, stream, start, count)
    return GAUSS_TABLE[(d >> np.uint64(48)).astype(np.int64)]


def gauss_at(seed: int, stream: int, idx: np.ndarray) -> np.ndarray:
    d = draws_at(seed, stream, idx)
    return GAUSS_TABLE[(d >> np.uint64(48)).astype(np.int64)]


def outlier_channels(seed: int, stream: int, k: int, count: int = N_OUTLIERS) -> np.ndarray:
    chosen: list[int] = []
    i = 0
    while len(chosen) < min(count, k):
        d = int(draws(seed, stream, i, 1)[0])
        c = ((d >> 11) * k) >> 53
        if c not in chosen:
            chosen.append(c)
        i += 1
    return np.array(chosen, dtype=np.int64)


def activations(seed: int, m: int, k: int, stream: int = S_X,
                outlier_stream: int = S_OUTLIERS) -> np.ndarray:
    """fp32 [m, k]: N(0,1) with N_OUTLIERS channels (same for every row) x50."""
    x = gauss(seed, stream, m * k).reshape(m, k).copy()
    ch = outlier_channels(seed, outlier_stream, k)
    x[:, ch] *= OUTLIER_GAIN
    return x


def signs(seed: int, stream: int = S_SIGNS, n: int = 1024) -> np.ndarray:
    d = draws(seed, stream, 0, n)
    return np.where((d >> np.uint64(63)) == np.uint64(1), np.float32(-1.0), np.float32(1.0)).astype(np.float32)


def table_rows(seed: int, stream: int, rows: np.ndarray, d: int) -> np.ndarray:
    """fp32 rows of a synthetic [V, d] embedding table, element (r, c) = gauss index r*d + c."""
    rows = np.asarray(rows, dtype=np.int64)
    idx = (rows[:, None] * d + np.arange(d, dtype=np.int64)[None, :]).ravel()
    return gauss_at(seed, stream, idx).reshape(len(rows), d)


def token_ids(seed: int, count: int, vocab: int, stream: int = S_IDS) -> np.ndarray:
    d = draws(seed, stream, 0, count)
    return (((d >> np.uint64(11)).astype(object) * vocab) >> 53).astype(np.int32)
