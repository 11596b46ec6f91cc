"""Pins for the fp64 oracle against facts the pages and mathematics fix.

Each test names the passage (page title, section) or the mathematical fact
it checks.  No expected value here comes from the HIP path.
"""
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PAGE1 = "A 27B model in 5.5 GB: Bonsai ternary on Ferrox, locally"


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            if line.startswith("#") or ":" not in line:
                continue
            key, val = line.split(":", 1)
            out[key.strip()] = val.strip()
    return out


# ---------------------------------------------------------------- codec ----

def test_float_peel_equals_integer_digits_all_bytes():
    """S1 [page 1, "What Ferrox does with it"]: trit n = floor(3^(n+1) u) -
    3 floor(3^n u), u = b/256, exact in fp32.  Evaluated here in fp32 and fp64
    for all 256 bytes and all five digits; the oracle's integer route must
    agree everywhere."""
    b = np.arange(256)
    u32 = b.astype(np.float32) / np.float32(256.0)
    u64 = b.astype(np.float64) / 256.0
    for n in range(5):
        p_hi32, p_lo32 = np.float32(3.0 ** (n + 1)), np.float32(3.0 ** n)
        peel32 = np.floor(p_hi32 * u32) - np.float32(3.0) * np.floor(p_lo32 * u32)
        peel64 = np.floor(3.0 ** (n + 1) * u64) - 3.0 * np.floor(3.0 ** n * u64)
        ref = np.array([oracle.byte_digits(int(v))[n] for v in b])
        assert peel32.dtype == np.float32
        np.testing.assert_array_equal(peel32.astype(np.int64), ref)
        np.testing.assert_array_equal(peel64.astype(np.int64), ref)
        assert set(ref.tolist()) <= {0, 1, 2}


def test_all_243_codes_round_trip():
    """S2 [page 1, "What Bonsai is": five trits in a byte, base 3]: every one
    of the 3^5 = 243 digit patterns encodes to a distinct byte and decodes
    back; code 242 (all digits 2) is byte 255; every byte decodes."""
    seen = {}
    for v in range(243):
        d = [(v // 3 ** (4 - n)) % 3 for n in range(5)]
        byte = oracle.digits_byte(d)
        assert 0 <= byte <= 255
        assert oracle.byte_digits(byte) == d
        assert byte not in seen
        seen[byte] = v
    assert oracle.digits_byte([2, 2, 2, 2, 2]) == 255
    assert oracle.digits_byte([0, 0, 0, 0, 0]) == 0
    # 256 bytes onto 243 codes: 13 codes are carried by two bytes; the encoder
    # must pick the smaller one, so the 13 larger bytes are never produced
    codes_of_bytes = [tuple(oracle.byte_digits(b)) for b in range(256)]
    assert len(set(codes_of_bytes)) == 243
    unused = sorted(set(range(256)) - set(seen))
    assert len(unused) == 13
    for b in unused:
        assert codes_of_bytes[b] == codes_of_bytes[b - 1]  # duplicate of its predecessor


def test_worked_block_bytes():
    """Golden block derived by hand in tests/golden/ptq1_worked_block.txt."""
    g = _golden("ptq1_worked_block.txt")
    t = np.zeros((1, 128), dtype=np.int8)
    for item in g["trits_nonzero"].split():
        k, v = item.split(":")
        t[0, int(k)] = int(v)
    s = np.array([[int(g["scale_f16"], 16)]], dtype=np.uint16)
    blocks = oracle.pack(t, s)
    expect = np.array([int(v) for v in g["bytes"].split()], dtype=np.uint8)
    np.testing.assert_array_equal(blocks[0], expect)
    w = oracle.dequant(blocks, 1, 128)
    np.testing.assert_array_equal(w[0], t[0].astype(np.float64))
    x = np.arange(1, 129, dtype=np.float64)
    assert oracle.matvec(blocks, 1, 128, x)[0] == float(g["dot_with_k_plus_1"])


def test_pack_unpack_round_trip_random():
    t = synth.trits(5, synth.S_W_TRITS, 7, 384)
    s = synth.scales(5, synth.S_W_SCALES, 7, 3)
    blocks = oracle.pack(t, s)
    assert blocks.shape == (7, 3 * 28)
    t2, s2 = oracle.unpack(blocks, 7, 384)
    np.testing.assert_array_equal(t, t2)
    np.testing.assert_array_equal(s, s2)
    # padding digits of byte 25 are written as 1
    for blk in blocks.reshape(-1, 28):
        d = oracle.byte_digits(int(blk[25]))
        assert d[3] == 1 and d[4] == 1


def test_pack_refuses_bad_input():
    with pytest.raises(ValueError):
        oracle.pack(np.zeros((1, 100), np.int8), np.zeros((1, 1), np.uint16))
    bad = np.zeros((1, 128), np.int8)
    bad[0, 3] = 2
    with pytest.raises(ValueError):
        oracle.pack(bad, np.zeros((1, 1), np.uint16))


def test_byte_accounting():
    """S3 [page 1, intro and "What Bonsai is"]: 1.75 bits per weight and
    5.5 GB for 27 billion weights."""
    assert oracle.lib().orc_block_bytes() == 28
    assert oracle.lib().orc_block_trit_bytes() == 26
    assert oracle.lib().orc_block_weights() == 128
    bits_per_weight = 28 * 8 / 128
    assert bits_per_weight == 1.75
    size = 27e9 * bits_per_weight / 8
    assert abs(size / 2 ** 30 - 5.5) < 0.01  # the page's 5.5 GB, read as GiB
    t = np.zeros((17408, 128), np.int8)
    s = np.zeros((17408, 1), np.uint16)
    assert oracle.pack(t, s).nbytes == 17408 * 28
    assert 17408 * (5120 // 128) * 28 == 19_496_960


def test_f16_decoder_exhaustive():
    """The oracle's own binary16 decoder against numpy's float16, all 65536
    bit patterns (the scale is 16-bit [page 1, "What Bonsai is"]; read as IEEE
    binary16)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_dequant_scale_edge_cases():
    t = np.ones((1, 256), np.int8)
    t[0, 1::2] = -1
    s = np.array([[0x0000, 0xC000]], dtype=np.uint16)  # 0.0 and -2.0
    w = oracle.dequant(oracle.pack(t, s), 1, 256)
    np.testing.assert_array_equal(w[0, :128], 0.0 * t[0, :128])
    np.testing.assert_array_equal(w[0, 128:], -2.0 * t[0, 128:].astype(np.float64))


# ------------------------------------------------------------- Hadamard ----

def _fwht_textbook(v):
    """Iterative in-place fast Walsh-Hadamard transform (natural order), a
    different algorithm from the oracle's dense popcount definition."""
    a = np.array(v, dtype=np.float64)
    h = 1
    while h < len(a):
        for i in range(0, len(a), 2 * h):
            x = a[i:i + h].copy()
            y = a[i + h:i + 2 * h].copy()
            a[i:i + h] = x + y
            a[i + h:i + 2 * h] = x - y
        h *= 2
    return a


def test_hadamard_matrix_is_sylvester():
    """S4 [page 1, "What Bonsai is": a 1024-wide Walsh-Hadamard butterfly]:
    the oracle's dense matrix equals scipy's Sylvester construction and
    H H^T = 1024 I exactly."""
    from scipy.linalg import hadamard

    ones = np.ones(1024)
    H = 32.0 * oracle.rotate(np.eye(1024), ones)  # row j = (1/32) H e_j; H symmetric
    Href = hadamard(1024).astype(np.float64)
    np.testing.assert_array_equal(H, Href)
    np.testing.assert_array_equal(H @ H.T, 1024.0 * np.eye(1024))
    for i, j in [(0, 0), (1, 1), (3, 5), (1023, 1023), (512, 768)]:
        assert oracle.hadamard_entry(i, j) == Href[i, j]


def test_rotation_closed_forms():
    s = synth.signs(3)
    e0 = np.zeros(1024)
    e0[0] = 1.0
    np.testing.assert_array_equal(oracle.rotate(e0, s), np.full(1024, s[0] / 32.0))
    np.testing.assert_array_equal(oracle.rotate(np.ones(1024), np.ones(1024)), 32.0 * e0)
    # signs first, then the butterfly: rotate(x) = (1/32) H (s * x)
    x = synth.gauss(4, 99, 1024).astype(np.float64)
    np.testing.assert_allclose(oracle.rotate(x, s), _fwht_textbook(s * x) / 32.0, rtol=0, atol=1e-13)


def test_rotation_orthogonal_and_invertible():
    s = synth.signs(1)
    x = synth.activations(1, 3, 5120).astype(np.float64)
    y = oracle.rotate(x, s)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    np.testing.assert_allclose(oracle.unrotate(y, s), x, rtol=0, atol=1e-12)
    # chunks are independent: the 3rd chunk of the rotated row is the rotation of the 3rd chunk
    np.testing.assert_array_equal(y[:, 2048:3072], oracle.rotate(x[:, 2048:3072], s))
    # outliers are spread: max |y| is far below the x50 outlier magnitude
    assert np.abs(y).max() < 0.5 * np.abs(x).max()


def test_rotate_refuses_ragged_width():
    with pytest.raises(ValueError):
        oracle.rotate(np.zeros((1, 1536)), np.ones(1024))


def test_fold_invariant():
    """S5 [page 1, "What Bonsai is": the rotation is folded into the stored
    weights, and the same rotation is applied to the activations]: with
    W' = rows of W rotated, W' (R x) = W x, for dense fp64 W."""
    rng = np.random.default_rng(0)
    s = synth.signs(7)
    for n, k in [(8, 1024), (64, 2048)]:
        W = rng.standard_normal((n, k))
        x = rng.standard_normal(k)
        Wf = oracle.rotate(W, s)
        np.testing.assert_allclose(Wf @ oracle.rotate(x, s), W @ x, rtol=1e-12, atol=1e-12)
        # and embedding rows stored rotated are restored by unrotate
        np.testing.assert_allclose(oracle.embedding_unrotate(Wf, s), W, rtol=0, atol=1e-12)


# --------------------------------------------------------- matvec / GEMM ----

def test_gemm_is_dense_product_of_dequantised_weights():
    """S6: the matvec / GEMM reduces to the textbook dense product of the
    dequantised matrix (numpy matmul on the oracle's dequant)."""
    n, k, m = 37, 1024, 3
    t = synth.trits(2, synth.S_W_TRITS, n, k)
    s = synth.scales(2, synth.S_W_SCALES, n, k // 128)
    blocks = oracle.pack(t, s)
    x = synth.activations(2, m, k).astype(np.float64)
    W = oracle.dequant(blocks, n, k)
    # dequant itself: trit times the fp16 scale of its block
    sf = s.view(np.float16).astype(np.float64)
    np.testing.assert_array_equal(W, t * np.repeat(sf, 128, axis=1))
    Y = oracle.gemm(blocks, n, k, x)
    np.testing.assert_allclose(Y, x @ W.T, rtol=1e-12, atol=1e-12)
    rows = np.array([36, 0, 5])
    np.testing.assert_array_equal(oracle.gemm(blocks, n, k, x, rows=rows), Y[:, rows])
    np.testing.assert_array_equal(oracle.matvec(blocks, n, k, x[1]), Y[1])


def test_gemm_special_cases():
    k = 512
    x = synth.gauss(9, 1, k).astype(np.float64)
    # all-zero trits -> exactly zero
    z = oracle.pack(np.zeros((4, k), np.int8), np.full((4, 4), 0x3C00, np.uint16))
    np.testing.assert_array_equal(oracle.matvec(z, 4, k, x), np.zeros(4))
    # all +1 trits, scale 1 -> sum of the activations
    o = oracle.pack(np.ones((2, k), np.int8), np.full((2, 4), 0x3C00, np.uint16))
    np.testing.assert_allclose(oracle.matvec(o, 2, k, x), np.full(2, x.sum()), rtol=1e-14)
    # a zero scale removes exactly its block
    sc = np.full((1, 4), 0x3C00, np.uint16)
    sc[0, 2] = 0
    b = oracle.pack(np.ones((1, k), np.int8), sc)
    expect = x[:256].sum() + x[384:].sum()
    np.testing.assert_allclose(oracle.matvec(b, 1, k, x)[0], expect, rtol=1e-14)


def test_gemm_brute_force_tiny():
    """Brute force from trits and decoded scales with pure-Python loops."""
    n, k = 3, 256
    t = synth.trits(11, synth.S_W_TRITS, n, k)
    s = synth.scales(11, synth.S_W_SCALES, n, 2)
    x = synth.gauss(11, 5, 2 * k).reshape(2, k).astype(np.float64)
    sf = s.view(np.float16).astype(np.float64)
    ref = np.zeros((2, n))
    for i in range(2):
        for r in range(n):
            acc = 0.0
            for q in range(k):
                acc += x[i, q] * sf[r, q // 128] * int(t[r, q])
            ref[i, r] = acc
    np.testing.assert_allclose(oracle.gemm(oracle.pack(t, s), n, k, x), ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------- SwiGLU / FFN ----

def test_swiglu_closed_forms():
    """[page 1, "Speed, and where it goes": the block is gate, SwiGLU, down];
    silu(g) u with silu(z) = z * sigmoid(z), checked against scipy's expit."""
    from scipy.special import expit

    g = np.array([0.0, 1.0, -1.0, 20.0, -30.0, 3.5])
    u = np.array([5.0, 2.0, 2.0, 1.0, 1.0, -1.0])
    h = oracle.swiglu(g, u)
    np.testing.assert_allclose(h, g * expit(g) * u, rtol=1e-14, atol=1e-300)
    assert h[0] == 0.0
    assert abs(h[1] - 2.0 / (1.0 + np.exp(-1.0))) < 1e-15


def test_rms_scale():
    x = np.full((2, 1024), 3.0)
    x[1] = -0.5
    a = oracle.rms_scale(x, 1e-6)
    np.testing.assert_allclose(a, [1 / np.sqrt(9 + 1e-6), 1 / np.sqrt(0.25 + 1e-6)], rtol=1e-15)
    np.testing.assert_array_equal(oracle.rms_scale(x, 0.0), [1.0, 1.0])


def _ffn_weights(seed, d, f):
    mats = []
    for (tr, sc, n, k) in [(synth.S_GATE_TRITS, synth.S_GATE_SCALES, f, d),
                           (synth.S_UP_TRITS, synth.S_UP_SCALES, f, d),
                           (synth.S_DOWN_TRITS, synth.S_DOWN_SCALES, d, f)]:
        mats.append(oracle.pack(synth.trits(seed, tr, n, k), synth.scales(seed, sc, n, k // 128)))
    return mats


# --------------------------------------------------------------- PQ2_0 ----

def test_pq2_worked_block_and_accounting():
    """[page 2, Level 2]: 2 bits per weight + a 16-bit scale for every 128 weights
    = 2.125 bits per weight, 7.2 GB for 27e9 weights; the block in the fixture
    is worked out by hand."""
    g = _golden("pq2_worked_block.txt")
    assert int(g["block_bytes"]) * 8 / 128 == float(g["bits_per_weight"])
    assert int(27e9) * int(g["block_bytes"]) // 128 == int(g["bytes_27e9_weights"])
    assert round(int(g["bytes_27e9_weights"]) / 1e9, 1) == 7.2
    t = np.zeros((1, 128), np.int8)
    t[0, :4] = [-1, 0, 1, 0]
    t[0, 124:] = [1, 1, -1, 0]
    b = oracle.pq2_pack(t, np.array([[0x4000]], np.uint16))[0]
    assert b.size == int(g["block_bytes"])
    assert b[0] == int(g["first_byte"]) and np.all(b[1:31] == int(g["middle_byte"]))
    assert b[31] == int(g["last_code_byte"])
    assert b[32:34].tolist() == [int(v) for v in g["scale_bytes"].split()]
    w = oracle.pq2_dequant(b[None, :], 1, 128)[0]
    assert w @ np.arange(1, 129, dtype=np.float64) == float(g["dot_with_k_plus_1"])


def test_pq2_all_codes_round_trip():
    """Every group of four trits maps to the byte sum (t_n + 1) 4^n and back;
    code 3 (never written) decodes as weight 0."""
    groups = np.array(np.meshgrid(*[[-1, 0, 1]] * 4, indexing="ij")).reshape(4, -1).T  # 81 x 4
    groups = np.concatenate([groups, groups[:15]])  # 96 groups: three whole blocks
    t = groups.reshape(-1, 128).astype(np.int8)
    sc = np.full((t.shape[0], 1), 0x3C00, np.uint16)
    b = oracle.pq2_pack(t, sc)
    codes = b.reshape(t.shape[0], 34)[:, :32].reshape(-1)
    want = ((groups[: codes.size] + 1) * (4 ** np.arange(4))).sum(axis=1)
    np.testing.assert_array_equal(codes, want)
    t2, sc2 = oracle.pq2_unpack(b, t.shape[0], 128)
    np.testing.assert_array_equal(t2, t)
    np.testing.assert_array_equal(sc2, sc)
    # every byte decodes; fields equal to 3 give 0
    blk = np.zeros((1, 34), np.uint8)
    blk[0, :32] = [0xFF, 0x3F, 0xC0, 0x1B] * 8  # fields low to high: 3333, 3330, 0003, 3210
    blk[0, 33] = 0x3C
    tb, _ = oracle.pq2_unpack(blk, 1, 128)
    np.testing.assert_array_equal(tb[0, :16], [0, 0, 0, 0, 0, 0, 0, -1, -1, -1, -1, 0, 0, 1, 0, -1])


def test_pq2_dequant_is_scale_times_trit():
    rng = np.random.default_rng(3)
    t = rng.integers(-1, 2, size=(5, 384)).astype(np.int8)
    sc = rng.integers(0x1000, 0x5000, size=(5, 3)).astype(np.uint16)
    w = oracle.pq2_dequant(oracle.pq2_pack(t, sc), 5, 384)
    ref = t.astype(np.float64) * np.repeat(sc.view(np.float16).astype(np.float64), 128, axis=1)
    np.testing.assert_array_equal(w, ref)


def test_ffn_block_composition():
    """[page 1, "What Bonsai is" + "Speed, and where it goes"; page 2, Level 4]:
    x + Wd R(silu(Wg R(a gain x)) * (Wu R(a gain x))), composed here from numpy
    matmuls on dequantised weights and the textbook FWHT; the RMS scale a
    comes from x itself, the per-channel gain (the layer's norm weight) scales
    the input of the rotation."""
    from scipy.special import expit

    d, f, m = 1024, 2048, 2
    wg, wu, wd = _ffn_weights(3, d, f)
    s = synth.signs(3)
    x = synth.activations(3, m, d).astype(np.float64)
    gain = 0.5 + synth.gauss(3, 7, d).astype(np.float64) ** 2
    for eps, gv in ((0.0, None), (1e-6, None), (1e-6, gain), (0.0, gain)):
        out = oracle.ffn_block(x, wg, wu, wd, s, d, f, eps, gain=gv)
        a = np.ones(m) if eps <= 0 else 1.0 / np.sqrt((x * x).mean(axis=1) + eps)

        def rot(v):
            return np.stack([np.concatenate([_fwht_textbook(s * c) / 32.0
                                             for c in row.reshape(-1, 1024)]) for row in v])

        xr = rot(a[:, None] * (np.ones(d) if gv is None else gv)[None, :] * x)
        g = xr @ oracle.dequant(wg, f, d).T
        u = xr @ oracle.dequant(wu, f, d).T
        h = g * expit(g) * u
        ref = x + rot(h) @ oracle.dequant(wd, d, f).T
        np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-9)


def test_ffn_block_unit_gain_is_no_gain():
    d, f = 1024, 1024
    wg, wu, wd = _ffn_weights(5, d, f)
    x = synth.activations(5, 2, d).astype(np.float64)
    s = synth.signs(5)
    np.testing.assert_array_equal(oracle.ffn_block(x, wg, wu, wd, s, d, f, 1e-6, gain=np.ones(d)),
                                  oracle.ffn_block(x, wg, wu, wd, s, d, f, 1e-6))


def test_ffn_block_zero_down_is_identity():
    d, f = 1024, 1024
    wg, wu, _ = _ffn_weights(4, d, f)
    wd = oracle.pack(np.zeros((d, f), np.int8), np.full((d, f // 128), 0x3C00, np.uint16))
    x = synth.activations(4, 1, d).astype(np.float64)
    np.testing.assert_array_equal(oracle.ffn_block(x, wg, wu, wd, synth.signs(4), d, f, 1e-6), x)


# ------------------------------------------------------------ generator ----

def test_generator_mixer_matches_published_vector():
    g = _golden("splitmix64_vector.txt")
    state = int(g["seed"])
    outs = []
    for _ in range(5):
        state = (state + synth.GOLDEN) & synth.M64
        outs.append(synth._mix_int(state))
    assert outs == [int(v) for v in g["outputs"].split()]


def test_generator_counter_based_and_distributions():
    a = synth.trits(0, synth.S_W_TRITS, 64, 1024)
    b = synth.trits_rows(0, synth.S_W_TRITS, np.array([10, 63]), 1024)
    np.testing.assert_array_equal(a[[10, 63]], b)
    np.testing.assert_array_equal(synth.trits(0, synth.S_W_TRITS, 2, 1024, row0=10), a[10:12])
    assert abs((a == 0).mean() - 0.4) < 0.01
    sc = synth.scales(0, synth.S_W_SCALES, 4096, 8).view(np.float16).astype(np.float64)
    assert np.all(np.isfinite(sc)) and np.all(sc > 6.2e-5)  # positive normal fp16
    assert abs(np.median(sc) - 0.02) < 5e-4
    assert abs(np.log(sc).std() - 0.3) < 0.01
    x = synth.activations(0, 1, 1024)
    assert x.dtype == np.float32 and len(synth.outlier_channels(0, synth.S_OUTLIERS, 1024)) == 8
    s = synth.signs(0)
    assert set(np.unique(s).tolist()) == {-1.0, 1.0}


def test_pq2_gemm_is_rowwise_matvec():
    """The PQ2_0 GEMM oracle row by row equals the matvec oracle (and a
    sampled-row call equals the same rows of the whole product)."""
    n, k, m = 37, 384, 3
    rng = np.random.default_rng(2)
    t = rng.integers(-1, 2, size=(n, k), dtype=np.int8)
    s = np.full((n, k // 128), 0x3C00, np.uint16)
    b = oracle.pq2_pack(t, s)
    x = rng.standard_normal((m, k))
    y = oracle.pq2_gemm(b, n, k, x)
    for i in range(m):
        np.testing.assert_allclose(y[i], oracle.pq2_matvec(b, n, k, x[i]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(y, x @ t.astype(np.float64).T, rtol=0, atol=1e-12)
    rows = [0, 5, 36]
    np.testing.assert_allclose(oracle.pq2_gemm(b, n, k, x, rows=rows), y[:, rows], rtol=0, atol=1e-12)


def test_pq2_ffn_block_equals_ptq1_block_on_the_same_weights():
    """The same trits and scales packed in both formats give the same block:
    the PQ2_0 composition (numpy steps over the PQ2_0 product) against the C
    oracle's PTQ1_0 block, with and without the RMS scale and the gain."""
    d, f, m = 1024, 2048, 2
    mats2, mats1 = [], []
    for (tr, sc, n, k) in [(synth.S_GATE_TRITS, synth.S_GATE_SCALES, f, d),
                           (synth.S_UP_TRITS, synth.S_UP_SCALES, f, d),
                           (synth.S_DOWN_TRITS, synth.S_DOWN_SCALES, d, f)]:
        t, s = synth.trits(4, tr, n, k), synth.scales(4, sc, n, k // 128)
        mats1.append(oracle.pack(t, s))
        mats2.append(oracle.pq2_pack(t, s))
    sg = synth.signs(4)
    x = synth.activations(4, m, d).astype(np.float64)
    gain = 0.5 + synth.gauss(4, 7, d).astype(np.float64) ** 2
    for eps, gv in ((0.0, None), (1e-6, gain)):
        a = oracle.pq2_ffn_block(x, *mats2, sg, d, f, eps, gain=gv)
        b = oracle.ffn_block(x, *mats1, sg, d, f, eps, gain=gv)
        assert np.linalg.norm(a - b) <= 1e-12 * np.linalg.norm(b)


# ----------------------------------------------------------------- W2A8 ----
# "Why I Am Building Another Inference Engine", Level 5 (8-bit activations
# times ternary weights) and Level 4 (quantised before the projections).

def test_w2a8_quant_worked_values():
    """max|x| = 1 -> c = 127: 0.5 -> 63.5 -> 64 and -0.5 -> -64 (ties to even),
    0.25 -> 31.75 -> 32, 1/256 -> 0.496 -> 0, the extreme -> -127."""
    q, step = oracle.w2a8_quant(np.array([0.5, -1.0, 0.25, 1.0 / 256, -0.5], np.float32))
    assert q.tolist() == [64, -127, 32, 0, -64]
    assert step == 1.0 / 127
    q, step = oracle.w2a8_quant(np.zeros(256, np.float32))
    assert not q.any() and step == 0.0


def test_w2a8_quant_range_and_grid_fixed_point():
    x = synth.activations(3, 1, 5120)[0]
    q, step = oracle.w2a8_quant(x)
    assert np.abs(q).max() == 127 and q[np.argmax(np.abs(x))] == np.sign(x[np.argmax(np.abs(x))]) * 127
    # quantising q itself (already on the grid, max 127) returns q with step 1
    q2, step2 = oracle.w2a8_quant(q.astype(np.float32))
    np.testing.assert_array_equal(q2, q)
    assert step2 == 1.0
    # the error of q * step is at most half a step per element
    assert np.abs(q * step - x.astype(np.float64)).max() <= 0.5 * step * (1 + 1e-6)


def test_w2a8_matvec_on_the_grid_equals_the_float_matvec():
    """Activations already on the 8-bit grid (integers, max 127): the W2A8
    product equals the C oracle's fp64 matvec of the same x."""
    n, k = 64, 1024
    rng = np.random.default_rng(4)
    t, s = synth.trits(4, synth.S_W_TRITS, n, k), synth.scales(4, synth.S_W_SCALES, n, k // 128)
    b = oracle.pack(t, s)
    x = rng.integers(-127, 128, size=k).astype(np.float64)
    x[7] = 127
    np.testing.assert_allclose(oracle.w2a8_matvec(b, n, k, x), oracle.matvec(b, n, k, x), rtol=1e-13, atol=0)


def test_w2a8_matvec_brute_force():
    """Two rows of one block, written out term by term."""
    rng = np.random.default_rng(6)
    t = rng.integers(-1, 2, size=(2, 128), dtype=np.int8)
    s = np.array([[0x3C00], [0xB800]], np.uint16)  # 1.0, -0.5
    x = rng.standard_normal(128).astype(np.float32)
    g = max(abs(float(v)) for v in x)
    c = float(np.float32(127.0 / g))
    q = [int(np.rint(np.float32(float(v)) * np.float32(c))) for v in x]
    ref = [sc * sum(int(t[r, i]) * q[i] for i in range(128)) * (g / 127.0) for r, sc in ((0, 1.0), (1, -0.5))]
    np.testing.assert_allclose(oracle.w2a8_matvec(oracle.pack(t, s), 2, 128, x), ref, rtol=1e-15, atol=0)


def test_w2a8_gemm_rows_on_the_grid_equal_the_float_gemm():
    """Rows already on the integer grid, each with max |x| = 127: the
    per-token W2A8 product equals the C oracle's fp64 GEMM."""
    n, k, m = 40, 640, 3
    rng = np.random.default_rng(8)
    b = oracle.pack(synth.trits(8, synth.S_W_TRITS, n, k), synth.scales(8, synth.S_W_SCALES, n, k // 128))
    x = rng.integers(-127, 128, size=(m, k)).astype(np.float64)
    x[:, 3] = 127
    np.testing.assert_allclose(oracle.w2a8_gemm(b, n, k, x), oracle.gemm(b, n, k, x), rtol=1e-13, atol=0)
