"""Host-only checks of the C ABI: the library loads, exports every function
include/ptq1.h declares, agrees with the oracle on the block geometry, and
refuses bad arguments before enqueuing anything (no GPU needed: every call
below fails validation, so no HIP call is made)."""
import ctypes as C

import pytest

import oracle
import ternary_weight_ptq1_amd as P

FAKE = 1 << 20  # a 16-byte-aligned fake device address, never dereferenced


def L():
    return P.lib()


def test_library_exports_every_header_function():
    names = P.header_functions()
    assert len(names) >= 17
    for n in names:
        assert hasattr(L(), n), f"{n} declared in ptq1.h but not exported"
    assert set(P._SIGS) == set(names)


def test_geometry_single_source():
    """One table, held together by a test ("A 27B model in 5.5 GB...",
    section "What I learned building it": derive copies from one table)."""
    g = P.ptq1_geometry()
    assert g == (128, 26, 28, 1024, 32, 2)
    assert g[:4] == (oracle.lib().orc_block_weights(), oracle.lib().orc_block_trit_bytes(),
                     oracle.lib().orc_block_bytes(), oracle.lib().orc_hadamard_width())
    assert (P.BLOCK_WEIGHTS, P.TRIT_BYTES, P.BLOCK_BYTES, P.HADAMARD, P.TILE_ROWS, P.TILE_BLOCKS) == g
    hdr = open(P.HEADER).read()
    for name, v in zip(("PTQ1_BLOCK_WEIGHTS", "PTQ1_TRIT_BYTES", "PTQ1_BLOCK_BYTES", "PTQ1_HADAMARD",
                        "PTQ1_TILE_ROWS", "PTQ1_TILE_BLOCKS"), g):
        assert f"#define {name} {v}" in hdr


def test_packed_bytes():
    assert P.ptq1_packed_bytes(17408, 5120) == 19_496_960
    assert P.ptq1_packed_bytes(5120, 17408) == 19_496_960
    assert P.ptq1_packed_bytes(1024, 1024) == 229_376
    assert P.ptq1_packed_bytes(0, 128) == 0
    assert P.ptq1_packed_bytes(1, 100) == -1
    assert P.ptq1_packed_bytes(-1, 128) == -1
    assert P.ptq1_packed_bytes(1 << 62, 1 << 20) == -1


def test_status_strings():
    for code, name in P.STATUS.items():
        assert L().ptq1_status_string(code).decode() == name


def test_tiled_bytes():
    # ceil(n/32)*32 rows x ceil(k/256)*2 blocks x 28 bytes
    assert P.ptq1_tiled_bytes(17408, 5120) == 19_496_960
    assert P.ptq1_tiled_bytes(5120, 17408) == 19_496_960
    assert P.ptq1_tiled_bytes(1, 128) == 32 * 2 * 28
    assert P.ptq1_tiled_bytes(33, 384) == 64 * 4 * 28
    assert P.ptq1_tiled_bytes(0, 128) == 0
    assert P.ptq1_tiled_bytes(1, 100) == -1
    assert P.ptq1_tiled_bytes(1 << 62, 1 << 20) == -1


def test_tile_validation():
    rc, msg = _err(L().ptq1_tile(None, 4, 128, C.c_void_p(FAKE), None))
    assert rc == 1 and "blocks" in msg
    rc, msg = _err(L().ptq1_tile(C.c_void_p(FAKE), 4, 130, C.c_void_p(FAKE * 2), None))
    assert rc == 2
    rc, msg = _err(L().ptq1_tile(C.c_void_p(FAKE), 4, 128, C.c_void_p(FAKE * 2 + 8), None))
    assert rc == 3 and "tiled" in msg
    rc, msg = _err(L().ptq1_tile(C.c_void_p(FAKE), 4, 128, C.c_void_p(FAKE + 64), None))
    assert rc == 7
    assert L().ptq1_tile(None, 0, 128, None, None) == 0


def test_profile_arm_validation():
    assert _err(L().ptq1_profile_arm(b"no_such_kernel", None, None, 0))[0] == 5
    assert _err(L().ptq1_profile_arm(None, None, None, 0))[0] == 1
    assert _err(L().ptq1_profile_arm(b"gemm", None, None, -1))[0] == 2
    assert _err(L().ptq1_profile_arm(b"gemm", None, None, 3))[0] == 1
    assert L().ptq1_profile_arm(b"lut_matvec_2", None, None, 0) == 0  # disarm is always fine
    assert L().ptq1_profile_count(b"lut_matvec_2") == 0
    assert L().ptq1_profile_count(b"nope") == -1


def _err(rc):
    return rc, L().ptq1_last_error().decode()


def test_pack_validation():
    rc, msg = _err(L().ptq1_pack(None, C.c_void_p(FAKE), 4, 128, C.c_void_p(FAKE * 2), None))
    assert rc == 1 and "trits" in msg
    rc, msg = _err(L().ptq1_pack(C.c_void_p(FAKE), C.c_void_p(FAKE), 4, 100, C.c_void_p(FAKE * 2), None))
    assert rc == 2 and "128" in msg
    rc, msg = _err(L().ptq1_pack(C.c_void_p(FAKE), C.c_void_p(FAKE), 4, 128, C.c_void_p(FAKE * 2 + 4), None))
    assert rc == 3 and "blocks" in msg
    rc, msg = _err(L().ptq1_pack(C.c_void_p(FAKE), C.c_void_p(FAKE), 1 << 60, 1 << 20, C.c_void_p(FAKE * 2), None))
    assert rc == 4
    # output overlapping the trits
    rc, msg = _err(L().ptq1_pack(C.c_void_p(FAKE), C.c_void_p(FAKE * 4), 4, 128, C.c_void_p(FAKE + 16), None))
    assert rc == 7
    # empty input is a no-op, not an error
    assert L().ptq1_pack(None, None, 0, 128, None, None) == 0


def test_rotate_validation():
    s = C.c_void_p(FAKE * 8)
    assert _err(L().hadamard_rotate(C.c_void_p(FAKE), C.c_void_p(FAKE * 2), 1, 1536, s, None))[0] == 2
    assert _err(L().hadamard_rotate(C.c_void_p(FAKE), C.c_void_p(FAKE * 2), 1, 1024, None, None))[0] == 1
    assert _err(L().hadamard_rotate(C.c_void_p(FAKE), C.c_void_p(FAKE + 4096), 2, 1024, s, None))[0] == 7
    assert _err(L().hadamard_rotate(C.c_void_p(FAKE + 8), C.c_void_p(FAKE * 2), 1, 1024, s, None))[0] == 3
    assert _err(L().hadamard_rotate(None, None, 0, 1024, None, None))[0] == 0


def test_unrotate_validation():
    s = C.c_void_p(FAKE * 8)
    rc, msg = _err(L().hadamard_unrotate_rows(C.c_void_p(FAKE), 10, 1024, None, 11, s, C.c_void_p(FAKE * 4), None))
    assert rc == 2 and "n_rows" in msg
    rc, _ = _err(L().hadamard_unrotate_rows(C.c_void_p(FAKE), 10, 1000, None, 1, s, C.c_void_p(FAKE * 4), None))
    assert rc == 2
    rc, _ = _err(L().hadamard_unrotate_rows(C.c_void_p(FAKE), 10, 1024, None, 2, s, C.c_void_p(FAKE + 4096), None))
    assert rc == 7


def test_matvec_validation():
    ws_need = L().ptq1_matvec_workspace_bytes(5120, 17408)
    assert ws_need >= 68 * 5120 * 4  # one partial per 256-wide K-slice and row
    B, X, Y, WS, S = (C.c_void_p(FAKE * i) for i in (1, 200, 300, 400, 500))
    rc, msg = _err(L().ptq1_matvec(B, 5120, 17408, X, S, None, Y, None, 0, None))
    assert rc == 6 and "ws" in msg
    rc, msg = _err(L().ptq1_matvec(B, 5120, 17408, X, S, None, Y, WS, ws_need - 1, None))
    assert rc == 6
    rc, msg = _err(L().ptq1_matvec(B, 5120, 17408 + 128, X, S, None, Y, WS, 1 << 30, None))
    assert rc == 2 and "1024" in msg
    rc, msg = _err(L().ptq1_matvec(B, 5120, 17408, X, S, None, C.c_void_p(FAKE * 200 + 64), WS, 1 << 30, None))
    assert rc == 7
    rc, msg = _err(L().ptq1_matvec(B, 5120, 17408, None, S, None, Y, WS, 1 << 30, None))
    assert rc == 1 and "x" in msg
    rc, msg = _err(L().ptq1_matvec(B, 5120, 17408, X, S, None, Y, C.c_void_p(FAKE * 400 + 16), 1 << 30, None))
    assert rc == 3


def test_gemm_and_ffn_validation():
    B, X, Y, WS, S = (C.c_void_p(FAKE * i) for i in (1, 200, 300, 400, 500))
    rc, msg = _err(L().ptq1_gemm(B, 17408, 5120, X, 65537, S, Y, WS, 1 << 40, None))
    assert rc == 5 and "m" in msg
    rc, _ = _err(L().ptq1_gemm(B, 17408, 5120, X, -1, S, Y, WS, 1 << 40, None))
    assert rc == 2
    need = L().ptq1_gemm_workspace_bytes(256, 17408, 5120)
    # bf16 activations, then two fp32 partial tiles (128 x 128) for each of
    # the 256 workgroups (one per CU) that share the tiles x K blocks
    assert need == 256 * 5120 * 2 + 256 * 2 * 128 * 128 * 4
    rc, _ = _err(L().ptq1_gemm(B, 17408, 5120, X, 256, S, Y, WS, need - 1, None))
    assert rc == 6
    W2, W3 = C.c_void_p(FAKE * 600), C.c_void_p(FAKE * 700)
    rc, msg = _err(L().ptq1_ffn_block(X, Y, 1, 5120, 17408, B, W2, W3, None, 0.0, None, WS, 1 << 40, None))
    assert rc == 1 and "signs" in msg
    rc, _ = _err(L().ptq1_ffn_block(X, Y, 1, 5000, 17408, B, W2, W3, S, 0.0, None, WS, 1 << 40, None))
    assert rc == 2
    rc, _ = _err(L().ptq1_ffn_block(X, C.c_void_p(FAKE * 200 + 16), 2, 5120, 17408, B, W2, W3, S, 0.0, None,
                                    WS, 1 << 40, None))
    assert rc == 7
    # the norm's gain: 16-byte aligned, disjoint from x_out and the workspace
    rc, msg = _err(L().ptq1_ffn_block(X, Y, 1, 5120, 17408, B, W2, W3, S, 1e-6, C.c_void_p(FAKE * 800 + 4), WS,
                                      1 << 40, None))
    assert rc == 3 and "rms_gain" in msg
    rc, msg = _err(L().ptq1_ffn_block(X, Y, 1, 5120, 17408, B, W2, W3, S, 1e-6, C.c_void_p(FAKE * 300 + 64), WS,
                                      1 << 40, None))
    assert rc == 7 and "rms_gain" in msg
    assert L().ptq1_ffn_workspace_bytes(1, 5120, 17408) > 0
    assert L().ptq1_ffn_workspace_bytes(8, 5120, 17408) >= 32 * 17408 * 2
    assert L().ptq1_ffn_workspace_bytes(1, 5120, 17400) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(P, "_lib", None)
    monkeypatch.setattr(P, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        P.lib()


def test_empty_calls_enqueue_nothing():
    """Zero rows or tokens: every entry point returns PTQ1_OK without touching
    the (fake) device pointers and without a workspace."""
    B, X, Y, WS, S = (C.c_void_p(FAKE * i) for i in (1, 200, 300, 400, 500))
    assert L().ptq1_gemm(B, 17408, 5120, X, 0, S, Y, WS, 0, None) == 0
    assert L().ptq1_matvec(B, 0, 5120, X, S, None, Y, WS, 0, None) == 0
    assert L().ptq1_gate_up(B, B, 0, 5120, X, S, Y, Y, WS, 0, None) == 0
    assert L().ptq1_ffn_block(X, Y, 0, 5120, 17408, B, B, B, S, 0.0, None, WS, 0, None) == 0
    assert L().hadamard_unrotate_rows(X, 100, 1024, None, 0, S, Y, None) == 0
    assert L().ptq1_swiglu(X, X, Y, 0, None) == 0
    assert L().ptq1_dequant(B, 0, 128, Y, None) == 0


def test_pq2_sizes():
    """PQ2_0 ("Why I Am Building Another Inference Engine", Level 2): 34-byte
    blocks, held against the oracle's block size; tiles of 32 rows x 2 blocks
    of 2176 bytes (64 records of 32 code bytes, then 64 scales)."""
    assert oracle.lib().orc_pq2_block_bytes() == P.PQ2_BLOCK_BYTES == 34
    assert P.pq2_packed_bytes(17408, 5120) == 17408 * 40 * 34
    assert P.pq2_packed_bytes(0, 128) == 0
    assert P.pq2_packed_bytes(1, 100) == -1
    assert P.pq2_packed_bytes(1 << 62, 1 << 20) == -1
    assert P.pq2_tiled_bytes(17408, 5120) == (17408 // 32) * 20 * 2176
    assert P.pq2_tiled_bytes(1, 128) == 2176
    assert P.pq2_tiled_bytes(33, 384) == 2 * 2 * 2176
    assert P.pq2_tiled_bytes(1, 100) == -1
    assert P.pq2_tiled_bytes(1 << 62, 1 << 20) == -1
    # bytes per weight at a whole tile: 2176 / (32 * 256) = 2.125 bits / 8
    assert P.pq2_tiled_bytes(32, 256) * 8 / (32 * 256) == 2.125


def test_pq2_validation():
    B, X, Y, WS, S = (C.c_void_p(FAKE * i) for i in (1, 200, 300, 400, 500))
    rc, msg = _err(L().pq2_pack(None, C.c_void_p(FAKE), 4, 128, C.c_void_p(FAKE * 2), None))
    assert rc == 1 and "trits" in msg
    rc, msg = _err(L().pq2_pack(C.c_void_p(FAKE), C.c_void_p(FAKE), 4, 100, C.c_void_p(FAKE * 2), None))
    assert rc == 2
    rc, msg = _err(L().pq2_pack(C.c_void_p(FAKE), C.c_void_p(FAKE * 4), 4, 128, C.c_void_p(FAKE + 16), None))
    assert rc == 7
    rc, msg = _err(L().pq2_tile(C.c_void_p(FAKE), 4, 128, C.c_void_p(FAKE * 2 + 8), None))
    assert rc == 3 and "tiled" in msg
    rc, msg = _err(L().pq2_tile(C.c_void_p(FAKE), 4, 128, C.c_void_p(FAKE + 64), None))
    assert rc == 7
    rc, msg = _err(L().pq2_dequant(B, 4, 128, C.c_void_p(FAKE + 64), None))
    assert rc == 7
    need = L().pq2_matvec_workspace_bytes(5120, 17408)
    assert need == L().ptq1_matvec_workspace_bytes(5120, 17408) or need >= 68 * 5120 * 4
    rc, msg = _err(L().pq2_matvec(B, 5120, 17408, X, S, None, Y, None, 0, None))
    assert rc == 6 and "ws" in msg
    rc, msg = _err(L().pq2_matvec(B, 5120, 17408 + 128, X, S, None, Y, WS, 1 << 30, None))
    assert rc == 2 and "1024" in msg
    rc, msg = _err(L().pq2_matvec(B, 5120, 17408, X, S, None, C.c_void_p(FAKE * 200 + 64), WS, 1 << 30, None))
    assert rc == 7
    rc, msg = _err(L().pq2_matvec(C.c_void_p(FAKE + 8), 5120, 17408, X, S, None, Y, WS, 1 << 30, None))
    assert rc == 3
    # 1 << 20 rows x 4096: the tiled matrix is above 2 GiB
    far = [C.c_void_p((1 << 40) * i) for i in (1, 2, 3, 4)]
    rc, msg = _err(L().pq2_matvec(B, 1 << 20, 1 << 13, far[0], far[1], None, far[2], far[3], 1 << 40, None))
    assert rc == 5 and "2 GiB" in msg
    assert L().pq2_matvec(B, 0, 5120, X, S, None, Y, WS, 0, None) == 0
    assert L().pq2_pack(None, None, 0, 128, None, None) == 0
    assert L().pq2_tile(None, 0, 128, None, None) == 0
    assert L().pq2_dequant(B, 0, 128, Y, None) == 0
    assert L().ptq1_profile_arm(b"pq2_matvec", None, None, 0) == 0
    # the PQ2_0 GEMM: same argument rules as ptq1_gemm
    gneed = L().pq2_gemm_workspace_bytes(256, 17408, 5120)
    assert gneed >= 256 * 5120 * 2  # bf16 activation fragments at least
    rc, msg = _err(L().pq2_gemm(B, 17408, 5120, X, 256, S, Y, WS, gneed - 1, None))
    assert rc == 6
    rc, msg = _err(L().pq2_gemm(B, 17408, 5120 + 128, X, 256, S, Y, WS, 1 << 40, None))
    assert rc == 2 and "1024" in msg
    rc, msg = _err(L().pq2_gemm(B, 17408, 5120, X, 65537, S, Y, WS, 1 << 40, None))
    assert rc == 5
    assert L().pq2_gemm(B, 17408, 5120, X, 0, S, Y, WS, 0, None) == 0
    # the PQ2_0 feed-forward block
    fneed = L().pq2_ffn_workspace_bytes(1, 5120, 17408)
    assert fneed >= 68 * 5120 * 4
    rc, msg = _err(L().pq2_ffn_block(X, Y, 1, 5120, 17408, B, B, B, S, 0.0, None, WS, fneed - 1, None))
    assert rc == 6
    rc, msg = _err(L().pq2_ffn_block(X, Y, 1, 5120, 17408, B, B, B, None, 0.0, None, WS, 1 << 40, None))
    assert rc == 1 and "signs" in msg
    assert L().pq2_ffn_block(X, Y, 0, 5120, 17408, B, B, B, S, 0.0, None, WS, 0, None) == 0



def test_w2a8_validation():
    B, X, Y, WS = (C.c_void_p(FAKE * i) for i in (1, 200, 300, 400))
    need = L().ptq1_matvec_w2a8_workspace_bytes(5120, 17408)
    # the activations are quantised inside the lookup kernel: the same split-K partials as the fp32 matvec
    assert need == L().ptq1_matvec_workspace_bytes(5120, 17408)
    rc, msg = _err(L().ptq1_matvec_w2a8(B, 5120, 17408, X, None, Y, WS, need - 1, None))
    assert rc == 6
    rc, msg = _err(L().ptq1_matvec_w2a8(B, 5120, 17408 + 64, X, None, Y, WS, 1 << 30, None))
    assert rc == 2
    rc, msg = _err(L().ptq1_matvec_w2a8(B, 5120, 17408, None, None, Y, WS, 1 << 30, None))
    assert rc == 1 and "x" in msg
    rc, msg = _err(L().ptq1_matvec_w2a8(B, 5120, 17408, X, None, C.c_void_p(FAKE * 200 + 64), WS, 1 << 30, None))
    assert rc == 7
    assert L().ptq1_matvec_w2a8(B, 0, 17408, X, None, Y, WS, 0, None) == 0
