"""Host-only checks that the Python binding refuses tensors the C call
would read or write out of range, before anything is enqueued.  The
device check is relaxed to accept host tensors here (there is no GPU), so
each case reaches the size checks; every case must raise ValueError before
a compute entry point is called."""
import pytest
import torch

import ternary_weight_ptq1_amd as P

D, F = 1024, 2048


@pytest.fixture
def host_ok(monkeypatch):
    real = P.lib()
    calls = []

    class Guard:
        """Stands in for the library: host-only size queries pass through,
        any compute entry point fails the test."""
        def __getattr__(self, name):
            fn = getattr(real, name)
            if name.endswith(("_bytes", "_string", "_error")) or name == "ptq1_geometry":
                return fn

            def refuse(*a):
                calls.append(name)
                raise AssertionError(f"{name} reached with invalid arguments")
            return refuse

    guard = Guard()
    monkeypatch.setattr(P, "_on_device", lambda t: True)
    monkeypatch.setattr(P, "lib", lambda: guard)
    yield calls


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def u8(n):
    return torch.zeros(n, dtype=torch.uint8)


def test_host_tensor_refused():
    with pytest.raises(ValueError, match="device tensor"):
        P.ptq1_matvec(u8(P.ptq1_tiled_bytes(D, D)), D, D, f32(D), None)


def test_matvec_sizes(host_ok):
    w = u8(P.ptq1_tiled_bytes(D, D))
    with pytest.raises(ValueError, match="blocks"):
        P.ptq1_matvec(u8(100), D, D, f32(D), None)
    with pytest.raises(ValueError, match="x has"):
        P.ptq1_matvec(w, D, D, f32(D - 1), None)
    with pytest.raises(ValueError, match="signs1024"):
        P.ptq1_matvec(w, D, D, f32(D), f32(512))
    with pytest.raises(ValueError, match="residual"):
        P.ptq1_matvec(w, D, D, f32(D), None, residual=f32(D - 4))
    with pytest.raises(ValueError, match="y has"):
        P.ptq1_matvec(w, D, D, f32(D), None, out=f32(D // 2))
    with pytest.raises(ValueError, match="ws has"):
        P.ptq1_matvec(w, D, D, f32(D), None, ws=u8(16))
    with pytest.raises(ValueError, match="ws must be"):
        P.ptq1_matvec(w, D, D, f32(D), None, ws=f32(1 << 20))
    with pytest.raises(ValueError, match="blocks"):
        P.ptq1_matvec_float_peel(u8(P.ptq1_tiled_bytes(D, D) - 1), D, D, f32(D), None)
    assert host_ok == []


def test_gate_up_and_swiglu_sizes(host_ok):
    tb = P.ptq1_tiled_bytes(F, D)
    with pytest.raises(ValueError, match="w_up"):
        P.ptq1_gate_up(u8(tb), u8(tb - 28), F, D, f32(D), None)
    with pytest.raises(ValueError, match="g has"):
        P.ptq1_gate_up(u8(tb), u8(tb), F, D, f32(D), None, g=f32(F - 1))
    with pytest.raises(ValueError, match="u has"):
        P.ptq1_swiglu(f32(F), f32(F - 1))
    assert host_ok == []


def test_gemm_sizes(host_ok):
    w = u8(P.ptq1_tiled_bytes(F, D))
    with pytest.raises(ValueError, match="not a multiple of k"):
        P.ptq1_gemm(w, F, D, f32(3 * D + 5), None)  # a remainder is no longer dropped
    with pytest.raises(ValueError, match="y has"):
        P.ptq1_gemm(w, F, D, f32(4, D), None, out=f32(4, F - 1))
    with pytest.raises(ValueError, match="blocks"):
        P.ptq1_gemm(u8(1000), F, D, f32(4, D), None)
    with pytest.raises(ValueError, match="not a multiple of k"):
        P.ptq1_gemm_w2a8(w, F, D, f32(D + 1))
    assert host_ok == []


def test_ffn_block_sizes(host_ok):
    wg = u8(P.ptq1_tiled_bytes(F, D))
    wd = u8(P.ptq1_tiled_bytes(D, F))
    s = f32(1024)
    with pytest.raises(ValueError, match="w_down"):
        P.ptq1_ffn_block(f32(2, D), wg, wg, wg[:100], s, D, F)
    with pytest.raises(ValueError, match="signs1024"):
        P.ptq1_ffn_block(f32(2, D), wg, wg, wd, f32(1000), D, F)
    with pytest.raises(ValueError, match="signs1024 is required"):
        P.ptq1_ffn_block(f32(2, D), wg, wg, wd, None, D, F)
    with pytest.raises(ValueError, match="rms_gain"):
        P.ptq1_ffn_block(f32(2, D), wg, wg, wd, s, D, F, rms_gain=f32(D - 1))
    with pytest.raises(ValueError, match="x_out"):
        P.ptq1_ffn_block(f32(2, D), wg, wg, wd, s, D, F, out=f32(1, D))
    with pytest.raises(ValueError, match="not a multiple of k"):
        P.ptq1_ffn_block(f32(D + 7), wg, wg, wd, s, D, F)
    with pytest.raises(ValueError, match="w_gate"):
        P.pq2_ffn_block(f32(1, D), wg, wg, wd, s, D, F)  # PTQ1_0-sized matrices are short for PQ2_0
    assert host_ok == []


def test_codec_and_rotation_sizes(host_ok):
    t = torch.zeros((4, 256), dtype=torch.int8)
    with pytest.raises(ValueError, match="scales_f16"):
        P.ptq1_pack(t, torch.zeros(7, dtype=torch.int16))
    with pytest.raises(ValueError, match="blocks has"):
        P.ptq1_pack(t, torch.zeros(8, dtype=torch.int16), out=u8(10))
    with pytest.raises(ValueError, match="blocks"):
        P.ptq1_tile(u8(10), 4, 256)
    with pytest.raises(ValueError, match="w has"):
        P.ptq1_dequant(u8(P.ptq1_packed_bytes(4, 256)), 4, 256, out=f32(4, 255))
    with pytest.raises(ValueError, match="signs1024"):
        P.hadamard_rotate(f32(2, 1024), f32(1023))
    with pytest.raises(ValueError, match="y has"):
        P.hadamard_rotate(f32(2, 1024), f32(1024), out=f32(1024))
    with pytest.raises(ValueError, match="out has"):
        P.hadamard_unrotate_rows(f32(8, 1024), f32(1024), n_rows=4, out=f32(3, 1024))
    with pytest.raises(ValueError, match="ids must be"):
        P.hadamard_unrotate_rows(f32(8, 1024), f32(1024), ids=torch.zeros(3, dtype=torch.int64))
    with pytest.raises(ValueError, match="tiled"):
        P.pq2_matvec(u8(5), D, D, f32(D), None)
    with pytest.raises(ValueError, match="residual"):
        P.ptq1_matvec_w2a8(u8(P.ptq1_tiled_bytes(D, D)), D, D, f32(D), residual=f32(3))
    assert host_ok == []
