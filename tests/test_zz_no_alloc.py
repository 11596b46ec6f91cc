"""ptq1_ffn_block_noalloc (the block on the library's static per-GPU scratch,
for callers that cannot allocate) against ptq1_ffn_block with a workspace:
the same kernels in the same order, so the outputs must agree bit for bit.
Two calls in a row, the second with a smaller input (the scratch keeps the
first call's contents and must not leak into the second), and a refusal,
before anything is enqueued, of a shape whose scratch exceeds the buffer."""
import numpy as np
import pytest
import torch

import synth
import synth.device as sdev
import ternary_weight_ptq1_amd as P

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _layer(seed, d, f):
    ls = synth.layer_stream
    out = []
    for tr, sc, n, k in ((synth.S_GATE_TRITS, synth.S_GATE_SCALES, f, d),
                         (synth.S_UP_TRITS, synth.S_UP_SCALES, f, d),
                         (synth.S_DOWN_TRITS, synth.S_DOWN_SCALES, d, f)):
        t = sdev.trits(seed, ls(tr, 0), n, k, device=DEV)
        s = sdev.scales(seed, ls(sc, 0), n, k // 128, device=DEV)
        out.append(P.ptq1_tile(P.ptq1_pack(t, s), n, k))
    return out


def test_noalloc_matches_workspace_call():
    # the 27B decode shape, then a smaller batch-8 block (bf16 MFMA path) with a gain
    for m, d, f, seed, gain in ((1, 5120, 17408, 4, False), (8, 1024, 2048, 5, True)):
        wg, wu, wd = _layer(seed, d, f)
        x = torch.from_numpy(synth.activations(seed, m, d)).to(DEV)
        s = torch.from_numpy(synth.signs(seed)).to(DEV)
        gv = torch.from_numpy((0.5 + synth.gauss(seed, 7, d) ** 2).astype(np.float32)).to(DEV) if gain else None
        ref = P.ptq1_ffn_block(x, wg, wu, wd, s, d, f, 1e-6, rms_gain=gv)
        got = P.ptq1_ffn_block_noalloc(x, wg, wu, wd, s, d, f, 1e-6, out=torch.empty_like(x), rms_gain=gv)
        torch.cuda.synchronize()
        r, g = ref.cpu().numpy(), got.cpu().numpy()
        assert np.isfinite(g).all(), f"m={m} d={d} f={f}"
        np.testing.assert_array_equal(g, r, err_msg=f"m={m} d={d} f={f}")


def test_noalloc_refuses_beyond_its_scratch():
    d, f, m = 5120, 17408, 16  # needs about 11 MiB of scratch, the buffer holds 8 MiB
    assert P.workspace_bytes("ffn", m, d, f) > 8 << 20
    w = torch.zeros(P.ptq1_tiled_bytes(f, d), dtype=torch.uint8, device=DEV)
    wd = torch.zeros(P.ptq1_tiled_bytes(d, f), dtype=torch.uint8, device=DEV)
    x = torch.zeros((m, d), dtype=torch.float32, device=DEV)
    out = torch.full_like(x, 7.0)
    s = torch.ones(1024, dtype=torch.float32, device=DEV)
    with pytest.raises(P.Ptq1Error) as ei:
        P.ptq1_ffn_block_noalloc(x, w, w, wd, s, d, f, 1e-6, out=out)
    assert ei.value.status == 5 and "scratch" in ei.value.message
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())  # nothing was enqueued
