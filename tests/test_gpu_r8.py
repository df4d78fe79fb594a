"""GPU parity of the row-interleaved (R8) layout: q8_0_repack_r8 writes the
oracle's bytes exactly (padding included), and q8_0_matvec_r8 matches the
oracle's R8 matvec within 1e-5 per-row relative L2, exactly where every block
scale is 1 (integer outputs), and bitwise from run to run."""
import numpy as np
import pytest

import synth

from gpu_cases import acts_q8, assert_rows_close, nan_like, to_gpu, weights_q8

pytestmark = pytest.mark.gpu

SHAPES = [(1, 32), (9, 64), (13, 96), (777, 768), (1000, 768), (1031, 2048), (200, 3072),
          (64, 4096), (37, 8192), (40, 16384), (5, 32768)]


@pytest.fixture(scope="module")
def q():
    import moe_expert_ffn_q8_amd as q
    return q


@pytest.mark.parametrize("n,k", SHAPES)
def test_r8_repack_bytes(q, orc, n, k):
    import torch
    w = weights_q8(orc, n, k, "r8", n, k)
    out = torch.full((q.q8_0_r8_bytes(n, k),), 0xAB, dtype=torch.uint8, device="cuda")
    q.q8_0_repack_r8(to_gpu(w), n, k, out=out)
    assert np.array_equal(out.cpu().numpy(), orc.repack_r8(w, n, k))


@pytest.mark.parametrize("n,k", SHAPES)
def test_r8_matvec(q, orc, n, k):
    w = weights_q8(orc, n, k, "r8", n, k)
    x = acts_q8(orc, 1, k, "r8-x", n, k)
    wr = q.q8_0_repack_r8(to_gpu(w), n, k)
    xg = to_gpu(x)
    y = nan_like((n,))
    q.q8_0_matvec_r8(wr, xg, n, k, y=y)
    ref = orc.matvec_r8(orc.repack_r8(w, n, k), x, n, k)
    assert_rows_close(y.cpu().numpy()[None, :], ref[None, :])
    y2 = q.q8_0_matvec_r8(wr, xg, n, k)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y2.cpu().numpy().view(np.uint32))
    # the native layout's product agrees within the same tolerance
    yn = q.q8_0_matvec(to_gpu(w), xg, n, k)
    assert_rows_close(yn.cpu().numpy()[None, :], ref[None, :])


@pytest.mark.parametrize("n,k", [(17, 2048), (300, 768), (8, 96)])
def test_r8_matvec_unit_scales_exact(q, orc, n, k):
    """Every scale 1.0: each block term is the integer block sum, and every
    partial sum stays an integer below 2^24, so the fp32 output is exact in any
    order and must equal the oracle bit for bit."""
    g = np.random.default_rng(n + k)
    nb = k // 32

    def unit_blocks(rows):
        b = np.zeros((rows, nb, 34), dtype=np.uint8)
        b[:, :, 0], b[:, :, 1] = 0x00, 0x3C
        b[:, :, 2:] = g.integers(-40, 41, size=(rows, nb, 32)).astype(np.int8).view(np.uint8)
        return b.reshape(rows, nb * 34)

    w, x = unit_blocks(n), unit_blocks(1)
    y = nan_like((n,))
    q.q8_0_matvec_r8(q.q8_0_repack_r8(to_gpu(w), n, k), to_gpu(x), n, k, y=y)
    ref = orc.matvec_r8(orc.repack_r8(w, n, k), x, n, k)
    assert np.all(np.abs(ref) < 2 ** 24)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)


def test_r8_full_size_vocab(q, orc):
    """262144 x 2048 at full size: weights drawn on the GPU, quantized and
    repacked by the library; sampled groups are re-quantized and repacked by
    the oracle from the same fp32 values (bytes must match), and the outputs
    of their rows computed by the oracle."""
    import torch
    n, k = 262144, 2048
    nb = k // 32
    gbytes = 8 * nb * 34
    wf = synth.normal_f32_torch((n, k), 0.02, "cuda", 0, "c5b", "w")
    wq = q.q8_0_quantize_rows(wf)
    wr = q.q8_0_repack_r8(wq, n, k)
    del wq
    xq = orc.quantize_rows(synth.normal_f32((1, k), 1.0, 0, "c5b", "x"))
    y = nan_like((n,))
    q.q8_0_matvec_r8(wr, to_gpu(xq), n, k, y=y)
    groups = np.unique(np.concatenate([np.arange(4), n // 8 - 1 - np.arange(4),
                                       np.random.default_rng(1).integers(0, n // 8, 512)]))
    rows = (groups[:, None] * 8 + np.arange(8)[None, :]).ravel()
    w_rows = orc.quantize_rows(wf[torch.from_numpy(rows).cuda()].cpu().numpy())
    del wf
    wr_h = wr.view(n // 8, gbytes)[torch.from_numpy(groups).cuda()].cpu().numpy()
    assert np.array_equal(wr_h.ravel(), orc.repack_r8(w_rows, rows.size, k))
    ref = orc.matvec_r8(wr_h.ravel(), xq, rows.size, k)
    yy = y.cpu().numpy()
    assert np.all(np.isfinite(yy))
    assert_rows_close(yy[rows][None, :], ref[None, :])


def test_r8_limits(q):
    import torch
    w = torch.zeros(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(q.Q8Error):
        q.q8_0_matvec_r8(w, w, 1, 32768 + 32)
