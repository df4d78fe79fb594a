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
    """k above 32768 is refused by the library (its LDS staging limit); the
    call goes through the C ABI directly, since the binding would already
    refuse the undersized tensors."""
    import torch
    w = torch.zeros(64, dtype=torch.uint8, device="cuda")
    p = w.data_ptr()
    assert q.raw.q8_0_matvec_r8(p, p, p, 1, 32768 + 32, None) == -4


def test_r8_batched_step(q, orc):
    """Several descriptors in one launch, stacks of matrices with gaps between
    output vectors (the gaps must stay untouched), a ragged row count, and both
    activation staging paths (k <= 2048 and k = 8192)."""
    import torch
    cases = [(777, 768, 3), (64, 2048, 2), (13, 96, 1), (5, 8192, 2), (2048, 768, 2)]
    descs, refs, keep = [], [], []
    for ci, (n, k, batch) in enumerate(cases):
        nb = k // 32
        mb = q.q8_0_r8_bytes(n, k)
        ws = [weights_q8(orc, n, k, "r8b", ci, b) for b in range(batch)]
        xs = acts_q8(orc, batch, k, "r8b-x", ci)
        wr = torch.cat([q.q8_0_repack_r8(to_gpu(w), n, k) for w in ws])
        xg = to_gpu(xs.reshape(-1))
        ys = n + 7                                   # a gap after every output vector
        y = nan_like((batch * ys,))
        descs.append(q.make_r8_desc(wr, xg, y, n, k, batch=batch, w_batch_stride=mb,
                                    x_batch_stride=nb, y_batch_stride=ys))
        refs.append([orc.matvec_r8(orc.repack_r8(ws[b], n, k), xs[b], n, k)
                     for b in range(batch)])
        keep.append((wr, xg, y, n, ys))
    q.q8_0_matvec_r8_batched(descs, keep[0][0])
    for (wr, xg, y, n, ys), ref in zip(keep, refs):
        yy = y.cpu().numpy().reshape(-1, ys)
        assert np.all(np.isnan(yy[:, n:])), "a gap between output vectors was written"
        assert_rows_close(yy[:, :n], np.stack(ref))


def test_r8_f32_batched_quantizes_inside(q, orc):
    """fp32 activation rows quantized inside the launch: bitwise equal to
    q8_0_quantize_rows followed by q8_0_matvec_r8_batched, and within the
    tolerance of the oracle on the oracle's quantization of the same rows;
    one and two quantization passes held in registers (k <= 2048) and the
    looped form (k = 4096, 8192), ragged block counts."""
    import torch
    cases = [(777, 768, 3), (64, 2048, 2), (13, 96, 1), (40, 4096, 2), (5, 8192, 1),
             (100, 1056, 1)]
    d8, d32, refs, keep = [], [], [], []
    for ci, (n, k, batch) in enumerate(cases):
        nb = k // 32
        mb = q.q8_0_r8_bytes(n, k)
        ws = [weights_q8(orc, n, k, "r8f", ci, b) for b in range(batch)]
        xf = synth.normal_f32((batch, k), 1.0, "r8f-x", ci)
        wr = torch.cat([q.q8_0_repack_r8(to_gpu(w), n, k) for w in ws])
        xg = to_gpu(xf.reshape(-1))
        xq = q.q8_0_quantize_rows(xg.view(batch, k))
        y8 = nan_like((batch * n,))
        y32 = nan_like((batch * n,))
        d8.append(q.make_r8_desc(wr, xq, y8, n, k, batch=batch, w_batch_stride=mb,
                                 x_batch_stride=nb, y_batch_stride=n))
        d32.append(q.make_r8_f32_desc(wr, xg, y32, n, k, batch=batch, w_batch_stride=mb,
                                      x_batch_stride=k, y_batch_stride=n))
        xo = orc.quantize_rows(xf)
        assert np.array_equal(xq.cpu().numpy(), xo)
        refs.append(np.stack([orc.matvec_r8(orc.repack_r8(ws[b], n, k), xo[b], n, k)
                              for b in range(batch)]))
        keep.append((wr, xg, xq, y8, y32, n, batch))
    q.q8_0_matvec_r8_batched(d8, keep[0][0])
    q.q8_0_matvec_r8_f32_batched(d32, keep[0][0])
    for (wr, xg, xq, y8, y32, n, batch), ref in zip(keep, refs):
        a = y8.cpu().numpy()
        b = y32.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        assert_rows_close(b.reshape(batch, n), ref)


MM_CASES = [(777, 768, 8, 1), (2304, 768, 8, 2), (40, 3072, 8, 1), (100, 96, 5, 1),
            (33, 32, 3, 2), (300, 2048, 16, 1), (129, 768, 9, 2), (64, 4096, 2, 1),
            (50257 // 8 * 8 + 3, 768, 8, 1), (17, 8192, 16, 1), (8, 768, 1, 1)]


@pytest.mark.parametrize("n,k,m,batch", MM_CASES)
def test_r8_matmul_small_batch(q, orc, n, k, m, batch):
    """1..16 token rows over R8 weights on the matrix cores: within 1e-5 of
    the oracle per token row, bitwise repeatable; batch entries with strided
    activation and output rows and gaps that must stay untouched."""
    import torch
    nb = k // 32
    mb = q.q8_0_r8_bytes(n, k)
    ws = [weights_q8(orc, n, k, "r8mm", n, k, m, b) for b in range(batch)]
    xs = [acts_q8(orc, m, k, "r8mm-x", n, k, m, b) for b in range(batch)]
    wr = torch.cat([q.q8_0_repack_r8(to_gpu(w), n, k) for w in ws])
    xrs = nb + 3                                 # activation row stride (blocks)
    xbuf = np.zeros((batch, m, xrs * 34), dtype=np.uint8)
    for b in range(batch):
        xbuf[b, :, :nb * 34] = xs[b]
    xg = to_gpu(xbuf.reshape(-1))
    yrs, ybs = n + 5, m * (n + 5) + 11
    y = nan_like((batch * ybs,))
    d = [q.make_r8_mm_desc(wr, xg, y, n, k, m=m, batch=batch, w_batch_stride=mb,
                           x_row_stride=xrs, x_batch_stride=m * xrs, y_row_stride=yrs,
                           y_batch_stride=ybs)]
    q.q8_0_matmul_r8_batched(d, wr)
    yy = y.cpu().numpy()
    for b in range(batch):
        got = yy[b * ybs:b * ybs + m * yrs].reshape(m, yrs)
        assert np.all(np.isnan(got[:, n:])), "a gap was written"
        assert_rows_close(got[:, :n], orc.matmul(ws[b], xs[b], n, k, m))
    assert np.all(np.isnan(yy.reshape(batch, ybs)[:, m * yrs:]))
    y2 = nan_like((batch * ybs,))
    d2 = [q.make_r8_mm_desc(wr, xg, y2, n, k, m=m, batch=batch, w_batch_stride=mb,
                            x_row_stride=xrs, x_batch_stride=m * xrs, y_row_stride=yrs,
                            y_batch_stride=ybs)]
    q.q8_0_matmul_r8_batched(d2, wr)
    a, c = yy, y2.cpu().numpy()
    fin = ~np.isnan(a)
    assert np.array_equal(a[fin].view(np.uint32), c[fin].view(np.uint32))


def test_r8_matmul_unit_scales_exact(q, orc):
    """Every scale 1: the fp32 outputs are integers below 2^24, exact."""
    g = np.random.default_rng(5)
    n, k, m = 96, 2048, 8
    nb = k // 32

    def unit_blocks(rows):
        b = np.zeros((rows, nb, 34), dtype=np.uint8)
        b[:, :, 0], b[:, :, 1] = 0x00, 0x3C
        b[:, :, 2:] = g.integers(-40, 41, size=(rows, nb, 32)).astype(np.int8).view(np.uint8)
        return b.reshape(rows, nb * 34)

    w, x = unit_blocks(n), unit_blocks(m)
    y = nan_like((m, n))
    q.q8_0_matmul_r8_batched([q.make_r8_mm_desc(q.q8_0_repack_r8(to_gpu(w), n, k), to_gpu(x), y,
                                                n, k, m=m)], y)
    ref = orc.matmul(w, x, n, k, m)
    assert np.all(np.abs(ref) < 2 ** 24)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)
