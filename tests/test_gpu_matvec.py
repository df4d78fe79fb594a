"""GPU parity of q8_0_matvec / q8_0_matmul (streaming engine) against the
oracle: exact int32 block sums, fp32 outputs within 1e-5 per-row relative L2,
every output written (outputs are pre-filled with NaN), bitwise determinism."""
import numpy as np
import pytest

import synth

from gpu_cases import acts_q8, assert_rows_close, nan_like, to_gpu, weights_q8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import moe_expert_ffn_q8_amd as q
    return q


def test_c1_matvec_768(q, orc):
    """The 768 x 768 matvec, seed 0 (weights N(0,0.02), activation N(0,1))."""
    n = k = 768
    w = weights_q8(orc, n, k, 0, "c1", "w")
    x = acts_q8(orc, 1, k, 0, "c1", "x")
    ref = orc.matmul(w, x, n, k, 1)
    y = nan_like((n,))
    q.q8_0_matvec(to_gpu(w), to_gpu(x), n, k, y=y)
    assert_rows_close(y.cpu().numpy()[None, :], ref)
    _, sums = q.q8_0_matmul_blocksums(to_gpu(w), to_gpu(x), n, k, 1)
    assert np.array_equal(sums.cpu().numpy(), orc.matmul_blocksums(w, x, n, k, 1))


@pytest.mark.parametrize("n,k", [(1000, 256), (777, 768), (1031, 2048), (200, 3072),
                                 (130, 4096), (37, 8192), (513, 1024)])
def test_matvec_shapes(q, orc, n, k):
    w = weights_q8(orc, n, k, "mv", n, k)
    x = acts_q8(orc, 1, k, "mv-x", n, k)
    ref = orc.matmul(w, x, n, k, 1)
    y = nan_like((n,))
    wg, xg = to_gpu(w), to_gpu(x)
    q.q8_0_matvec(wg, xg, n, k, y=y)
    assert_rows_close(y.cpu().numpy()[None, :], ref)
    y2 = q.q8_0_matvec(wg, xg, n, k)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y2.cpu().numpy().view(np.uint32))
    _, sums = q.q8_0_matmul_blocksums(wg, xg, n, k, 1)
    assert np.array_equal(sums.cpu().numpy(), orc.matmul_blocksums(w, x, n, k, 1))


@pytest.mark.parametrize("n,k", [(65, 96), (40, 16384), (3, 32)])
def test_matvec_generic_path(q, orc, n, k):
    """k/32 not a multiple of 8, or k above the fast path's limit."""
    w = weights_q8(orc, n, k, "gen", n, k)
    x = acts_q8(orc, 1, k, "gen-x", n, k)
    y = nan_like((n,))
    q.q8_0_matvec(to_gpu(w), to_gpu(x), n, k, y=y)
    assert_rows_close(y.cpu().numpy()[None, :], orc.matmul(w, x, n, k, 1))
    _, sums = q.q8_0_matmul_blocksums(to_gpu(w), to_gpu(x), n, k, 1)
    assert np.array_equal(sums.cpu().numpy(), orc.matmul_blocksums(w, x, n, k, 1))


def test_matvec_misaligned_weights(q, orc):
    """A weight matrix starting 2 bytes past a 16-byte boundary (generic path)."""
    import torch
    n, k = 50, 512
    w = weights_q8(orc, n, k, "mis")
    x = acts_q8(orc, 1, k, "mis-x")
    buf = torch.zeros(w.size + 16, dtype=torch.uint8, device="cuda")
    buf[2:2 + w.size] = to_gpu(w.reshape(-1))
    y = nan_like((n,))
    rc = q.raw.q8_0_matvec(buf.data_ptr() + 2, to_gpu(x).data_ptr(), y.data_ptr(), n, k,
                           torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    assert_rows_close(y.cpu().numpy()[None, :], orc.matmul(w, x, n, k, 1))


@pytest.mark.parametrize("n,k,m", [(300, 768, 2), (129, 2048, 3), (1000, 768, 8),
                                   (257, 3072, 8), (100, 4096, 16), (90, 512, 5),
                                   (70, 768, 17), (33, 1024, 40)])
def test_matmul_small_m(q, orc, n, k, m):
    w = weights_q8(orc, n, k, "mm", n, k, m)
    x = acts_q8(orc, m, k, "mm-x", n, k, m)
    ref = orc.matmul(w, x, n, k, m)
    y = nan_like((m, n))
    q.q8_0_matmul(to_gpu(w), to_gpu(x), n, k, m, y=y)
    assert_rows_close(y.cpu().numpy(), ref)
    if m <= 16:
        _, sums = q.q8_0_matmul_blocksums(to_gpu(w), to_gpu(x), n, k, m)
        assert np.array_equal(sums.cpu().numpy(), orc.matmul_blocksums(w, x, n, k, m))


@pytest.mark.parametrize("m", [3, 8, 13])
def test_matmul_small_m_unaligned_activations(q, orc, m):
    """Activation rows that start 2 bytes past a dword boundary (an odd block
    offset and an odd row stride in blocks): the engine takes them with
    halfword loads."""
    import torch
    n, k = 100, 768
    nb = k // 32
    w = weights_q8(orc, n, k, "mu", m)
    xs = acts_q8(orc, m, k, "mu-x", m)
    stride = nb + 1
    xbuf = np.zeros((m * stride + 1, 34), dtype=np.uint8)
    for r in range(m):
        xbuf[1 + r * stride: 1 + r * stride + nb] = xs[r].reshape(nb, 34)
    wg, xg = to_gpu(w), to_gpu(xbuf)
    y = nan_like((m, n))
    d = q.make_desc(wg, (xg, 1), y, n, k, m=m, x_row_stride=stride)
    q.q8_0_matmul_batched([d], wg)
    torch.cuda.synchronize()
    assert_rows_close(y.cpu().numpy(), orc.matmul(w, xs, n, k, m))


def test_batched_descriptors(q, orc):
    """Several products in one launch: two weight stacks with a batch
    dimension, a strided activation layout, and a single matrix."""
    import torch
    specs = [  # (n, k, m, batch)
        (96, 768, 1, 5), (160, 256, 1, 3), (50, 2048, 1, 1), (70, 768, 4, 2)]
    descs, checks, keep = [], [], []
    for i, (n, k, m, batch) in enumerate(specs):
        nb = k // 32
        w = weights_q8(orc, batch * n, k, "bd-w", i)
        # activations: rows of all batch entries in one [batch*m][k] block, with a
        # larger row stride (2 extra blocks) to exercise strides
        xs = acts_q8(orc, batch * m, k, "bd-x", i)
        stride = nb + 2
        xbuf = np.zeros((batch * m, stride * 34), dtype=np.uint8)
        xbuf[:, : nb * 34] = xs
        wg, xg = to_gpu(w), to_gpu(xbuf)
        y = nan_like((batch, m, n + 3))
        keep += [wg, xg, y]
        descs.append(q.make_desc(wg, xg, y, n, k, m=m, batch=batch, w_batch_stride=n * nb,
                                 x_row_stride=stride, x_batch_stride=m * stride,
                                 y_row_stride=n + 3, y_batch_stride=m * (n + 3)))
        checks.append((w, xs, y, n, k, m, batch))
    q.q8_0_matmul_batched(descs, keep[0])
    torch.cuda.synchronize()
    for w, xs, y, n, k, m, batch in checks:
        nb34 = k // 32 * 34
        yy = y.cpu().numpy()
        for b in range(batch):
            ref = orc.matmul(w[b * n:(b + 1) * n], xs[b * m:(b + 1) * m], n, k, m)
            assert_rows_close(yy[b, :, :n], ref)
            assert np.all(np.isnan(yy[b, :, n:]))      # padding columns untouched


def test_c5b_vocab_projection_full_size(q, orc):
    """262144 x 2048 at full size: weights drawn on the GPU (torch's generator),
    quantized by the library; sampled rows are re-quantized by the oracle from
    the same fp32 values (bytes must match) and their outputs computed by the
    oracle."""
    import torch
    import synth
    n, k = 262144, 2048
    wf = synth.normal_f32_torch((n, k), 0.02, "cuda", 0, "c5b", "w")
    wq = q.q8_0_quantize_rows(wf)
    xf = synth.normal_f32((1, k), 1.0, 0, "c5b", "x")
    xq = orc.quantize_rows(xf)
    y = nan_like((n,))
    q.q8_0_matvec(wq, to_gpu(xq), n, k, y=y)
    rows = np.unique(np.concatenate([np.arange(8), n - 1 - np.arange(8),
                                     np.random.default_rng(0).integers(0, n, 4096)]))
    rows_t = torch.from_numpy(rows).cuda()
    w_rows = orc.quantize_rows(wf[rows_t].cpu().numpy())
    assert np.array_equal(wq[rows_t].cpu().numpy(), w_rows)
    ref = orc.matmul(w_rows, xq, rows.size, k, 1)
    yy = y.cpu().numpy()
    assert np.all(np.isfinite(yy))
    assert_rows_close(yy[rows][None, :], ref)
    del wf


def test_matvec_paired_tiles_odd_and_straddling(q, orc):
    """Launches of 8192 tiles or more take two tiles per workgroup: an odd tile
    count (8193 one-row tiles at k = 8192: the last workgroup has a single
    tile) and a pair that straddles two descriptors (8191 tiles of one product
    and 1 tile of another in one batched call), against the oracle on sampled
    and boundary rows."""
    import torch
    k = 8192
    nb = k // 32
    x = acts_q8(orc, 1, k, "pair-x")
    xg = to_gpu(x)
    rng = np.random.default_rng(5)
    # odd count: 8193 rows -> 8193 tiles
    n = 8193
    w = weights_q8(orc, n, k, "pair-w", n)
    wg = to_gpu(w)
    y = nan_like((n,))
    q.q8_0_matvec(wg, xg, n, k, y=y)
    rows = np.unique(np.concatenate([[0, 1, n - 3, n - 2, n - 1], rng.integers(0, n, 200)]))
    ref = orc.matmul(np.ascontiguousarray(w.reshape(n, nb * 34)[rows]), x, rows.size, k, 1)
    yy = y.cpu().numpy()
    assert np.all(np.isfinite(yy))
    assert_rows_close(yy[rows][None, :], ref)
    # a pair across two descriptors: tiles 8190 (last of the first) and 8191
    n1, n2, k2 = 8191, 5, 768
    w2 = weights_q8(orc, n2, k2, "pair-w2")
    x2 = acts_q8(orc, 1, k2, "pair-x2")
    y1, y2 = nan_like((n1,)), nan_like((n2,))
    d = [q.make_desc(wg, xg, y1, n1, k), q.make_desc(to_gpu(w2), to_gpu(x2), y2, n2, k2)]
    q.q8_0_matmul_batched(d, wg)
    torch.cuda.synchronize()
    rows1 = np.unique(np.concatenate([[0, n1 - 2, n1 - 1], rng.integers(0, n1, 100)]))
    ref1 = orc.matmul(np.ascontiguousarray(w.reshape(n, nb * 34)[rows1]), x, rows1.size, k, 1)
    assert_rows_close(y1.cpu().numpy()[rows1][None, :], ref1)
    assert_rows_close(y2.cpu().numpy()[None, :], orc.matmul(w2, x2, n2, k2, 1))


@pytest.mark.parametrize("m,n,k", [(17, 70, 768), (128, 128, 256), (129, 257, 512),
                                   (200, 300, 2048), (512, 96, 4096), (33, 1000, 768),
                                   (256, 40, 3072)])
def test_prefill_gemm_shapes(q, orc, m, n, k):
    """The matrix-core path (m > 16): ragged m and n on both sides of the
    128 x 128 tile, every K step size the library uses."""
    w = weights_q8(orc, n, k, "gemm", m, n, k)
    x = acts_q8(orc, m, k, "gemm-x", m, n, k)
    ref = orc.matmul(w, x, n, k, m)
    y = nan_like((m, n))
    q.q8_0_matmul(to_gpu(w), to_gpu(x), n, k, m, y=y)
    yy = y.cpu().numpy()
    assert_rows_close(yy, ref)
    y2 = q.q8_0_matmul(to_gpu(w), to_gpu(x), n, k, m)
    assert np.array_equal(yy.view(np.uint32), y2.cpu().numpy().view(np.uint32))


def test_c5a_prefill_full_size(q, orc):
    """512 tokens x K=4096 against 14336 x 4096 weights: the full prefill
    product; the oracle checks 96 sampled weight rows for all 512 tokens (and
    the first and last rows)."""
    import torch
    import synth
    m, n, k = 512, 14336, 4096
    wf = synth.normal_f32_torch((n, k), 0.02, "cuda", 0, "c5a", "w")
    wq = q.q8_0_quantize_rows(wf)
    xf = synth.normal_f32((m, k), 1.0, 0, "c5a", "x")
    xq = orc.quantize_rows(xf)
    y = nan_like((m, n))
    q.q8_0_matmul(wq, to_gpu(xq), n, k, m, y=y)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, n - 1],
                                     np.random.default_rng(5).integers(0, n, 96)]))
    rows_t = torch.from_numpy(rows).cuda()
    w_rows = orc.quantize_rows(wf[rows_t].cpu().numpy())
    assert np.array_equal(wq[rows_t].cpu().numpy(), w_rows)
    ref = orc.matmul(w_rows, xq, rows.size, k, m)
    yy = y.cpu().numpy()
    assert np.all(np.isfinite(yy))
    assert_rows_close(yy[:, rows], ref)


@pytest.mark.parametrize("n,k,m,batch", [(300, 768, 1, 1), (1000, 2048, 1, 1), (257, 768, 2, 3),
                                         (129, 3072, 3, 1), (1000, 768, 8, 2), (100, 4096, 16, 1),
                                         (70, 256, 5, 4), (33, 8192, 1, 1), (40, 8192, 2, 1)])
def test_matmul_f32_fused(q, orc, n, k, m, batch):
    """fp32 activations quantized inside the product launch: bitwise equal to
    q8_0_quantize_rows followed by q8_0_matmul_batched, and within tolerance of
    the oracle.  Rows longer than the early-load window (k > 768 at m = 1)
    take the pass-by-pass path."""
    import torch
    nb = k // 32
    w = weights_q8(orc, batch * n, k, "f32", n, k, m)
    stride = k + 12                       # padded fp32 rows (floats, multiple of 4)
    xf = synth.normal_f32((batch * m, k), 1.0, "f32-x", n, k, m)
    xbuf = np.zeros((batch * m, stride), dtype=np.float32)
    xbuf[:, :k] = xf
    wg, xg = to_gpu(w), to_gpu(xbuf)
    y1 = nan_like((batch, m, n))
    d = q.make_f32_desc(wg, xg, y1, n, k, m=m, batch=batch, w_batch_stride=n * nb,
                        x_row_stride=stride, x_batch_stride=m * stride, y_row_stride=n,
                        y_batch_stride=m * n)
    q.q8_0_matmul_f32_batched([d], wg)
    # two-step reference on the GPU
    xq = q.q8_0_quantize_rows(torch.from_numpy(xf).cuda())
    y2 = nan_like((batch, m, n))
    d2 = q.make_desc(wg, xq, y2, n, k, m=m, batch=batch, w_batch_stride=n * nb,
                     x_row_stride=nb, x_batch_stride=m * nb, y_row_stride=n, y_batch_stride=m * n)
    q.q8_0_matmul_batched([d2], wg)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    xq_ref = orc.quantize_rows(xf)
    assert np.array_equal(xq.cpu().numpy(), xq_ref)
    yy = y1.cpu().numpy()
    for b in range(batch):
        ref = orc.matmul(w[b * n:(b + 1) * n], xq_ref[b * m:(b + 1) * m], n, k, m)
        assert_rows_close(yy[b], ref)


@pytest.mark.parametrize("m", [1, 2, 6])
def test_matmul_f32_fused_many_jobs(q, orc, m):
    """Several products of different widths in one fused launch (waves cross
    from one product to the next mid-range and requantize), against the
    two-launch path, bitwise."""
    import torch
    specs = [(96, 768, 5), (160, 2048, 2), (50, 256, 1), (700, 768, 1), (64, 4096, 1)]
    k_total = sum(k * b for _, k, b in specs)
    xf = synth.normal_f32((m, k_total), 1.0, "f32-many", m)
    xg = to_gpu(xf)
    xq = q.q8_0_quantize_rows(xg)
    nb_total = k_total // 32
    n_out = sum(n * b for n, _, b in specs)
    y1, y2 = nan_like((m, n_out)), nan_like((m, n_out))
    d1, d2, keep = [], [], []
    xoff = yoff = 0
    for i, (n, k, b) in enumerate(specs):
        nb = k // 32
        w = to_gpu(weights_q8(orc, b * n, k, "f32-many-w", i))
        keep.append(w)
        d1.append(q.make_f32_desc(w, (xg, xoff), (y1, yoff), n, k, m=m, batch=b,
                                  w_batch_stride=n * nb, x_row_stride=k_total, x_batch_stride=k,
                                  y_row_stride=n_out, y_batch_stride=n))
        d2.append(q.make_desc(w, (xq, xoff // 32), (y2, yoff), n, k, m=m, batch=b,
                              w_batch_stride=n * nb, x_row_stride=nb_total, x_batch_stride=nb,
                              y_row_stride=n_out, y_batch_stride=n))
        xoff += b * k
        yoff += b * n
    q.q8_0_matmul_f32_batched(d1, xg)
    q.q8_0_matmul_batched(d2, xg)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_read_probe(q):
    """The streaming-read probe reads every byte: a buffer whose 16-byte
    chunks xor to a known word gives that word's fold in the sink."""
    import torch
    n = 1 << 22
    buf = torch.zeros(n, dtype=torch.uint8, device="cuda")
    buf.view(torch.int32)[0] = 0x5A5A5A5A     # one nonzero word in the first range
    sink = torch.full((4096,), -1, dtype=torch.int32, device="cuda")
    q.q8_read_probe(buf, sink)
    torch.cuda.synchronize()
    s = sink.cpu().numpy()
    assert s[0] == 0x5A5A5A5A                 # lane 0 folds with lane 1 (which read zeros)
    assert (s[1:64] == 0).all()               # 64 ranges of 64 KB, the rest read zeros
    assert (s[64:] == -1).all()               # no workgroup past the buffer
