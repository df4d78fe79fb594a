"""GPU parity of the Q8_1 quantizer (bytes exact) and of the decode product
over Q4_K / Q5_K super-blocks (within 1e-5 per-row relative L2 of the oracle;
exact where every value and scale is an integer; bitwise from run to run)."""
import numpy as np
import pytest

import synth

from gpu_cases import assert_rows_close, nan_like, to_gpu

pytestmark = pytest.mark.gpu

KSHAPES = [(1, 256), (21, 768), (22, 768), (777, 768), (1000, 2048), (100, 4096), (37, 8192),
           (3, 512)]


@pytest.fixture(scope="module")
def q():
    import moe_expert_ffn_q8_amd as q
    return q


@pytest.mark.parametrize("n_rows,k", [(1, 32), (3, 768), (17, 2048), (512, 4096)])
def test_q8_1_quantize_bytes(q, orc, n_rows, k):
    import torch
    x = synth.normal_f32((n_rows, k), 1.0, "q81", n_rows, k)
    x[0, :32] = 0.0
    if k >= 64:
        x[-1, 32:64] *= 1e-3
    y = q.q8_1_quantize_rows(torch.from_numpy(x).cuda()).cpu().numpy()
    ref = orc.quantize_rows_q8_1(x)
    bad = np.argwhere(y != ref)
    assert bad.size == 0, f"{len(bad)} bytes differ, first at (row, byte) {bad[:8].tolist()}: " \
        f"got {[int(y[tuple(b)]) for b in bad[:8]]}, want {[int(ref[tuple(b)]) for b in bad[:8]]}"


def test_q8_1_quantize_strided(q, orc):
    import torch
    x = synth.normal_f32((5, 1024), 1.0, "q81s")
    xg = torch.from_numpy(x).cuda()[:, :512]                 # row stride 1024 floats
    y = q.q8_1_quantize_rows(xg, k=512)
    assert np.array_equal(y.cpu().numpy(), orc.quantize_rows_q8_1(x[:, :512]))


@pytest.mark.parametrize("t", [4, 5])
@pytest.mark.parametrize("n,k", KSHAPES)
def test_kq_matvec(q, orc, t, n, k):
    w = synth.kq_blocks(t, n, k, "kq", t, n, k)
    x = orc.quantize_rows_q8_1(synth.normal_f32((1, k), 1.0, "kq-x", t, n, k))
    wg, xg = to_gpu(w), to_gpu(x)
    y = nan_like((n,))
    q.kq_matvec(t, wg, xg, n, k, y=y)
    ref = orc.kq_matvec(t, w, x, n, k)
    assert_rows_close(y.cpu().numpy()[None, :], ref[None, :])
    y2 = q.kq_matvec(t, wg, xg, n, k)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y2.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("t", [4, 5])
def test_kq_matvec_integer_case_exact(q, orc, t):
    """d = 1, dmin = 1 and activation scale 1 (amax 127): every term is an
    integer and every partial sum stays below 2^24, so the fp32 output is exact
    in any order."""
    n, k = 40, 2048
    w = synth.kq_blocks(t, n, k, "kqi", t).reshape(n, k // 256, -1)
    w[..., 0:4] = [0x00, 0x3C, 0x00, 0x3C]
    w = w.reshape(n, -1)
    xf = np.rint(synth.normal_f32((1, k), 30.0, "kqi-x", t)).clip(-127, 127).astype(np.float32)
    xf.reshape(-1, 32)[:, 0] = 127.0                          # amax 127 in every block: d = 1
    x = orc.quantize_rows_q8_1(xf)
    y = nan_like((n,))
    q.kq_matvec(t, to_gpu(w), to_gpu(x), n, k, y=y)
    ref = orc.kq_matvec(t, w, x, n, k)
    assert np.all(np.abs(ref) < 2 ** 24) and np.all(ref == np.rint(ref))
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("t", [4, 5])
def test_kq_batched_with_gaps(q, orc, t):
    import torch
    cases = [(300, 768, 3), (64, 2048, 2), (5, 8192, 1), (21, 256, 2)]
    bb = {4: 144, 5: 176}[t]
    descs, keep = [], []
    for ci, (n, k, batch) in enumerate(cases):
        ws = [synth.kq_blocks(t, n, k, "kqb", t, ci, b) for b in range(batch)]
        xs = [orc.quantize_rows_q8_1(synth.normal_f32((1, k), 1.0, "kqb-x", t, ci, b))
              for b in range(batch)]
        wg = to_gpu(np.concatenate([w.ravel() for w in ws]))
        xg = to_gpu(np.concatenate([x.ravel() for x in xs]))
        ys = n + 5
        y = nan_like((batch * ys,))
        descs.append(q.make_kq_desc(wg, xg, y, n, k, batch=batch, w_batch_stride=n * (k // 256),
                                    x_batch_stride=k // 32, y_batch_stride=ys))
        refs = np.stack([orc.kq_matvec(t, ws[b], xs[b], n, k) for b in range(batch)])
        keep.append((wg, xg, y, n, ys, refs))
    q.kq_matvec_batched(t, descs, keep[0][0])
    for wg, xg, y, n, ys, refs in keep:
        yy = y.cpu().numpy().reshape(-1, ys)
        assert np.all(np.isnan(yy[:, n:])), "a gap between output vectors was written"
        assert_rows_close(yy[:, :n], refs)


@pytest.mark.parametrize("t", [4, 5])
def test_kq_full_size_vocab(q, orc, t):
    """262144 x 2048 at full size, super-blocks drawn on the GPU; sampled rows
    computed by the oracle from the same bytes."""
    import torch
    n, k = 262144, 2048
    w = synth.kq_blocks_torch(t, n, k, "cuda", 0, "kq-c5b", t)
    xf = synth.normal_f32((1, k), 1.0, 0, "kq-c5b", "x")
    x = orc.quantize_rows_q8_1(xf)
    y = nan_like((n,))
    q.kq_matvec(t, w, to_gpu(x), n, k, y=y)
    rows = np.unique(np.concatenate([np.arange(8), n - 1 - np.arange(8),
                                     np.random.default_rng(2).integers(0, n, 2048)]))
    w_rows = w[torch.from_numpy(rows).cuda()].cpu().numpy()
    ref = orc.kq_matvec(t, w_rows, x, rows.size, k)
    yy = y.cpu().numpy()
    assert np.all(np.isfinite(yy))
    assert_rows_close(yy[rows][None, :], ref[None, :])
