"""Exact int32 block sums from the kernels the product path runs (built with
the sums output), against the oracle's block sums, bit for bit: the prefill
matrix-core kernel (more than 16 token rows), the R8 decode engine (from Q8_0
rows and from fp32 rows quantized inside the launch), and the R8 small-batch
engine.  The fp32 results of each validation call are bitwise those of the
product call on the same inputs.  Also the two decode steps the benchmark
times, at their full sizes: every product of the Llama-2-110M-shaped step
(85 matvecs, one launch over R8 weights from fp32 rows) and of the
GPT-2-124M-shaped batch-8 step (49 products, one launch), every output row
against the oracle."""
import numpy as np
import pytest

import synth

from gpu_cases import acts_q8, assert_rows_close, nan_like, to_gpu, weights_q8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import moe_expert_ffn_q8_amd as q
    return q


def _same_bits(a, b):
    import torch
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("m,n,k", [(17, 70, 768), (129, 257, 512), (200, 300, 2048),
                                   (512, 96, 4096), (33, 1000, 256)])
def test_prefill_gemm_blocksums(q, orc, m, n, k):
    """More than 16 token rows: the matrix-core kernel's block sums, ragged m
    and n on both sides of its 128 x 128 tile."""
    print(f"case: gemm blocksums m={m} n={n} k={k}", flush=True)
    w = weights_q8(orc, n, k, "bs-gemm", m, n, k)
    x = acts_q8(orc, m, k, "bs-gemm-x", m, n, k)
    wg, xg = to_gpu(w), to_gpu(x)
    y, sums = q.q8_0_matmul_blocksums(wg, xg, n, k, m)
    assert np.array_equal(sums.cpu().numpy(), orc.matmul_blocksums(w, x, n, k, m))
    assert _same_bits(y, q.q8_0_matmul(wg, xg, n, k, m))
    assert_rows_close(y.cpu().numpy(), orc.matmul(w, x, n, k, m))


def test_c5a_blocksums_sampled(q, orc):
    """The full 512 x 4096 x 14336 prefill product: the block sums of 48
    sampled weight rows for all 512 tokens and all 128 blocks."""
    import torch
    m, n, k = 512, 14336, 4096
    print("case: gemm blocksums 512 x 14336 x 4096 (sampled rows)", flush=True)
    wf = synth.normal_f32_torch((n, k), 0.02, "cuda", 0, "c5a", "w")
    wq = q.q8_0_quantize_rows(wf)
    xq = orc.quantize_rows(synth.normal_f32((m, k), 1.0, 0, "c5a", "x"))
    _, sums = q.q8_0_matmul_blocksums(wq, to_gpu(xq), n, k, m)
    rows = np.unique(np.concatenate([[0, 127, 128, n - 1],
                                     np.random.default_rng(9).integers(0, n, 44)]))
    rows_t = torch.from_numpy(rows).cuda()
    w_rows = orc.quantize_rows(wf[rows_t].cpu().numpy())
    assert np.array_equal(wq[rows_t].cpu().numpy(), w_rows)     # the weights the oracle sees
    got = sums[:, rows_t, :].cpu().numpy()
    del sums
    assert np.array_equal(got, orc.matmul_blocksums(w_rows, xq, rows.size, k, m))


@pytest.mark.parametrize("n,k,batch", [(777, 768, 3), (13, 96, 1), (5, 8192, 2), (2048, 768, 2),
                                       (1031, 2048, 1)])
@pytest.mark.parametrize("x_f32", [False, True])
def test_r8_matvec_blocksums(q, orc, n, k, batch, x_f32):
    import torch
    print(f"case: r8 matvec blocksums n={n} k={k} batch={batch} f32={x_f32}", flush=True)
    nb = k // 32
    mb = q.q8_0_r8_bytes(n, k)
    ws = [weights_q8(orc, n, k, "bs-r8", n, k, b) for b in range(batch)]
    wr = torch.cat([q.q8_0_repack_r8(to_gpu(w), n, k) for w in ws])
    xf = synth.normal_f32((batch, k), 1.0, "bs-r8-x", n, k)
    xq = orc.quantize_rows(xf)
    y, y2 = nan_like((batch, n)), nan_like((batch, n))
    sums = torch.empty((batch, n, nb), dtype=torch.int32, device="cuda")
    if x_f32:
        xg = to_gpu(xf)
        d = q.make_r8_f32_desc(wr, xg, y, n, k, batch=batch, w_batch_stride=mb,
                               x_batch_stride=k, y_batch_stride=n)
        d2 = q.make_r8_f32_desc(wr, xg, y2, n, k, batch=batch, w_batch_stride=mb,
                                x_batch_stride=k, y_batch_stride=n)
        q.q8v_matvec_r8_f32_batched_blocksums([d], [sums], wr)
        q.q8_0_matvec_r8_f32_batched([d2], wr)
    else:
        xg = to_gpu(xq)
        d = q.make_r8_desc(wr, xg, y, n, k, batch=batch, w_batch_stride=mb, x_batch_stride=nb,
                           y_batch_stride=n)
        d2 = q.make_r8_desc(wr, xg, y2, n, k, batch=batch, w_batch_stride=mb, x_batch_stride=nb,
                            y_batch_stride=n)
        q.q8v_matvec_r8_batched_blocksums([d], [sums], wr)
        q.q8_0_matvec_r8_batched([d2], wr)
    torch.cuda.synchronize()
    assert _same_bits(y, y2)
    ss = sums.cpu().numpy()
    for b in range(batch):
        assert np.array_equal(ss[b], orc.matmul_blocksums(ws[b], xq[b:b + 1], n, k, 1)[0])
        assert_rows_close(y[b].cpu().numpy()[None, :], orc.matmul(ws[b], xq[b:b + 1], n, k, 1))


@pytest.mark.parametrize("n,k,m,batch", [(1000, 768, 1, 1), (257, 3072, 8, 2), (100, 4096, 16, 1),
                                         (70, 256, 5, 3), (2304, 768, 8, 1), (33, 2048, 13, 1)])
def test_r8_mm_blocksums(q, orc, n, k, m, batch):
    import torch
    print(f"case: r8 mm blocksums n={n} k={k} m={m} batch={batch}", flush=True)
    nb = k // 32
    mb = q.q8_0_r8_bytes(n, k)
    ws = [weights_q8(orc, n, k, "bs-r8mm", n, k, m, b) for b in range(batch)]
    wr = torch.cat([q.q8_0_repack_r8(to_gpu(w), n, k) for w in ws])
    xq = acts_q8(orc, batch * m, k, "bs-r8mm-x", n, k, m)
    xg = to_gpu(xq)
    y, y2 = nan_like((batch, m, n)), nan_like((batch, m, n))
    sums = torch.empty((batch, m, n, nb), dtype=torch.int32, device="cuda")
    kw = dict(m=m, batch=batch, w_batch_stride=mb, x_row_stride=nb, x_batch_stride=m * nb,
              y_row_stride=n, y_batch_stride=m * n)
    q.q8v_matmul_r8_batched_blocksums([q.make_r8_mm_desc(wr, xg, y, n, k, **kw)], [sums], wr)
    q.q8_0_matmul_r8_batched([q.make_r8_mm_desc(wr, xg, y2, n, k, **kw)], wr)
    torch.cuda.synchronize()
    assert _same_bits(y, y2)
    ss = sums.cpu().numpy()
    for b in range(batch):
        xb = xq[b * m:(b + 1) * m]
        assert np.array_equal(ss[b], orc.matmul_blocksums(ws[b], xb, n, k, m))
        assert_rows_close(y[b].cpu().numpy(), orc.matmul(ws[b], xb, n, k, m))


LLAMA_STACKS = [(768, 768, 48), (2048, 768, 24), (768, 2048, 12), (32000, 768, 1)]
GPT2_STACKS = [(2304, 768, 12), (768, 768, 12), (3072, 768, 12), (768, 3072, 12), (50257, 768, 1)]


def test_llama_step_r8_full(q, orc):
    """The Llama-2-110M-shaped decode step as the benchmark times it: every
    one of the 85 products over R8 weights from its fresh fp32 activation row,
    one launch.  All outputs against the oracle, all block sums exact, and
    the validation launch's outputs bitwise those of the product launch."""
    import torch
    print("case: Llama-110M step, 85 products, R8 weights from fp32 rows", flush=True)
    k_total = sum(k * b for _, k, b in LLAMA_STACKS)
    xf = synth.normal_f32((k_total,), 1.0, "step-full", "x")
    xg = to_gpu(xf)
    n_out = sum(n * b for n, _, b in LLAMA_STACKS)
    y, y2 = nan_like((n_out,)), nan_like((n_out,))
    descs, descs2, sums, keep, refs = [], [], [], [], []
    xoff = yoff = 0
    for si, (n, k, b) in enumerate(LLAMA_STACKS):
        nb = k // 32
        mb = q.q8_0_r8_bytes(n, k)
        wq = orc.quantize_rows(synth.normal_f32((b * n, k), 0.02, "step-full", si))
        wr = torch.cat([q.q8_0_repack_r8(to_gpu(wq[i * n:(i + 1) * n]), n, k) for i in range(b)])
        keep.append(wr)
        s = torch.empty((b, n, nb), dtype=torch.int32, device="cuda")
        sums.append(s)
        kw = dict(batch=b, w_batch_stride=mb, x_batch_stride=k, y_batch_stride=n)
        descs.append(q.make_r8_f32_desc(wr, (xg, xoff), (y, yoff), n, k, **kw))
        descs2.append(q.make_r8_f32_desc(wr, (xg, xoff), (y2, yoff), n, k, **kw))
        refs.append((wq, xoff, yoff, n, k, b))
        xoff += b * k
        yoff += b * n
    q.q8v_matvec_r8_f32_batched_blocksums(descs, sums, xg)
    q.q8_0_matvec_r8_f32_batched(descs2, xg)
    torch.cuda.synchronize()
    assert _same_bits(y, y2)
    yy = y.cpu().numpy()
    for (wq, xo, yo, n, k, b), s in zip(refs, sums):
        ss = s.cpu().numpy()
        xq = orc.quantize_rows(xf[xo:xo + b * k].reshape(b, k))
        for i in range(b):
            wi = wq[i * n:(i + 1) * n]
            assert np.array_equal(ss[i], orc.matmul_blocksums(wi, xq[i:i + 1], n, k, 1)[0])
            assert_rows_close(yy[yo + i * n:yo + (i + 1) * n][None, :],
                              orc.matmul(wi, xq[i:i + 1], n, k, 1))


def test_gpt2_step_batch8_full(q, orc):
    """The GPT-2-124M-shaped batch-8 step as the benchmark times it: 49
    products at 8 token rows in one q8_0_matmul_batched launch (the
    matrix-core small-batch engine), every output row of every product against
    the oracle; and the 50257 x 768 head's block sums at 8 rows from the same
    engine, exact."""
    import torch
    m = 8
    print("case: GPT-2 step, 49 products at 8 rows, one launch", flush=True)
    k_total = sum(k * b for _, k, b in GPT2_STACKS)
    nb_total = k_total // 32
    xq = orc.quantize_rows(synth.normal_f32((m, k_total), 1.0, "gpt2-full", "x"))
    xg = to_gpu(xq)
    n_out = sum(n * b for n, _, b in GPT2_STACKS)
    y = nan_like((m, n_out))
    descs, keep, refs = [], [], []
    xoff = yoff = 0
    for si, (n, k, b) in enumerate(GPT2_STACKS):
        nb = k // 32
        wq = orc.quantize_rows(synth.normal_f32((b * n, k), 0.02, "gpt2-full", si))
        wg = to_gpu(wq)
        keep.append(wg)
        descs.append(q.make_desc(wg, (xg, xoff), (y, yoff), n, k, m=m, batch=b,
                                 w_batch_stride=n * nb, x_row_stride=nb_total, x_batch_stride=nb,
                                 y_row_stride=n_out, y_batch_stride=n))
        refs.append((wq, xoff, yoff, n, k, b))
        xoff += b * nb
        yoff += b * n
    q.q8_0_matmul_batched(descs, xg)
    torch.cuda.synchronize()
    yy = y.cpu().numpy()
    xrows = xq.reshape(m, nb_total, 34)
    for wq, xo, yo, n, k, b in refs:
        nb = k // 32
        for i in range(b):
            xb = np.ascontiguousarray(xrows[:, xo + i * nb:xo + (i + 1) * nb]).reshape(m, -1)
            assert_rows_close(yy[:, yo + i * n:yo + (i + 1) * n],
                              orc.matmul(wq[i * n:(i + 1) * n], xb, n, k, m))
    wq, xo, _, n, k, _ = refs[-1]
    xb = np.ascontiguousarray(xrows[:, xo:xo + k // 32]).reshape(m, -1)
    _, sums = q.q8_0_matmul_blocksums(keep[-1], to_gpu(xb), n, k, m)
    assert np.array_equal(sums.cpu().numpy(), orc.matmul_blocksums(wq, xb, n, k, m))
