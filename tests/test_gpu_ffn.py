"""GPU parity of q8_0_up_gate_swiglu_batched (the dense FFN up_gate with SwiGLU
in one pass) against the oracle's dense up_gate (the one-expert MoE form):
fp32 h within 1e-5 per-row relative L2, every output written (outputs are
pre-filled with NaN), stacks of layers in one launch, ragged last tiles."""
import numpy as np
import pytest

import synth

from gpu_cases import assert_rows_close, nan_like, to_gpu, weights_q8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import moe_expert_ffn_q8_amd as q
    return q


def _check_stack(q, orc, specs, m, tag, sample_rows=None):
    """specs: (n_ff, n_embd, batch) stacks over one activation buffer [m][sum
    batch*n_embd] (Q8_0) and one output buffer [m][sum batch*n_ff]."""
    import torch
    k_total = sum(k * b for _, k, b in specs)
    h_total = sum(n * b for n, _, b in specs)
    xf = synth.normal_f32((m, k_total), 1.0, tag, "x")
    xq = orc.quantize_rows(xf)
    xg = to_gpu(xq)
    h = nan_like((m, h_total))
    descs, keep, ws = [], [], []
    xoff = hoff = 0
    for i, (n_ff, k, b) in enumerate(specs):
        nb = k // 32
        w = weights_q8(orc, b * 2 * n_ff, k, tag, "w", i)
        ws.append(w)
        wg = to_gpu(w)
        keep.append(wg)
        descs.append(q.make_up_gate_desc(wg, (xg, xoff), (h, hoff), n_ff, k, m=m, batch=b,
                                         w_batch_stride=2 * n_ff * nb, x_row_stride=k_total // 32,
                                         x_batch_stride=nb, h_row_stride=h_total,
                                         h_batch_stride=n_ff))
        xoff += b * nb
        hoff += b * n_ff
    q.q8_0_up_gate_swiglu_batched(descs, xg)
    torch.cuda.synchronize()
    hh = h.cpu().numpy()
    assert not np.isnan(hh).any()
    xoff = hoff = 0
    rng = np.random.default_rng(3)
    for (n_ff, k, b), w in zip(specs, ws):
        nb = k // 32
        wb = w.reshape(b, 2 * n_ff, nb * 34)
        entries = range(b) if sample_rows is None else sorted({0, b - 1, int(rng.integers(b))})
        for e in entries:
            xe = np.ascontiguousarray(xq[:, (xoff + e * nb) * 34:(xoff + (e + 1) * nb) * 34])
            if sample_rows is None:
                ref = orc.up_gate_swiglu(wb[e], xe, k, n_ff)
                assert_rows_close(hh[:, hoff + e * n_ff:hoff + (e + 1) * n_ff], ref)
            else:
                rows = np.unique(np.concatenate([[0, n_ff - 1], rng.integers(0, n_ff, sample_rows)]))
                wsel = np.ascontiguousarray(np.concatenate([wb[e][rows], wb[e][n_ff + rows]]))
                ref = orc.up_gate_swiglu(wsel, xe, k, len(rows))
                assert_rows_close(hh[:, hoff + e * n_ff + rows], ref)
        xoff += b * nb
        hoff += b * n_ff


@pytest.mark.parametrize("m", [1, 2])
def test_dense_up_gate_shapes(q, orc, m):
    """Several widths in one launch: k from 256 to 8192, ragged last tiles
    (n_ff not a multiple of the tile's rows), stacks of several layers."""
    specs = [(2048, 768, 3), (100, 256, 2), (777, 2048, 1), (64, 8192, 1), (5, 768, 4)]
    _check_stack(q, orc, specs, m, f"ffn-{m}")


def test_dense_up_gate_llama_ffn(q, orc):
    """The Llama-2-110M FFN up_gate of all 12 layers (n_embd 768, n_ff 2048)
    in one launch; sampled rows of three layers against the oracle."""
    _check_stack(q, orc, [(2048, 768, 12)], 1, "ffn-llama", sample_rows=40)


def test_dense_up_gate_matches_matmul_halves(q, orc):
    """The gate sums agree with q8_0_matmul_batched: every up row is
    made to give exactly 1 (one code 1 at scale 1.0 against an activation
    block whose first code is 1 at scale 1.0, all other up blocks at scale 0),
    so h = silu(g) with g the engine's gate output; the device's fp32 silu is
    checked against fp64 within the rounding of expf and two divisions."""
    import torch
    n_ff, k, m = 300, 768, 1
    nb = k // 32
    w = weights_q8(orc, 2 * n_ff, k, "ffn-halves", "w").reshape(2 * n_ff, nb * 34).copy()
    w[n_ff:] = 0
    w[n_ff:, 0:2] = np.array([0x3C00], dtype=np.uint16).view(np.uint8)     # block 0 scale 1.0
    w[n_ff:, 2] = 1                                                          # code 0 = 1
    xq = orc.quantize_rows(synth.normal_f32((m, k), 1.0, "ffn-halves", "x"))
    xq = xq.reshape(m, nb * 34).copy()
    xq[0, 0:2] = np.array([0x3C00], dtype=np.uint16).view(np.uint8)
    xq[0, 2] = 1
    wg, xg = to_gpu(w), to_gpu(xq)
    h = nan_like((m, n_ff))
    q.q8_0_up_gate_swiglu_batched([q.make_up_gate_desc(wg, xg, h, n_ff, k)], wg)
    y = nan_like((m, 2 * n_ff))
    q.q8_0_matmul_batched([q.make_desc(wg, xg, y, 2 * n_ff, k)], wg)
    torch.cuda.synchronize()
    yy = y.cpu().numpy().astype(np.float64)
    assert np.all(yy[0, n_ff:] == 1.0)
    g = yy[0, :n_ff]
    got = h.cpu().numpy()[0].astype(np.float64)
    np.testing.assert_allclose(got, g / (1.0 + np.exp(-g)), rtol=1e-6, atol=1e-30)
