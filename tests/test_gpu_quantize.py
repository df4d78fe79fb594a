"""GPU parity: q8_0_quantize_rows must reproduce the oracle's Q8_0 bytes bit
for bit (the quantized codes are integers decided in fp32 on both sides)."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import moe_expert_ffn_q8_amd as q
    return q


def _gpu_quant(q, x, stride=None):
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, k = x.shape
    if stride is not None and stride != k:
        buf = np.full((rows, stride), np.nan, dtype=np.float32)
        buf[:, :k] = x
        xt = torch.from_numpy(buf).cuda()
        out = q.q8_0_quantize_rows(xt, k=k)
    else:
        out = q.q8_0_quantize_rows(torch.from_numpy(x).cuda())
    return out.cpu().numpy()


def _mismatch(a, b):
    bad = np.nonzero(a.reshape(-1) != b.reshape(-1))[0]
    return bad.size, (bad[:5] if bad.size else None)


@pytest.mark.parametrize("rows,k,sigma", [(1, 768, 1.0), (768, 768, 0.02), (7, 2048, 1.0),
                                          (33, 4096, 3.0), (5, 32, 1.0), (3, 96, 1e-4),
                                          (1000, 160, 1e3)])
def test_quantize_bitexact(q, orc, rows, k, sigma):
    x = synth.normal_f32((rows, k), sigma, "gpu", "quant", rows, k)
    ref = orc.quantize_rows(x)
    got = _gpu_quant(q, x)
    assert got.shape == ref.shape
    assert _mismatch(got, ref)[0] == 0, _mismatch(got, ref)


def test_quantize_row_stride(q, orc):
    x = synth.normal_f32((9, 256), 1.0, "gpu", "stride")
    assert np.array_equal(_gpu_quant(q, x, stride=260), orc.quantize_rows(x))


def test_quantize_ties_zeros_tiny_and_huge(q, orc):
    g = np.random.default_rng(3)
    n = 2048
    ints = g.integers(-126, 126, size=(n, 32)).astype(np.float64) + 0.5
    ints[:, 0] = 127.0
    scale = 2.0 ** g.integers(-30, 20, size=(n, 1))
    x = (ints * scale).astype(np.float32)
    x[5] = 0.0                                   # all-zero block
    x[6, :] = 0.0; x[6, 3] = -1e-40              # subnormal input, subnormal d
    x[7] = g.standard_normal(32).astype(np.float32) * np.float32(1e-38)
    x[8] = g.standard_normal(32).astype(np.float32) * np.float32(1e6)
    x[9, :] = -0.0
    x = x.reshape(1, -1)
    ref = orc.quantize_rows(x)
    got = _gpu_quant(q, x)
    assert _mismatch(got, ref)[0] == 0, _mismatch(got, ref)


def test_quantize_c5a_activations(q, orc):
    """The prefill activations: 512 x 4096 N(0,1)."""
    x = synth.normal_f32((512, 4096), 1.0, "c5a", "x")
    assert np.array_equal(_gpu_quant(q, x), orc.quantize_rows(x))
