"""Pins for the oracle's block dot product and Q8_0 matvec/matmul.

The block dot product (the role of ggml_vec_dot_q8_0_q8_0 on the Gemma-4-on-Xeon
page, section on narrowing down the cause) is an exact integer sum followed by
scaling with both block scales.  Pins: closed-form block sums, an int64 brute
force with numpy, the dequantize-then-fp64 matmul (numpy), and special cases
where the fp64 result is exact."""
import numpy as np
import pytest

import synth
from qref import blocksums as np_blocksums, matmul as np_matmul, parse


def _blk(scale_bits, codes):
    b = np.zeros(34, dtype=np.uint8)
    b[0] = scale_bits & 0xFF
    b[1] = scale_bits >> 8
    b[2:] = np.asarray(codes, dtype=np.int8).view(np.uint8)
    return b


def test_block_dot_closed_forms(orc):
    one = 0x3C00
    assert orc.block_dot(_blk(one, [127] * 32), _blk(one, [127] * 32)) == 32 * 127 * 127
    assert orc.block_dot(_blk(one, [-128] * 32), _blk(one, [-128] * 32)) == 524288
    assert orc.block_dot(_blk(one, [127] * 32), _blk(one, [-128] * 32)) == -32 * 127 * 128
    alt = [(-1) ** j * 100 for j in range(32)]
    assert orc.block_dot(_blk(one, alt), _blk(one, [50] * 32)) == 0
    ramp = list(range(-16, 16))
    assert orc.block_dot(_blk(one, ramp), _blk(one, ramp)) == sum(v * v for v in ramp)
    # the scale bytes do not enter the integer sum
    assert orc.block_dot(_blk(0x7BFF, ramp), _blk(0x0001, ramp)) == sum(v * v for v in ramp)


def _rand_q8(rows, k, seed):
    g = np.random.default_rng(seed)
    nb = k // 32
    b = g.integers(0, 256, size=(rows, nb, 34), dtype=np.uint8)
    # keep the scales finite: exponent field below 31
    d = g.integers(0, 0x7C00, size=(rows, nb), dtype=np.uint16)
    d |= (g.integers(0, 2, size=(rows, nb), dtype=np.uint16) << 15)
    b[..., 0] = d & 0xFF
    b[..., 1] = d >> 8
    return b.reshape(rows, nb * 34)


@pytest.mark.parametrize("n,k,m", [(7, 32, 1), (5, 96, 3), (33, 768, 2), (16, 256, 8)])
def test_blocksums_brute_force(orc, n, k, m):
    w = _rand_q8(n, k, 1 + n)
    x = _rand_q8(m, k, 2 + m)
    assert np.array_equal(orc.matmul_blocksums(w, x, n, k, m), np_blocksums(w, x, n, k, m))


@pytest.mark.parametrize("n,k,m", [(64, 32, 1), (48, 64, 3), (37, 768, 2), (8, 2048, 5),
                                   (3, 4096, 1)])
def test_matmul_vs_dequantized_fp64(orc, n, k, m):
    wf = synth.normal_f32((n, k), 0.02, "test", "mm-w", n, k)
    xf = synth.normal_f32((m, k), 1.0, "test", "mm-x", m, k)
    w = orc.quantize_rows(wf)
    x = orc.quantize_rows(xf)
    got = orc.matmul(w, x, n, k, m)
    ref = np_matmul(w, x, n, k, m)
    assert got.shape == (m, n)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_matmul_random_bytes_vs_dequantized(orc):
    """Arbitrary block bytes (codes -128..127, any finite scale), not just
    quantizer output; catches a transposed operand on a non-square case."""
    n, k, m = 29, 320, 4
    w = _rand_q8(n, k, 11)
    x = _rand_q8(m, k, 12)
    got = orc.matmul(w, x, n, k, m)
    ref = np_matmul(w, x, n, k, m)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-300)


def test_single_block_is_exact(orc):
    """k = 32: y = d_w*d_x*s is one exact fp64 product."""
    w = _rand_q8(50, 32, 21)
    x = _rand_q8(1, 32, 22)
    dw, cw = parse(w, 1)
    dx, cx = parse(x, 1)
    want = dw[:, 0] * dx[0, 0] * (cw[:, 0, :] @ cx[0, 0, :])
    assert np.array_equal(orc.matvec(w, x, 50, 32), want)


def test_unit_scales_give_integer_sums(orc):
    """d_w = d_x = 1: y is the exact integer sum of all block sums."""
    n, k = 9, 512
    w = _rand_q8(n, k, 31).reshape(n, k // 32, 34)
    x = _rand_q8(1, k, 32).reshape(1, k // 32, 34)
    w[..., 0], w[..., 1] = 0x00, 0x3C
    x[..., 0], x[..., 1] = 0x00, 0x3C
    y = orc.matvec(w, x, n, k)
    s = np_blocksums(w, x, n, k, 1)[0].sum(axis=1)
    assert np.array_equal(y, s.astype(np.float64))


def test_row_ranges_and_selection_agree(orc):
    n, k, m = 40, 256, 3
    w = _rand_q8(n, k, 41)
    x = _rand_q8(m, k, 42)
    full = orc.matmul(w, x, n, k, m)
    part = orc.matmul(w, x, n, k, m, 10, 25)
    assert np.array_equal(part[:, 10:25], full[:, 10:25])
    assert np.all(part[:, :10] == 0) and np.all(part[:, 25:] == 0)
    rows = [0, 39, 17, 17, 5]
    assert np.array_equal(orc.matmul_rows(w, x, n, k, m, rows), full[:, rows])
