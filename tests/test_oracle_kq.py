"""Pins for the oracle's Q8_1 activations and 4/5-bit K-quant weights.

The Gemma-4-on-Xeon page names quantize_row_q8_1_x4_T beside the Q8_0
quantizer (section on the three-part fix, compile fix); the other pages run
Q4_K_M / Q5_K_M model files.  No page prints a layout; the readings are
stated in q8_oracle.c (Q8_1: d, s, 32 codes; Q4_K / Q5_K super-blocks of 256
with 6-bit packed sub-block scales and mins).

Pins: 6-bit fields packed by hand; hand-made Q4_K and Q5_K super-blocks whose
values are listed by hand; Q8_1 d and codes equal to the (pinned) Q8_0
quantizer's and s computed by hand and by numpy's float16; the matvec against
a numpy dequantize-then-fp64 product written separately here, and against the
per-sub-block integer-sum form the kernels use."""
import numpy as np
import pytest

SC = [1, 2, 3, 4, 37, 45, 50, 63]
MN = [0, 5, 10, 15, 20, 33, 48, 62]
# SC / MN packed by hand: bytes 0-3 hold sc[0..3] and the top 2 bits of
# sc[4..7]; bytes 4-7 m[0..3] and the top 2 bits of m[4..7]; bytes 8-11 the
# low nibbles of sc[4..7] (low) and m[4..7] (high)
PACKED = [129, 130, 195, 196, 64, 133, 202, 207, 69, 29, 2, 239]


def test_kq_scale_min_hand_packed(orc):
    for j in range(8):
        assert orc.kq_scale_min(PACKED, j) == (SC[j], MN[j])


def _header(d_bits=0x3C00, dmin_bits=0x3800):
    return [d_bits & 0xFF, d_bits >> 8, dmin_bits & 0xFF, dmin_bits >> 8] + PACKED


def _qs():
    # byte 32c + l: low nibble l % 16 (sub-block 2c), high nibble (l + c) % 16 (sub-block 2c+1)
    return [(l % 16) | (((l + c) % 16) << 4) for c in range(4) for l in range(32)]


def test_q4k_hand_block(orc):
    blk = np.array(_header() + _qs(), dtype=np.uint8)       # d = 1.0, dmin = 0.5
    assert blk.size == 144
    v = orc.kq_dequantize(4, blk, 1, 256)[0]
    assert v[0 * 32 + 3] == 3.0            # sub-block 0: sc 1, m 0, q 3
    assert v[1 * 32 + 20] == 5.5           # sub-block 1: 2*4 - 0.5*5
    assert v[4 * 32 + 31] == 545.0         # sub-block 4: 37*15 - 0.5*20
    assert v[7 * 32 + 0] == 158.0          # sub-block 7: 63*3 - 0.5*62
    assert v[6 * 32 + 17] == 26.0          # sub-block 6: 50*1 - 0.5*48
    q = [[(l % 16) if j % 2 == 0 else (l + j // 2) % 16 for l in range(32)] for j in range(8)]
    want = np.array([[SC[j] * q[j][l] - 0.5 * MN[j] for l in range(32)] for j in range(8)])
    assert np.array_equal(v, want.ravel())


def test_q5k_hand_block(orc):
    qh = [1 << (l % 8) for l in range(32)]                  # high bit of value l set in sub-block l % 8
    blk = np.array(_header() + qh + _qs(), dtype=np.uint8)
    assert blk.size == 176
    v = orc.kq_dequantize(5, blk, 1, 256)[0]
    assert v[0 * 32 + 8] == 24.0           # q 8 + 16, sc 1, m 0
    assert v[3 * 32 + 11] == 104.5         # q 12 + 16, 4*28 - 0.5*15
    assert v[5 * 32 + 5] == 1018.5         # q 7 + 16, 45*23 - 0.5*33
    assert v[5 * 32 + 6] == 343.5          # q 8, 45*8 - 0.5*33
    assert v[0 * 32 + 1] == 1.0            # no high bit
    q = [[((l % 16) if j % 2 == 0 else (l + j // 2) % 16) + 16 * (l % 8 == j) for l in range(32)]
         for j in range(8)]
    want = np.array([[SC[j] * q[j][l] - 0.5 * MN[j] for l in range(32)] for j in range(8)])
    assert np.array_equal(v, want.ravel())


def test_q8_1_rule(orc):
    g = np.random.default_rng(11)
    x = g.normal(0, 1, size=(9, 256)).astype(np.float32)
    x[0, :32] = 0.0                                          # zero block: d = 0, s = 0
    q1 = orc.quantize_rows_q8_1(x).reshape(9, 8, 36)
    q0 = orc.quantize_rows(x).reshape(9, 8, 34)
    assert np.array_equal(q1[..., :2], q0[..., :2])          # d
    assert np.array_equal(q1[..., 4:], q0[..., 2:])          # codes
    codes = q1[..., 4:].view(np.int8).astype(np.int64)
    d32 = (np.abs(x.reshape(9, 8, 32)).max(axis=2) / np.float32(127)).astype(np.float32)
    s_ref = (d32 * codes.sum(axis=2).astype(np.float32)).astype(np.float16).view(np.uint16)
    s = q1[..., 2].astype(np.uint16) | (q1[..., 3].astype(np.uint16) << 8)
    assert np.array_equal(s, s_ref)
    assert s[0, 0] == 0
    # hand values: amax 127 gives d = 1; codes [127, -127, 3, -3, 1, 0...] sum to 1 -> s = 1.0
    xb = np.zeros((1, 32), dtype=np.float32)
    xb[0, :5] = [127.0, -127.0, 2.5, -2.5, 1.0]
    b = orc.quantize_rows_q8_1(xb)[0]
    assert (int(b[0]) | (int(b[1]) << 8)) == 0x3C00 and (int(b[2]) | (int(b[3]) << 8)) == 0x3C00
    assert list(b[4:9].view(np.int8)) == [127, -127, 3, -3, 1]
    # all 127: sum 4064 = 127 * 2^5, s = 4064 exactly (binary16 0x6BF0)
    b = orc.quantize_rows_q8_1(np.full((1, 32), 127.0, dtype=np.float32))[0]
    assert (int(b[2]) | (int(b[3]) << 8)) == 0x6BF0


def _rand_kq(g, t, n, k):
    bb = {4: 144, 5: 176}[t]
    w = g.integers(0, 256, size=(n, k // 256, bb), dtype=np.uint8)
    d = (g.uniform(0.5, 1.5, size=(n, k // 256)) * 0.02 / 40).astype(np.float16).view(np.uint16)
    dm = (g.uniform(0.5, 1.5, size=(n, k // 256)) * 0.02 / 20).astype(np.float16).view(np.uint16)
    w[..., 0], w[..., 1] = d & 0xFF, d >> 8
    w[..., 2], w[..., 3] = dm & 0xFF, dm >> 8
    return w.reshape(n, -1)


def _np_unpack(t, w, n, k):
    """Separate numpy reading of the super-block layout: d, dmin [n][S],
    sc, m [n][S][8], codes [n][S][8][32] (S = k/256)."""
    bb = {4: 144, 5: 176}[t]
    b = w.reshape(n, k // 256, bb)
    d = b[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    dm = b[..., 2:4].copy().view(np.float16)[..., 0].astype(np.float64)
    s12 = b[..., 4:16].astype(np.int64)
    sc = np.zeros(b.shape[:2] + (8,), dtype=np.int64)
    mn = np.zeros_like(sc)
    sc[..., :4] = s12[..., 0:4] & 63
    mn[..., :4] = s12[..., 4:8] & 63
    sc[..., 4:] = (s12[..., 8:12] & 15) | ((s12[..., 0:4] >> 6) << 4)
    mn[..., 4:] = (s12[..., 8:12] >> 4) | ((s12[..., 4:8] >> 6) << 4)
    qs = b[..., (16 if t == 4 else 48):].astype(np.int64).reshape(n, k // 256, 4, 32)
    q = np.stack([qs & 15, qs >> 4], axis=3).reshape(n, k // 256, 8, 32)
    if t == 5:
        qh = b[..., 16:48].astype(np.int64)
        q = q + 16 * ((qh[:, :, None, :] >> np.arange(8)[None, None, :, None]) & 1)
    return d, dm, sc, mn, q


def _np_dequant(t, w, n, k):
    d, dm, sc, mn, q = _np_unpack(t, w, n, k)
    return (d[..., None, None] * sc[..., None] * q - dm[..., None, None] * mn[..., None]).reshape(n, k)


@pytest.mark.parametrize("t", [4, 5])
@pytest.mark.parametrize("n,k", [(3, 256), (17, 768), (5, 2048)])
def test_kq_matvec_vs_numpy(orc, t, n, k):
    g = np.random.default_rng(100 * t + n + k)
    w = _rand_kq(g, t, n, k)
    x = orc.quantize_rows_q8_1(g.normal(0, 1, size=(1, k)).astype(np.float32))
    wd = _np_dequant(t, w, n, k)
    assert np.array_equal(orc.kq_dequantize(t, w, n, k), wd)
    xb = x.reshape(k // 32, 36)
    xd = xb[:, 0:2].copy().view(np.float16)[:, 0].astype(np.float64)
    xv = (xd[:, None] * xb[:, 4:].view(np.int8).astype(np.float64)).ravel()
    y = orc.kq_matvec(t, w, x, n, k)
    ref = wd @ xv
    assert np.allclose(y, ref, rtol=1e-12, atol=0)
    # the per-sub-block integer form the kernels use:
    # sum_j (d sc_j dx_j) S_j - (dmin m_j dx_j) Q_j, S_j = sum q q_x, Q_j = sum q_x
    d, dm, sc, mn, q = _np_unpack(t, w, n, k)
    qx = xb[:, 4:].view(np.int8).astype(np.int64).reshape(k // 256, 8, 32)
    S = (q * qx[None]).sum(axis=3)
    Q = qx.sum(axis=2)
    dxj = xd.reshape(k // 256, 8)
    alt = ((d[..., None] * sc * dxj[None]) * S - (dm[..., None] * mn * dxj[None]) * Q[None]).sum(axis=(1, 2))
    assert np.allclose(y, alt, rtol=1e-9, atol=1e-12)


def test_kq_bad_args(orc):
    with pytest.raises(ValueError):
        orc.kq_matvec(4, np.zeros(144, np.uint8), np.zeros(288, np.uint8), 1, 255)
    with pytest.raises(ValueError):
        orc.kq_matvec(6, np.zeros(144, np.uint8), np.zeros(288, np.uint8), 1, 256)
