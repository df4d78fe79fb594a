"""Pins for the oracle's row-interleaved weight layout (R8) and its matvec.

The Gemma-4-on-Xeon page (section on the fallback's cost and the repacking
bug) names Q8_0_R8: quantized weights reordered at startup into an
interleaved form.  It prints no layout; the library's reading is 8-row groups
of 272*nb bytes, the group's binary16 scales ordered by (block, row), then its
codes ordered by (block, row, position), the last group padded with zero rows.

Pins: byte positions of a small case listed by hand from that statement; the
repacked bytes are the native bytes plus padding zeros (a permutation); the
R8 matvec equals the native matvec bit for bit (same sums, same order), and the
native matvec is pinned by its own tests."""
import numpy as np
import pytest


def _native(n, nb):
    """Row i, block b: scale bits 0x3C00 + 16*i + b; code j = (j + 3*b + 7*i) % 97 - 48."""
    w = np.zeros((n, nb, 34), dtype=np.uint8)
    for i in range(n):
        for b in range(nb):
            sb = 0x3C00 + 16 * i + b
            w[i, b, 0] = sb & 0xFF
            w[i, b, 1] = sb >> 8
            w[i, b, 2:] = np.array([(j + 3 * b + 7 * i) % 97 - 48 for j in range(32)],
                                   dtype=np.int8).view(np.uint8)
    return w.reshape(n, nb * 34)


def _u16(a, off):
    return int(a[off]) | (int(a[off + 1]) << 8)


def _code(i, b, j):
    return ((j + 3 * b + 7 * i) % 97 - 48) & 0xFF


def test_r8_hand_positions(orc):
    # n = 9 rows, k = 64 (2 blocks): two groups of 544 bytes; group 0 holds
    # rows 0..7, group 1 holds row 8 and seven zero rows.  Scales of a group
    # occupy its first 32 bytes (16 per block), codes start at byte 32, one
    # 256-byte run per block, 32 bytes per row inside it.
    n, k = 9, 64
    out = orc.repack_r8(_native(n, 2), n, k)
    assert out.size == 1088
    assert _u16(out, 0) == 0x3C00            # row 0, block 0
    assert _u16(out, 2) == 0x3C10            # row 1, block 0
    assert _u16(out, 14) == 0x3C70           # row 7, block 0
    assert _u16(out, 16) == 0x3C01           # row 0, block 1
    assert _u16(out, 30) == 0x3C71           # row 7, block 1
    assert out[32] == _code(0, 0, 0)
    assert out[63] == _code(0, 0, 31)
    assert out[64] == _code(1, 0, 0)
    assert out[288] == _code(0, 1, 0)
    assert out[517] == _code(7, 1, 5)
    assert out[543] == _code(7, 1, 31)
    assert _u16(out, 544) == 0x3C80          # row 8, block 0 (group 1)
    assert _u16(out, 546) == 0               # row 9: padding
    assert _u16(out, 560) == 0x3C81          # row 8, block 1
    assert out[576] == _code(8, 0, 0)
    assert out[607] == _code(8, 0, 31)
    assert out[608] == 0                     # row 9 code 0: padding
    assert out[832] == _code(8, 1, 0)
    assert out[1087] == 0


@pytest.mark.parametrize("n,k", [(1, 32), (8, 96), (13, 96), (40, 256), (7, 2048)])
def test_r8_is_a_permutation_plus_padding(orc, n, k):
    g = np.random.default_rng(n * 1000 + k)
    nb = k // 32
    w = g.integers(0, 256, size=(n, nb * 34), dtype=np.uint8)
    out = orc.repack_r8(w, n, k)
    groups = (n + 7) // 8
    assert out.size == groups * 8 * nb * 34 == orc.r8_bytes(n, k)
    pad = np.zeros((groups * 8 - n) * nb * 34, dtype=np.uint8)
    assert np.array_equal(np.sort(out), np.sort(np.concatenate([w.ravel(), pad])))
    if n % 8 == 0:
        assert orc.r8_bytes(n, k) == n * nb * 34


@pytest.mark.parametrize("n,k", [(1, 32), (9, 64), (21, 160), (64, 768), (3, 2048)])
def test_r8_matvec_equals_native(orc, n, k):
    g = np.random.default_rng(7 * n + k)
    w = orc.quantize_rows(g.normal(0, 0.02, size=(n, k)).astype(np.float32))
    x = orc.quantize_rows(g.normal(0, 1, size=(1, k)).astype(np.float32))
    y_r8 = orc.matvec_r8(orc.repack_r8(w, n, k), x, n, k)
    y = orc.matvec(w, x, n, k)
    assert np.array_equal(y_r8, y)


def test_r8_matvec_reads_scales_per_row_and_block(orc):
    # a swapped (block, row) order would pair row 0's codes with another
    # row's scale: with all codes 1 and scale 2^r for row r, block b scaled by
    # (b + 1), y[r] = sum_b 32 * 2^r * (b + 1) * d_x exactly
    n, nb = 8, 3
    w = np.zeros((n, nb, 34), dtype=np.uint8)
    for r in range(n):
        for b in range(nb):
            bits = orc.f32_to_f16_bits(float(2 ** r * (b + 1)))
            w[r, b, 0], w[r, b, 1] = bits & 0xFF, bits >> 8
            w[r, b, 2:] = 1
    x = orc.quantize_rows(np.full((1, nb * 32), 127.0, dtype=np.float32))  # d = 1, codes 127
    y = orc.matvec_r8(orc.repack_r8(w.reshape(n, -1), n, nb * 32), x, n, nb * 32)
    assert list(y) == [32 * 127 * 2 ** r * 6 for r in range(n)]


def test_r8_bad_shapes(orc):
    with pytest.raises(ValueError):
        orc.r8_bytes(4, 48)
    with pytest.raises(ValueError):
        orc.r8_bytes(-1, 64)
    assert orc.r8_bytes(0, 64) == 0
