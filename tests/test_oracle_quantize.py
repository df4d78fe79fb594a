"""Pins for the oracle's Q8_0 quantizer.

The rule (32 values per block; d = max|x|/127 in fp32, stored as binary16;
q = round(x/d), ties away from zero) is the format's definition; the pages name
the format and its quantizer (quantize_row_q8_0_x4, in the compile-fix part of
the three-part fix on the Gemma-4-on-Xeon page) but print no worked example.
So the pins are closed-form blocks whose scale is a power of two (every ratio
x/d is then exact and the expected codes can be written down), and invariants
that any correct implementation of the rule satisfies on random data.
"""
import numpy as np
import pytest

import synth


def q1(orc, x):
    """quantize one 32-value block -> (scale bits, codes)"""
    b = orc.quantize_rows(np.asarray(x, dtype=np.float32)[None, :])
    d, c = orc.split_blocks(b)
    return int(d[0, 0]), c[0, 0].astype(int)


def test_power_of_two_scale_and_ties(orc):
    # amax = 127 * 2^k -> d = 2^k exactly, x/d exact: expected codes by hand.
    for k in (0, -8, 3):
        s = 2.0 ** k
        vals = [127, 2.5, -2.5, 0.49, 0.5, -0.5, 1.5, -1.5, 126.5, -126.5, 0.0, -0.0,
                3.25, -3.75, 100.5, -7.5]
        want = [127, 3, -3, 0, 1, -1, 2, -2, 127, -127, 0, 0, 3, -4, 101, -8]
        x = np.zeros(32)
        x[: len(vals)] = np.array(vals) * s
        d, c = q1(orc, x)
        assert d == (15 + k) << 10                  # binary16 of 2^k
        assert list(c[: len(vals)]) == want         # half away from zero, not half even
        assert np.all(c[len(vals):] == 0)


def test_zero_block(orc):
    d, c = q1(orc, np.zeros(32))
    assert d == 0 and np.all(c == 0)


def test_negative_amax(orc):
    x = np.zeros(32); x[7] = -127.0; x[3] = 63.5
    d, c = q1(orc, x)
    assert d == 0x3C00 and c[7] == -127 and c[3] == 64


def test_scale_rounding_to_binary16(orc):
    # d32 = 1 + 2^-11 is halfway between binary16 1.0 and 1+2^-10: even -> 1.0
    x = np.zeros(32); x[0] = 127 * (1 + 2.0 ** -11); x[1] = 2.5 * (1 + 2.0 ** -11)
    d, c = q1(orc, x)
    assert d == 0x3C00 and c[0] == 127 and c[1] == 3     # codes use the fp32 d
    # d32 = 1 + 3*2^-11: halfway between mantissa 1 and 2: even -> 2
    x = np.zeros(32); x[0] = 127 * (1 + 3 * 2.0 ** -11)
    d, c = q1(orc, x)
    assert d == 0x3C02 and c[0] == 127


def test_scale_underflow_keeps_codes(orc):
    # d32 = 2^-26 is a quarter of the smallest binary16 subnormal: stored d = 0,
    # codes still come from the fp32 d.
    x = np.zeros(32); x[0] = 127 * 2.0 ** -26; x[1] = -2.5 * 2.0 ** -26
    d, c = q1(orc, x)
    assert d == 0 and c[0] == 127 and c[1] == -3
    # d32 = 2^-20 = 16 subnormal units
    x = np.zeros(32); x[0] = 127 * 2.0 ** -20
    d, c = q1(orc, x)
    assert d == 0x0010 and c[0] == 127


def _invariants(orc, x):
    x = np.asarray(x, dtype=np.float32)
    rows, k = x.shape
    q = orc.quantize_rows(x)
    dbits, codes = orc.split_blocks(q)
    xb = x.reshape(rows, k // 32, 32)
    amax = np.abs(xb).max(axis=2)
    d32 = amax / np.float32(127.0)                         # fp32 division (numpy)
    with np.errstate(over="ignore"):
        assert np.array_equal(dbits, d32.astype(np.float16).view(np.uint16))
    codes = codes.astype(np.int64)
    assert np.all(np.abs(codes) <= 127)
    nz = d32 > 0
    r = xb[nz].astype(np.float64) / d32[nz][:, None].astype(np.float64)   # exact-ish ratio
    c = codes[nz]
    # each code is a nearest integer to x/d (within 0.5, allowing one fp32 ulp of the
    # quotient), and at every amax position the code is +-127
    assert np.all(np.abs(r - c) <= 0.5 + 1e-5)
    at_max = np.abs(xb[nz]) == amax[nz][:, None]
    assert np.all(np.abs(c[at_max]) == 127)
    assert np.all(np.sign(c) * np.sign(xb[nz]) >= 0)      # never flips sign
    assert np.all(codes[~nz] == 0)
    return q


@pytest.mark.parametrize("sigma", [1.0, 0.02, 1e-3, 300.0])
def test_invariants_random(orc, sigma):
    x = synth.normal_f32((64, 2048), sigma, "test", "quant-invariants", int(sigma * 1000))
    _invariants(orc, x)


def test_invariants_with_exact_ties(orc):
    """Blocks with d a power of two and many values on n+1/2: every tie goes away
    from zero."""
    g = np.random.default_rng(7)
    n = 4096
    ints = g.integers(-126, 126, size=(n, 32)).astype(np.float64) + 0.5
    ints[:, 0] = 127.0 * np.where(g.random(n) < 0.5, -1, 1)
    scale = 2.0 ** g.integers(-12, 6, size=(n, 1))
    x = (ints * scale).astype(np.float32).reshape(1, n * 32)
    q = orc.quantize_rows(x)
    _, codes = orc.split_blocks(q)
    want = np.sign(ints) * np.floor(np.abs(ints) + 0.5)
    assert np.array_equal(codes[0].astype(np.float64), want)


def test_rows_and_stride_are_independent_blocks(orc):
    """Quantization is per 32-block: a [r][k] matrix gives the same bytes as its
    rows concatenated into one long row."""
    x = synth.normal_f32((5, 768), 1.0, "test", "rows")
    a = orc.quantize_rows(x)
    b = orc.quantize_rows(x.reshape(1, -1))
    assert np.array_equal(a.reshape(-1), b.reshape(-1))


def test_dequantization_error_bound(orc):
    """|x - fp16(d)*q| <= d/2 + |q| * |fp16(d) - d|: the block error bound."""
    x = synth.normal_f32((16, 1024), 1.0, "test", "deq")
    q = orc.quantize_rows(x)
    dbits, codes = orc.split_blocks(q)
    dh = dbits.view(np.float16).astype(np.float64)
    xb = x.reshape(16, 32, 32).astype(np.float64)
    d32 = (np.abs(x.reshape(16, 32, 32)).max(axis=2) / np.float32(127)).astype(np.float64)
    err = np.abs(xb - dh[..., None] * codes)
    bound = d32[..., None] / 2 * (1 + 1e-6) + np.abs(codes) * np.abs(dh - d32)[..., None]
    assert np.all(err <= bound + 1e-12)


def _round_half_away(r32):
    """sign(r) * floor(|r| + 1/2) of fp32 quotients, evaluated in fp64 (exact:
    an fp32 value plus one half is representable in fp64)."""
    r = np.asarray(r32, dtype=np.float32).astype(np.float64)
    return np.sign(r) * np.floor(np.abs(r) + 0.5)


def _codes_by_division(x):
    """Q8_0 codes of fp32 rows by the rule as written: d = amax / 127 and the
    quotient x / d, both IEEE fp32 divisions (numpy's float32 divide), then
    round half away from zero."""
    x = np.asarray(x, dtype=np.float32)
    xb = x.reshape(x.shape[0], -1, 32)
    d = (np.abs(xb).max(axis=2) / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = _round_half_away(xb / d[..., None])
    return np.where(d[..., None] > 0, q, 0.0)


@pytest.mark.parametrize("sigma", [1.0, 0.02])
def test_codes_equal_fp32_division_rule(orc, sigma):
    """Every code equals round-half-away(x / d) with the quotient an fp32
    division, exactly (not merely within half a unit): this separates the
    division from a reciprocal multiply or a 127/amax multiply, which give
    other codes for about one value in a million."""
    x = synth.normal_f32((256, 4096), sigma, "test", "quant-division", int(sigma * 1000))
    _, codes = orc.split_blocks(orc.quantize_rows(x))
    assert np.array_equal(codes.astype(np.float64), _codes_by_division(x))


def test_division_not_reciprocal_multiply(orc):
    """Blocks built from values one to three fp32 ulps from a rounding tie,
    chosen where x * (1/d) (and, for some, x * (127/amax)) rounds to another
    integer than x / d: the oracle must give the division's codes on all."""
    g = np.random.default_rng(11)
    blocks, n_recip, n_ratio = [], 0, 0
    while len(blocks) < 64:
        amax = np.float32(g.uniform(0.25, 8.0))
        d = amax / np.float32(127.0)
        inv = np.float32(1.0) / d
        ratio = np.float32(127.0) / amax
        ties = ((np.arange(126) + 0.5) * np.float64(d)).astype(np.float32)
        cand = []
        for direction in (np.float32(np.inf), np.float32(-np.inf)):
            x = ties.copy()
            for _ in range(3):
                x = np.nextafter(x, direction)
                a = _round_half_away(x / d)
                cand += [v for v, ok in zip(x, a != _round_half_away(x * inv)) if ok]
        if len(cand) < 8:
            continue
        vals = np.array(cand[:31], dtype=np.float32)
        sign = np.where(g.random(len(vals)) < 0.5, -1, 1).astype(np.float32)
        blk = np.zeros(32, dtype=np.float32)
        blk[0] = amax
        blk[1:1 + len(vals)] = vals * sign
        n_recip += int(np.sum(_round_half_away(blk / d) != _round_half_away(blk * inv)))
        n_ratio += int(np.sum(_round_half_away(blk / d) != _round_half_away(blk * ratio)))
        blocks.append(blk)
    x = np.stack(blocks).reshape(1, -1)
    _, codes = orc.split_blocks(orc.quantize_rows(x))
    assert n_recip >= 64 * 8                 # the blocks really separate the two forms
    assert n_ratio > 0
    assert np.array_equal(codes.astype(np.float64).reshape(1, -1, 32), _codes_by_division(x))
