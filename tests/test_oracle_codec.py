"""Pins for the oracle's binary16 codec: against numpy's float16 conversion
(an independent, round-to-nearest-even implementation)."""
import numpy as np
import pytest


def test_f16_to_f32_exhaustive(orc):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_bits_to_f32_array(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _check_f32_range(orc, bits):
    x = bits.view(np.float32)
    got = orc.f32_to_f16_bits_array(x)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x3FF) != 0)
    bad = np.nonzero(got[~nan] != ref[~nan])[0]
    assert bad.size == 0, (hex(int(bits[~nan][bad[0]])), hex(int(got[~nan][bad[0]])),
                           hex(int(ref[~nan][bad[0]])))


@pytest.mark.parametrize("e32", [0, 1, 101, 102, 103, 110, 111, 112, 113, 126, 127,
                                 141, 142, 143, 255])
def test_f32_to_f16_every_mantissa(orc, e32):
    """Every mantissa, both signs, for exponents at the interesting edges:
    fp16 underflow to zero (e<=101), subnormal results (102..112), the
    subnormal/normal seam (112/113), ordinary values, overflow (142/143), inf/NaN."""
    m = np.arange(1 << 23, dtype=np.uint32)
    for sign in (0, 1):
        _check_f32_range(orc, (np.uint32(sign << 31) | np.uint32(e32 << 23) | m))


def test_f32_to_f16_random(orc):
    g = np.random.default_rng(12345)
    _check_f32_range(orc, g.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32))


def test_f32_to_f16_ties(orc):
    """Exact halfway points round to the even neighbour."""
    assert orc.f32_to_f16_bits(1.0 + 2.0 ** -11) == 0x3C00          # tie, even is 1.0
    assert orc.f32_to_f16_bits(1.0 + 3 * 2.0 ** -11) == 0x3C02      # tie, even is up
    assert orc.f32_to_f16_bits(2.0 ** -25) == 0x0000                 # half the smallest subnormal
    assert orc.f32_to_f16_bits(3 * 2.0 ** -25) == 0x0002             # 1.5 ulp -> 2
    assert orc.f32_to_f16_bits(65520.0) == 0x7C00                    # rounds past 65504
    assert orc.f32_to_f16_bits(65519.996) == 0x7BFF
