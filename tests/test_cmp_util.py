"""CPU checks of the comparison rules the GPU parity tests use (tests/cmp_util.py):
the bf16 rounding reference is a single round-to-nearest-even of the double
value, the bf16 check rejects a truncating conversion, and the max-pool check
accepts only -0/+0 ties and counts them."""
import numpy as np
import pytest

import inputgen
from cmp_util import assert_bf16_rne, assert_pool_bitexact, bf16_rne


def test_bf16_rne_equals_integer_rounding_of_float32():
    x = inputgen.randn(11, (200000,), 3.0)
    assert np.array_equal(bf16_rne(x.astype(np.float64)), inputgen.to_bf16_bits(x))


def test_bf16_rne_ties_to_even_and_no_double_rounding():
    one = 0x3F80
    cases = [
        (1.0 + 2.0 ** -8, one),                       # midpoint -> even (1.0)
        (1.0 + 3 * 2.0 ** -8, one + 2),               # midpoint -> even (1 + 2^-6)
        (1.0 + 2.0 ** -8 + 2.0 ** -30, one + 1),      # just above the midpoint: rounds up;
                                                      # through float32 it would tie to 1.0
        (-(1.0 + 2.0 ** -8 + 2.0 ** -30), 0x8000 | (one + 1)),
        (1.0 + 2.0 ** -8 - 2.0 ** -30, one),
        (2.0 - 2.0 ** -9, 0x4000),                    # carries into the exponent
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (float("-inf"), 0xFF80),
    ]
    for v, bits in cases:
        assert int(bf16_rne(np.array([v]))[0]) == bits, (v, hex(bits))


def _truncate_bits(v):
    return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _as_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def test_bf16_check_accepts_rne_and_rejects_truncation():
    ref = inputgen.uniform(12, (50000,), -2.0, 2.0).astype(np.float64) + 1e-9
    assert_bf16_rne(_as_f32(bf16_rne(ref)), ref, "rne")
    # a value perturbed within the fp32 error budget, then rounded, still passes
    assert_bf16_rne(_as_f32(bf16_rne(ref + 3e-6)), ref, "rne of perturbed")
    with pytest.raises(AssertionError):
        assert_bf16_rne(_as_f32(_truncate_bits(ref)), ref, "truncated")
    # rounding half away from zero in the wrong direction on every value: rejected too
    off = bf16_rne(ref).astype(np.int32) + 1
    with pytest.raises(AssertionError):
        assert_bf16_rne(_as_f32(off.astype(np.uint16)), ref, "one ulp off")


def test_pool_check_counts_signed_zero_ties_only():
    ref = np.array([0.0, -0.0, 1.5, -2.0], dtype=np.float32)
    got = np.array([-0.0, 0.0, 1.5, -2.0], dtype=np.float32)
    assert assert_pool_bitexact(got, ref, "ties") == 2
    assert assert_pool_bitexact(ref.copy(), ref, "same") == 0
    bad = got.copy()
    bad[2] = np.nextafter(np.float32(1.5), np.float32(2.0))
    with pytest.raises(AssertionError):
        assert_pool_bitexact(bad, ref, "bad")
