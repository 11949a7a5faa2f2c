"""Comparison rules shared by the GPU parity tests.

- Max-pool results are compared bit for bit.  A -0/+0 pair in the same position
  is the one accepted difference (the max of a window holding both zeros may
  return either sign); such ties are counted and reported, never silently
  merged with the bit-exact positions.
- bf16 outputs are pinned to round-to-nearest-even of the oracle's double
  result: the stored bf16 value must be RNE(v) for some v within `err` of the
  oracle's value (err = the fp32 path's own error budget before the final
  rounding), and for large outputs at least 99% of the values must equal
  RNE(ref) exactly.  A truncating or otherwise biased conversion fails both.
"""
from __future__ import annotations

import sys

import numpy as np


def report(*a):
    print("[cmp]", *a, file=sys.stderr, flush=True)


def assert_pool_bitexact(got: np.ndarray, ref: np.ndarray, what: str = "") -> int:
    """Bit-for-bit equality of float32 arrays, -0/+0 ties excepted and counted."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert got.dtype == np.float32 and ref.dtype == np.float32
    gb = got.view(np.uint32)
    rb = ref.view(np.uint32)
    diff = gb != rb
    ndiff = int(np.count_nonzero(diff))
    ties = 0
    if ndiff:
        d_got = got[diff]
        d_ref = ref[diff]
        zero_pair = (d_got == 0) & (d_ref == 0)
        ties = int(np.count_nonzero(zero_pair))
        bad = ndiff - ties
        if bad:
            i = np.flatnonzero(diff)[np.flatnonzero(~zero_pair)[0]]
            raise AssertionError(f"{what}: {bad} of {got.size} outputs differ from the oracle "
                                 f"(first at flat index {i}: got {got.ravel()[i]!r}, "
                                 f"ref {ref.ravel()[i]!r})")
    report(f"{what}: {got.size} outputs bit-exact, -0/+0 ties: {ties}")
    return ties


def bf16_rne(v: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bit patterns, one rounding to nearest even (no double
    rounding through float32).  +-inf stay infinite; finite values beyond the
    bf16 range are not expected here."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    fin = np.isfinite(v)
    m, e = np.frexp(v[fin])              # v = m * 2^e, 0.5 <= |m| < 1
    r = np.rint(m * 256.0)               # 8 significant bits, ties to even
    q = np.ldexp(r, e - 8)               # exact in double and in float32
    out[fin] = (q.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    out[~fin] = (v[~fin].astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return out


def bf16_bits_of(got_f32: np.ndarray) -> np.ndarray:
    """The bf16 bit patterns of float32 values that are exact bf16 values."""
    g = np.ascontiguousarray(got_f32, dtype=np.float32)
    assert not np.any(g.view(np.uint32) & 0xFFFF), "values are not bf16"
    return (g.view(np.uint32) >> 16).astype(np.uint16)


def _bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# Error budget of the fp32 arithmetic before the final bf16 rounding: the fp32
# paths' products, sums and exp/reciprocal-based tanh, softmax and sigmoid stay
# within about 1e-6 of the double results at these magnitudes; the budget is 20x
# that plus a relative term for large plain-conv sums, and still far below half
# a bf16 ulp (2^-9 relative) wherever |ref| > 0.01.
BF16_ERR_ABS = 2e-5
BF16_ERR_REL = 2.0 ** -14


def assert_bf16_rne(got_f32: np.ndarray, ref: np.ndarray, what: str = "",
                    err_abs: float = BF16_ERR_ABS, err_rel: float = BF16_ERR_REL,
                    min_exact: float = 0.99) -> float:
    """got (bf16 values widened to float32) against the oracle's double results."""
    assert got_f32.shape == ref.shape, (got_f32.shape, ref.shape)
    gb = bf16_bits_of(got_f32)
    exact = gb == bf16_rne(ref)
    frac = float(np.count_nonzero(exact)) / max(1, exact.size)
    fin = np.isfinite(ref)
    g = _bits_to_f64(gb)
    rf = ref[fin]
    err = err_abs + err_rel * np.abs(rf)
    lo = _bits_to_f64(bf16_rne(rf - err))
    hi = _bits_to_f64(bf16_rne(rf + err))
    ok = (g[fin] >= lo) & (g[fin] <= hi)
    if not ok.all():
        i = np.flatnonzero(~ok)[0]
        raise AssertionError(f"{what}: {np.count_nonzero(~ok)} bf16 outputs are not a "
                             f"round-to-nearest-even of a value within {err_abs} + "
                             f"{err_rel}|ref| of the oracle "
                             f"(first: got {g[fin][i]!r}, ref {rf[i]!r})")
    assert np.array_equal(gb[~fin], bf16_rne(ref[~fin])), f"{what}: non-finite outputs differ"
    report(f"{what}: {exact.size} bf16 outputs, RNE(oracle) exactly: {frac:.6f}")
    if exact.size >= 10000:
        assert frac >= min_exact, f"{what}: only {frac:.4f} of the outputs equal RNE(oracle)"
    return frac


def max_abs_err(got: np.ndarray, ref: np.ndarray, what: str = "") -> float:
    fin = np.isfinite(ref)
    e = float(np.max(np.abs(got[fin].astype(np.float64) - ref[fin]))) if fin.any() else 0.0
    report(f"{what}: max abs err {e:.3e} over {int(fin.sum())} outputs")
    return e
