"""Pin for the oracle's float64 -> bfloat16 rounding (CPU only).

bf16_round feeds the per-tensor FP8 forward (h is stored in bf16 before its scale is
taken) and the MXFP8 backward (dH and dZ go back to bf16 after their GEMMs, as the
MXFP8 recipe of "Efficient MoE Training for Biological Foundation Models", Challenge 3,
returns a low-precision GEMM's result to the higher precision). The expected values
come from a search over every finite bfloat16 bit pattern: the nearest one, and on an
exact tie the one whose last significand bit is 0. Overflow follows IEEE rounding:
2^128 (the next value past the largest finite one, with an even significand) stands
for infinity.
"""
import numpy as np

import oracle
from moe_inputs import f32_to_bf16_bits


def _codebook():
    bits = np.arange(1 << 16, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        vals = (bits << 16).view(np.float32).astype(np.float64)
    ok = np.isfinite(vals) & ~((vals == 0) & (bits != 0))   # drop NaN/inf and -0
    vals, bits = vals[ok], bits[ok]
    # the overflow candidates 2^128 (stands for +inf) and -2^128, significand even
    vals = np.concatenate([vals, [2.0 ** 128, -(2.0 ** 128)]])
    bits = np.concatenate([bits, [0x7F80, 0xFF80]])
    o = np.argsort(vals, kind="stable")
    return vals[o], bits[o]


VALS, BITS = _codebook()


def _brute(x):
    """Nearest bf16 value of each float64 in x by search; ties to the even bit pattern."""
    x = np.asarray(x, np.float64)
    hi = np.clip(np.searchsorted(VALS, x, side="left"), 1, len(VALS) - 1)
    lo = hi - 1
    dlo, dhi = np.abs(x - VALS[lo]), np.abs(VALS[hi] - x)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((BITS[hi] & 1) == 0))
    r = np.where(pick_hi, VALS[hi], VALS[lo])
    r = np.where(np.abs(r) == 2.0 ** 128, np.copysign(np.inf, r), r)
    return np.where(x == 0, x, r)


def _check(x):
    got = oracle.bf16_round(x)
    want = _brute(x)
    bad = ~((got == want) | (np.isnan(got) & np.isnan(want)))
    assert not bad.any(), (x[bad][:5], got[bad][:5], want[bad][:5])


def test_every_tie_and_its_neighbours():
    # all midpoints between consecutive finite bf16 values (both signs, subnormals, the
    # overflow midpoint), and the float64 values just above and just below each
    mid = 0.5 * (VALS[:-1] + VALS[1:])
    mid = mid[np.isfinite(mid)]
    for x in (mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)):
        _check(x)


def test_exact_values_and_specials():
    _check(VALS[np.abs(VALS) < 2.0 ** 128])        # every finite bf16 value maps to itself
    got = oracle.bf16_round(np.array([0.0, -0.0, np.inf, -np.inf, np.nan]))
    assert got[0] == 0 and not np.signbit(got[0]) and got[1] == 0 and np.signbit(got[1])
    assert got[2] == np.inf and got[3] == -np.inf and np.isnan(got[4])


def test_no_double_rounding():
    # 1 + 2^-8 is the tie between 1 and 1 + 2^-7; the 2^-30 above it is lost by a float32
    # intermediate (which rounds to the tie, then to even = 1) but decides the bf16 result
    x = np.array([1 + 2.0 ** -8 + 2.0 ** -30, -(1 + 2.0 ** -8 + 2.0 ** -30), 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8])
    assert list(oracle.bf16_round(x)) == [1 + 2.0 ** -7, -(1 + 2.0 ** -7), 1.0, 1 + 2.0 ** -6]
    _check(x)


def test_random_float64_across_the_range():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(200000) * np.exp2(rng.uniform(-140, 129, 200000))
    _check(x)
    # values that float32 cannot hold but bf16 rounding must still get right: below the
    # float32 subnormal range and 24-53 bits of significand
    y = rng.uniform(1, 2, 100000) * np.exp2(rng.integers(-134, 0, 100000).astype(np.float64))
    _check(y)


def test_float32_inputs_agree_with_the_input_generator():
    # on float32 values (one rounding, no double rounding possible) the oracle's rounding
    # gives the bit patterns the seeded input generator produces
    rng = np.random.default_rng(12)
    x = (rng.standard_normal(100000) * np.exp2(rng.uniform(-130, 120, 100000))).astype(np.float32)
    want = (f32_to_bf16_bits(x).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(oracle.bf16_round(x.astype(np.float64)), want)


def test_large_inputs_round_in_chunks_to_the_same_bits():
    # above 2^22 elements the rounding runs in chunks on threads: the same values
    rng = np.random.default_rng(21)
    v = rng.standard_normal((1 << 22) + 12345) * np.exp(rng.uniform(-30, 30, (1 << 22) + 12345))
    big = oracle.bf16_round(v)
    for i in (0, 1 << 21, (1 << 22) + 100):
        part = v[i:i + 5000]
        assert np.array_equal(oracle.bf16_round(part), big[i:i + 5000])
