"""Pins of the oracle's rounding of an fp64 value to bfloat16 (round to nearest,
ties to even), which the gradient reference applies to the output row before
delta = sum_d dO o when the forward hands its output over in bf16.

The reference here is independent of the oracle's method (scaling by a power of
two and rounding to an integer): every finite non-negative bfloat16 value is
enumerated from its bit pattern, the two values that bracket |x| are found by
search, and the nearer one is chosen by exact rational arithmetic, the one with
an even bit pattern on a tie; the step past the largest finite value is
infinity.  The inputs are chosen so that the plausible mistakes fail: exact
midpoints (truncation and ties away from zero differ there), values one fp64
step either side of a midpoint, and values within half a binary32 spacing of a
midpoint (rounding through binary32 first lands on the midpoint and then
rounds to even, the wrong way).
"""
import bisect
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from sequence_long_context_amd import synth

# every finite non-negative bf16 value, in increasing order of bit pattern (= of value)
_PATTERNS = np.arange(0x0000, 0x7F80, dtype=np.uint16)
_VALUES = [float(v) for v in synth.bf16_bits_to_f32(_PATTERNS).astype(np.float64)]
_OVERFLOW = 2.0 ** 128  # the step after the largest finite value (pattern 0x7F80: infinity)


def _nearest_even(x: float) -> float:
    if np.isnan(x):
        return x
    if np.isinf(x) or x == 0.0:
        return x
    a = abs(x)
    i = bisect.bisect_right(_VALUES, a) - 1  # _VALUES[i] <= a
    lo, lo_pat = _VALUES[i], i
    if lo == a:
        r = lo
    else:
        hi, hi_pat = (_VALUES[i + 1], i + 1) if i + 1 < len(_VALUES) else (_OVERFLOW, 0x7F80)
        d_lo, d_hi = Fraction(a) - Fraction(lo), Fraction(hi) - Fraction(a)
        if d_lo < d_hi or (d_lo == d_hi and lo_pat % 2 == 0):
            r = lo
        else:
            r = np.inf if hi == _OVERFLOW else hi
    return -r if x < 0 else r


def _midpoints(lo_exp: int, hi_exp: int, per_binade: int, seed: int):
    """Midpoints between consecutive bf16 values (exact in fp64: 9 significant bits)."""
    g = np.random.default_rng(seed)
    out = []
    for e in range(lo_exp, hi_exp):
        m = g.integers(128, 255, size=per_binade)  # 8-bit significands 128..254
        out.extend(((m + 0.5) * 2.0 ** (e - 7)).tolist())
    return np.array(out)


def _cases():
    g = np.random.default_rng(2024)
    mids = _midpoints(-126, 127, 6, 1)
    sub_mids = (g.integers(0, 127, size=200) + 0.5) * 2.0 ** -133  # subnormal midpoints
    mids = np.concatenate([mids, sub_mids])
    f32_half = np.abs(mids) * 2.0 ** -26  # well inside half a binary32 spacing
    cases = [
        mids, -mids,
        np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
        mids + f32_half, mids - f32_half,
        # random doubles over the whole bf16 range and into the subnormals / overflow
        g.standard_normal(4000) * np.exp2(g.integers(-140, 129, size=4000)),
        np.array([0.0, -0.0, 2.0 ** -134, 2.0 ** -134 * 1.0000001, 2.0 ** -135, 3 * 2.0 ** -134,
                  255.5 * 2.0 ** 120, np.nextafter(255.5 * 2.0 ** 120, 0), 2.0 ** 128, 1e300,
                  -1e300, np.inf, -np.inf, 1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8,
                  1.0 + 2.0 ** -8 + 2.0 ** -40, 1.0 + 2.0 ** -8 - 2.0 ** -40]),
    ]
    return np.concatenate(cases)


def test_round_bf16_against_exact_nearest_even():
    x = _cases()
    got = oracle.round_bf16(x)
    want = np.array([_nearest_even(v) for v in x])
    same = (got == want) & (np.signbit(got) == np.signbit(want))
    bad = np.flatnonzero(~same)
    assert bad.size == 0, [(x[i], got[i], want[i]) for i in bad[:5]]


def test_round_bf16_inputs_catch_plausible_mistakes():
    """The cases above separate the correct rounding from truncation, from ties away
    from zero and from rounding through binary32 first."""
    x = _cases()
    finite = np.isfinite(x) & (np.abs(x) < 2.0 ** 127)
    x = x[finite]
    want = np.array([_nearest_even(v) for v in x])
    f = x.astype(np.float32)
    trunc = synth.bf16_bits_to_f32((f.view(np.uint32) >> 16).astype(np.uint16)).astype(np.float64)
    twice = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(f)).astype(np.float64)
    q = np.floor(np.log2(np.abs(np.where(x == 0, 1.0, x)))) - 7
    q = np.maximum(q, -133)
    away = np.sign(x) * np.floor(np.abs(x) / 2.0 ** q + 0.5) * 2.0 ** q
    for name, wrong in (("truncation", trunc), ("via binary32", twice), ("ties away", away)):
        assert np.count_nonzero(wrong != want) > 100, name


def test_round_bf16_matches_torch_on_binary32_values():
    """For values that are binary32 numbers there is one rounding step either way, and
    PyTorch's CPU cast to bfloat16 (round to nearest even) is a library reference."""
    g = np.random.default_rng(5)
    f = (g.standard_normal(20000) * np.exp2(g.integers(-120, 120, size=20000))).astype(np.float32)
    u = f.view(np.uint32) & ~np.uint32(0xFFFF) | np.uint32(0x8000)  # exact bf16 midpoints
    f = np.concatenate([f, u.view(np.float32)])
    want = torch.from_numpy(f).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_bf16(f.astype(np.float64)), want)


def test_round_bf16_nan_and_identity_on_bf16_values():
    assert np.isnan(oracle.round_bf16(np.array([np.nan]))[0])
    vals = np.array(_VALUES[::7])
    np.testing.assert_array_equal(oracle.round_bf16(vals), vals)
    np.testing.assert_array_equal(oracle.round_bf16(-vals), -vals)
