"""Pins of the oracle's rounding helpers (round_bf16, round_f32), which turn
its float64 values into exactly the bf16 / fp32 values the kernels store.

The expected values are worked out by hand from the formats, not by any
routine: bfloat16 has 8 significand bits (7 stored), so its spacing in
[1, 2) is 2^-7; fp32 has 24 (spacing 2^-23 in [1, 2)).  Ties go to the
neighbour with an even last significand bit.  Both formats share fp32's
exponent range, so fp32 subnormals map to bf16 subnormals with spacing
2^-133."""
import numpy as np
import pytest

import oracle

e = 2.0 ** -8  # half a bf16 spacing at 1


@pytest.mark.parametrize("x,want", [
    (1.0, 1.0),
    (1.0 + e, 1.0),                          # tie between 1 and 1 + 2^-7: even is 1
    (1.0 + e + 2.0 ** -20, 1.0 + 2.0 ** -7),  # just above the tie: up
    (1.0 + e - 2.0 ** -20, 1.0),             # just below the tie: down
    (1.0 + 3 * e, 1.0 + 2.0 ** -6),          # tie between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    (1.0 + 2 * e, 1.0 + 2.0 ** -7),          # representable
    (-(1.0 + e), -1.0),                      # negatives mirror
    (-(1.0 + 3 * e), -(1.0 + 2.0 ** -6)),
    (3.0 + 2.0 ** -7, 3.0),                  # spacing 2^-6 in [2, 4): tie, 3 = 1.1000000b even
    (255.5, 256.0),                          # spacing 1 at 255: 255 odd, tie goes up to 256
    (2.0 ** -133, 2.0 ** -133),              # smallest bf16 subnormal
    (1.5 * 2.0 ** -133, 2.0 ** -132),        # tie between 1 and 2 spacings: even is 2
    (0.75 * 2.0 ** -133, 2.0 ** -133),       # above half a spacing: up
    (2.0 ** -135, 0.0),                      # a quarter spacing: to zero (fp32 keeps it exactly)
    (0.0, 0.0),
])
def test_round_bf16_nearest_even(x, want):
    got = oracle.round_bf16(np.array([x]))[0]
    assert got == want, (x, got, want)


def test_round_bf16_overflow_and_specials():
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127     # largest bf16
    got = oracle.round_bf16(np.array([big, -big, np.inf, -np.inf, np.nan]))
    assert got[0] == big and got[1] == -big
    assert got[2] == np.inf and got[3] == -np.inf and np.isnan(got[4])
    # past largest + half a spacing (2^119) the value rounds to infinity
    assert oracle.round_bf16(np.array([big + 2.0 ** 120]))[0] == np.inf


def test_round_bf16_keeps_bf16_values_and_is_monotone():
    # every bf16 value of a few binades is a fixed point, and rounding keeps order
    m = np.arange(128)
    vals = np.concatenate([(1.0 + m / 128.0) * 2.0 ** p for p in (-126, -3, 0, 7, 100)])
    # and the bf16 subnormals: multiples of 2^-133 below 2^-126
    vals = np.concatenate([vals, m * 2.0 ** -133])
    vals = np.concatenate([vals, -vals])
    assert np.array_equal(oracle.round_bf16(vals), vals)
    x = np.sort(np.random.default_rng(0).standard_normal(20000))
    r = oracle.round_bf16(x)
    assert (np.diff(r) >= 0).all()
    # and the error is at most half a spacing (2^-8 relative to the binade)
    assert (np.abs(r - x) <= 2.0 ** (np.floor(np.log2(np.abs(x))) - 8)).all()


@pytest.mark.parametrize("x,want", [
    (1.0 + 2.0 ** -24, 1.0),                     # tie: even is 1
    (1.0 + 3 * 2.0 ** -24, 1.0 + 2.0 ** -22),    # tie between odd and even: even
    (1.0 + 2.0 ** -24 + 2.0 ** -40, 1.0 + 2.0 ** -23),
    (-(1.0 + 2.0 ** -24), -1.0),
    (2.0 ** -149, 2.0 ** -149),                  # smallest fp32 subnormal
    (1.5 * 2.0 ** -149, 2.0 ** -148),            # tie: even
    (2.0 ** -151, 0.0),
])
def test_round_f32_nearest_even(x, want):
    assert oracle.round_f32(np.array([x]))[0] == want
