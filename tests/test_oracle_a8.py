"""Pins of the INT8-activation oracle (oracle/a8.py) against a hand-worked
fixture, the rounding bound, the exact-representable case where it must equal
the W4A16 oracle, pure-Python brute force, and a planted per-row-scale mistake."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle.a8 import quantize_a8, dequantize_a8, gemv_w4a8

GOLD = os.path.join(os.path.dirname(__file__), "golden", "a8_hand.json")


def test_quantize_a8_hand_fixture():
    fx = json.load(open(GOLD))
    G = fx["group"]
    x = np.zeros((1, G * len(fx["groups"])), np.float16)
    for gi, grp in enumerate(fx["groups"]):
        for k, v in grp["values"].items():
            x[0, gi * G + int(k)] = v
    q, s = quantize_a8(x)
    for gi, grp in enumerate(fx["groups"]):
        want = np.zeros(G, np.int8)
        for k, c in grp["codes"].items():
            want[int(k)] = c
        np.testing.assert_array_equal(q[0, gi * G:(gi + 1) * G], want)
        if "scale" in grp:
            assert s[0, gi] == np.float32(grp["scale"])
        else:
            assert abs(float(s[0, gi]) - grp["scale_approx"]) < 1e-9


def test_quantize_a8_decision_is_binary32():
    """The code decision is the binary32 quotient rounded half to even: at
    x = max / 2 the exact quotient is just below 63.5, its binary32 rounding is
    63.5, and the code is the even neighbour 64 (a binary64 decision gives 63)."""
    from fractions import Fraction
    a, x = np.float16(1.884765625), np.float16(0.9423828125)
    row = np.zeros((1, 128), np.float16)
    row[0, 0], row[0, 1] = a, x
    q, s = quantize_a8(row)
    exact = Fraction(float(x)) / Fraction(float(s[0, 0]))
    assert Fraction(63) < exact < Fraction(127, 2)
    assert np.float32(np.float32(x) / s[0, 0]) == np.float32(63.5)
    assert q[0, 1] == 64 and q[0, 0] == 127
    assert int(np.rint(float(x) / float(s[0, 0]))) == 63


def test_quantize_a8_bound_range_and_symmetry():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((5, 1024)) * np.repeat(rng.uniform(0.01, 20, (5, 8)), 128, axis=1)).astype(np.float16)
    q, s = quantize_a8(x)
    err = np.abs(x.astype(np.float64) - dequantize_a8(q, s))
    sf = np.repeat(s.astype(np.float64), 128, axis=1)
    # half a step, plus the float32 rounding of the quotient |x / s| <= 127 the
    # decision is taken on (a quotient just below a tie may round onto it)
    assert np.all(err <= sf / 2 + sf * 127 * 2.0 ** -24)
    assert np.all(np.max(np.abs(q.reshape(5, 8, 128)), axis=2) == 127)
    q2, s2 = quantize_a8(-x)
    np.testing.assert_array_equal(q2, -q)
    np.testing.assert_array_equal(s2, s)


def test_gemv_w4a8_brute_force():
    rng = np.random.default_rng(1)
    N, K, B = 3, 256, 2
    qw = rng.integers(-8, 8, (N, K)).astype(np.int8)
    sw = rng.uniform(0.001, 0.1, (N, 2)).astype(np.float16)
    x = rng.standard_normal((B, K)).astype(np.float16)
    qx, sx = quantize_a8(x)
    got = gemv_w4a8(qw, sw, qx, sx)
    for b in range(B):
        for n in range(N):
            acc = 0.0
            for g in range(2):
                dot = sum(int(qw[n, k]) * int(qx[b, k]) for k in range(128 * g, 128 * (g + 1)))
                acc += float(sw[n, g]) * float(sx[b, g]) * dot
            assert abs(got[b, n] - acc) <= 1e-12 * max(1.0, abs(acc))


def test_gemv_w4a8_equals_w4a16_when_activations_are_exact():
    """x = q * 2^-e with max |q| = 127 per group is recovered exactly by the
    quantiser, so W4A8 and W4A16 compute the same number."""
    rng = np.random.default_rng(2)
    N, K, B = 40, 512, 3
    w = rng.standard_normal((N, K)).astype(np.float32) * 0.02
    qw, sw = oracle.quantize_w4(w)
    qx = rng.integers(-127, 128, (B, K)).astype(np.int64)
    qx[:, ::128] = 127
    e = rng.integers(3, 9, (B, K // 128))
    x = (qx * np.repeat(np.power(2.0, -e), 128, axis=1)).astype(np.float16)
    q2, s2 = quantize_a8(x)
    np.testing.assert_array_equal(q2, qx)
    np.testing.assert_allclose(gemv_w4a8(qw, sw, q2, s2), oracle.gemv_w4a16(qw, sw, x), rtol=1e-13, atol=0)


def test_planted_per_row_scale_fails_the_bound():
    """A variant with one scale per row (not per group) must break the per-group
    rounding bound on rows whose groups differ in magnitude."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((2, 512)) * np.repeat([[0.01, 1, 10, 0.1]], 128, axis=1)).astype(np.float16)
    xf = x.astype(np.float32)
    s_row = (np.max(np.abs(xf), axis=1, keepdims=True) / np.float32(127)).astype(np.float32)
    q_row = np.clip(np.rint(xf / s_row), -127, 127)
    err_row = np.abs(x.astype(np.float64) - q_row * s_row)
    _, s = quantize_a8(x)
    half = np.repeat(s.astype(np.float64), 128, axis=1) / 2
    assert np.any(err_row > half * (1 + 1e-6))
