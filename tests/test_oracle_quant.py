"""Pins for the oracle's INT4 quantiser (CPU only).

Each check is tied to something other than the quantiser's own formula: the
half-step error bound, hand-derived codes for a worked group (golden fixture),
idempotence, range facts, and the independence of groups along K.
"""
import json
import os

import numpy as np
import pytest

from oracle import quantize_w4, dequantize_w4

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(n, k, seed=0, std=0.02):
    return (np.random.default_rng(seed).standard_normal((n, k), dtype=np.float32) * np.float32(std))


def test_hand_worked_groups():
    g = json.load(open(os.path.join(GOLD, "quant_hand.json")))
    G = g["group"]
    w = np.zeros((1, G * len(g["groups"])), np.float32)
    for gi, grp in enumerate(g["groups"]):
        for i, v in grp["values"].items():
            w[0, gi * G + int(i)] = np.float32(v)
    q, s = quantize_w4(w)
    for gi, grp in enumerate(g["groups"]):
        assert int(s[0, gi].view(np.uint16)) == int(grp["scale_bits"], 16)
        exp = np.zeros(G, np.int8)
        for i, c in grp["codes"].items():
            exp[int(i)] = c
        np.testing.assert_array_equal(q[0, gi * G:(gi + 1) * G], exp)


def test_error_bound_half_scale():
    w = _rand(64, 1024)
    q, s = quantize_w4(w)
    err = np.abs(w.astype(np.float64) - dequantize_w4(q, s))
    bound = np.repeat(s.astype(np.float64), 128, axis=1) / 2
    assert np.all(err <= bound)


def test_error_bound_heavy_tails_and_signs():
    rng = np.random.default_rng(7)
    w = rng.standard_cauchy((16, 512)).astype(np.float32)
    w[3] = -np.abs(w[3])                 # all-negative rows
    w[4, :128] = 1.0                     # constant group
    q, s = quantize_w4(w)
    err = np.abs(w.astype(np.float64) - dequantize_w4(q, s))
    assert np.all(err <= np.repeat(s.astype(np.float64), 128, axis=1) / 2)


def test_code_range_and_extreme_reached():
    w = _rand(32, 2048, seed=3)
    q, s = quantize_w4(w)
    assert q.min() >= -7 and q.max() <= 7
    amax = np.abs(q.reshape(32, -1, 128)).max(axis=2)
    assert np.all(amax[s != 0] == 7)


def test_idempotent():
    w = _rand(16, 768, seed=4)
    q, s = quantize_w4(w)
    w2 = dequantize_w4(q, s).astype(np.float32)
    q2, s2 = quantize_w4(w2)
    np.testing.assert_array_equal(q, q2)
    np.testing.assert_array_equal(s.view(np.uint16), s2.view(np.uint16))


def test_zero_group():
    w = _rand(2, 256, seed=5)
    w[1, 128:] = 0
    q, s = quantize_w4(w)
    assert s[1, 1] == 0 and np.all(q[1, 128:] == 0)


def test_dequant_exact_in_fp32():
    w = _rand(8, 512, seed=6)
    q, s = quantize_w4(w)
    f32 = q.astype(np.float32) * np.repeat(s.astype(np.float32), 128, axis=1)
    np.testing.assert_array_equal(f32.astype(np.float64), dequantize_w4(q, s))


def test_rows_concatenate():
    """Groups run along K, so quantising [A; B] equals stacking the parts."""
    a, b = _rand(12, 384, seed=8), _rand(20, 384, seed=9)
    qa, sa = quantize_w4(a)
    qb, sb = quantize_w4(b)
    qc, sc = quantize_w4(np.concatenate([a, b]))
    np.testing.assert_array_equal(qc, np.concatenate([qa, qb]))
    np.testing.assert_array_equal(sc.view(np.uint16), np.concatenate([sa, sb]).view(np.uint16))


def test_groups_are_along_k():
    """Scaling one 128-wide K block of a row changes only that group's scale."""
    w = _rand(4, 512, seed=10)
    q, s = quantize_w4(w)
    w2 = w.copy()
    w2[2, 256:384] *= np.float32(4)
    q2, s2 = quantize_w4(w2)
    changed = s2.view(np.uint16) != s.view(np.uint16)
    assert changed[2, 2] and changed.sum() == 1
    np.testing.assert_array_equal(q2, q)


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        quantize_w4(np.zeros((2, 100), np.float32))
    with pytest.raises(ValueError):
        quantize_w4(np.full((1, 128), np.inf, np.float32))


def test_planted_bad_divisor_is_caught(monkeypatch):
    """A quantiser that divides by 8 instead of 7 breaks the half-step bound
    (the code for +max clamps to 7); the bound test must notice."""
    w = _rand(8, 256, seed=11)
    a = np.abs(w.reshape(8, 2, 128)).max(axis=2)
    s = (a / np.float32(8)).astype(np.float16)
    q = np.clip(np.rint(w.reshape(8, 2, 128) / s.astype(np.float64)[:, :, None]), -8, 7)
    err = np.abs(w.reshape(8, 2, 128) - q * s.astype(np.float64)[:, :, None])
    assert np.any(err > s.astype(np.float64)[:, :, None] / 2)


def test_row_block_quantiser_equals_whole_matrix_call():
    """The threaded row-block helper used by the 7B tests gives exactly the
    oracle's codes and scales (groups never cross rows)."""
    from gpu_util import quantize_rows
    w = np.random.default_rng(11).standard_normal((77, 384)).astype(np.float32)
    q0, s0 = quantize_w4(w)
    q1, s1 = quantize_rows(w, chunk=10, workers=3)
    np.testing.assert_array_equal(q0, q1)
    np.testing.assert_array_equal(s0.view(np.uint16), s1.view(np.uint16))
