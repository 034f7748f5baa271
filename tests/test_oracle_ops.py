"""Pins for the oracle's elementary operations (CPU only): closed forms,
invariants and pure-Python brute force on tiny inputs."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import (softmax, rmsnorm, rope, attend, attend_splitk, swiglu,
                    argmax_lowest, ContiguousKV, PagedKVEmu, gemv_w4a16,
                    quantize_w4)

GOLD = os.path.join(os.path.dirname(__file__), "golden")
F16 = np.float16


# ---------------------------------------------------------------- softmax

def test_softmax_textbook_values():
    g = json.load(open(os.path.join(GOLD, "softmax_textbook.json")))
    np.testing.assert_allclose(softmax(g["x"]), g["p"], rtol=0, atol=1e-15)


def test_softmax_sums_to_one_and_is_shift_invariant():
    x = np.random.default_rng(0).standard_normal((50, 300)) * 30
    p = softmax(x)
    assert np.all(np.abs(p.sum(-1) - 1) < 1e-12)
    np.testing.assert_allclose(softmax(x + 1e3), p, rtol=1e-12, atol=1e-300)


def test_softmax_stable_for_large_inputs():
    p = softmax([1000.0, 1000.0])
    np.testing.assert_allclose(p, [0.5, 0.5], rtol=0, atol=0)


# ---------------------------------------------------------------- rmsnorm

def test_rmsnorm_constant_vector_closed_form():
    c, eps = 0.75, 1e-6
    x = np.full(512, c, F16)
    g = np.full(512, 1.5, F16)
    exp = F16(c / math.sqrt(c * c + eps) * 1.5)
    assert np.all(rmsnorm(x, g, eps) == exp)


def test_rmsnorm_scale_invariant():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(256).astype(F16)
    g = (1 + 0.02 * rng.standard_normal(256)).astype(F16)
    a = rmsnorm(x, g, 1e-6).astype(np.float64)
    b = rmsnorm((x.astype(np.float32) * 4).astype(F16), g, 1e-6).astype(np.float64)
    np.testing.assert_array_equal(a, b)          # x4 is exact in fp16 and cancels exactly


def test_rmsnorm_unit_rms():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(4096).astype(F16)
    y = rmsnorm(x, np.ones(4096, F16), 1e-6).astype(np.float64)
    assert abs(math.sqrt(np.mean(y * y)) - 1) < 2e-4


# ---------------------------------------------------------------- RoPE

def test_rope_pos0_identity():
    x = np.random.default_rng(3).standard_normal((4, 128)).astype(F16)
    np.testing.assert_array_equal(rope(x, 0, 1e6), x)


def test_rope_pairing_sign_and_frequencies_closed_form():
    """d = 6, theta = 1e6: inverse frequencies are 1e6^(-2i/6) = 1, 1e-2, 1e-4
    exactly. At pos 100 the angles are 100, 1, 0.01. The unit vector e_1 turns
    into cos(1) e_1 + sin(1) e_4 (rotate-half pairs (i, i + d/2)); e_4 turns
    into -sin(1) e_1 + cos(1) e_4."""
    e1 = np.zeros((1, 6), F16); e1[0, 1] = 1
    e4 = np.zeros((1, 6), F16); e4[0, 4] = 1
    y1 = rope(e1, 100, 1e6).astype(np.float64)[0]
    y4 = rope(e4, 100, 1e6).astype(np.float64)[0]
    c1, s1 = math.cos(1.0), math.sin(1.0)
    np.testing.assert_allclose(y1, [0, F16(c1), 0, 0, F16(s1), 0], atol=0)
    np.testing.assert_allclose(y4, [0, -F16(s1), 0, 0, F16(c1), 0], atol=0)
    e2 = np.zeros((1, 6), F16); e2[0, 2] = 1
    y2 = rope(e2, 100, 1e6).astype(np.float64)[0]
    np.testing.assert_allclose(y2, [0, 0, F16(math.cos(0.01)), 0, 0, F16(math.sin(0.01))], atol=0)


def test_rope_preserves_norm():
    x = np.random.default_rng(4).standard_normal((8, 128)).astype(F16)
    y = rope(x, 12345, 1e6).astype(np.float64)
    n0 = np.linalg.norm(x.astype(np.float64), axis=-1)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), n0, rtol=2e-3)


def test_rope_relative_position():
    """<R_m q, R_n k> = <R_{m-n} q, k>, up to the fp16 rounding of outputs."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 128)).astype(F16)
    k = rng.standard_normal((1, 128)).astype(F16)
    for m, n in [(7, 3), (1000, 10), (32767, 32000)]:
        a = float(rope(q, m, 1e6).astype(np.float64)[0] @ rope(k, n, 1e6).astype(np.float64)[0])
        b = float(rope(q, m - n, 1e6).astype(np.float64)[0] @ k.astype(np.float64)[0])
        assert abs(a - b) < 0.05, (m, n, a, b)


# ---------------------------------------------------------------- attention

def _brute(q, K, V):
    """Pure-Python scaled dot-product attention for one query head."""
    d = len(q)
    s = [sum(q[i] * k[i] for i in range(d)) / math.sqrt(d) for k in K]
    m = max(s)
    e = [math.exp(v - m) for v in s]
    z = sum(e)
    return [sum(e[t] / z * V[t][i] for t in range(len(K))) for i in range(d)]


@pytest.mark.parametrize("L", [1, 2, 5, 8])
def test_attend_brute_force(L):
    rng = np.random.default_rng(L)
    q = rng.standard_normal((2, 4)).astype(F16)
    K = rng.standard_normal((L, 1, 4)).astype(F16)
    V = rng.standard_normal((L, 1, 4)).astype(F16)
    o = attend(q, K, V)
    for h in range(2):
        ref = _brute([float(v) for v in q[h]], [[float(v) for v in K[t, 0]] for t in range(L)],
                     [[float(v) for v in V[t, 0]] for t in range(L)])
        np.testing.assert_allclose(o[h], ref, rtol=0, atol=1e-12)


def test_attend_single_token_returns_v0():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((8, 64)).astype(F16)
    K = rng.standard_normal((1, 2, 64)).astype(F16)
    V = rng.standard_normal((1, 2, 64)).astype(F16)
    o = attend(q, K, V)
    for h in range(8):
        np.testing.assert_array_equal(o[h], V[0, h // 4].astype(np.float64))


def test_attend_zero_query_is_mean_of_v():
    rng = np.random.default_rng(10)
    K = rng.standard_normal((37, 1, 16)).astype(F16)
    V = rng.standard_normal((37, 1, 16)).astype(F16)
    o = attend(np.zeros((1, 16), F16), K, V)
    np.testing.assert_allclose(o[0], V[:, 0].astype(np.float64).mean(0), atol=1e-14)


def test_attend_scale_is_inverse_sqrt_d():
    """Two keys whose dot products with q differ by sqrt(d) * ln 3 give weights
    1/4 and 3/4 only with the 1/sqrt(d) scale."""
    d = 16
    q = np.zeros((1, d), F16); q[0, 0] = 1
    K = np.zeros((2, 1, d), F16); K[1, 0, 0] = F16(math.sqrt(d) * math.log(3))
    V = np.zeros((2, 1, d), F16); V[1, 0, 0] = 1
    o = attend(q, K, V)
    k1 = float(K[1, 0, 0]) / math.sqrt(d)
    np.testing.assert_allclose(o[0, 0], math.exp(k1) / (1 + math.exp(k1)), atol=1e-15)
    assert abs(o[0, 0] - 0.75) < 2e-3


def test_attend_gqa_grouping_consecutive():
    """Each KV head carries a constant, distinct V: query head h must return
    the V of KV head h // (nh / nkv)."""
    rng = np.random.default_rng(11)
    nh, nkv, d, L = 28, 4, 8, 5
    q = rng.standard_normal((nh, d)).astype(F16)
    K = rng.standard_normal((L, nkv, d)).astype(F16)
    V = np.zeros((L, nkv, d), F16)
    for j in range(nkv):
        V[:, j, :] = j + 1
    o = attend(q, K, V)
    for h in range(nh):
        np.testing.assert_allclose(o[h], np.full(d, h // 7 + 1), atol=1e-13)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 40])
def test_splitk_combine_matches(splits):
    rng = np.random.default_rng(12)
    q = rng.standard_normal((8, 64)).astype(F16)
    K = (rng.standard_normal((37, 2, 64)) * 3).astype(F16)
    V = rng.standard_normal((37, 2, 64)).astype(F16)
    np.testing.assert_allclose(attend_splitk(q, K, V, splits), attend(q, K, V), rtol=0, atol=1e-13)


def test_paged_equals_contiguous_bitwise_with_tail_pages():
    rng = np.random.default_rng(13)
    layers, nkv, d = 2, 2, 64
    pt = rng.permutation(12).astype(np.int32).reshape(2, 6)
    paged = PagedKVEmu(layers, 12, nkv, d, pt)
    cont = [ContiguousKV(layers, nkv, d) for _ in range(2)]
    for b, L in enumerate([47, 81]):            # 2 pages + 15, 5 pages + 1
        for p in range(L):
            for li in range(layers):
                k = rng.standard_normal((nkv, d)).astype(F16)
                v = rng.standard_normal((nkv, d)).astype(F16)
                paged.append(li, b, p, k, v)
                cont[b].append(li, p, k, v)
        for li in range(layers):
            kp, vp = paged.get(li, b, L)
            kc, vc = cont[b].get(li, L)
            np.testing.assert_array_equal(kp.view(np.uint16), kc.view(np.uint16))
            np.testing.assert_array_equal(vp.view(np.uint16), vc.view(np.uint16))
            q = rng.standard_normal((8, d)).astype(F16)
            np.testing.assert_array_equal(attend(q, kp, vp), attend(q, kc, vc))


def test_paged_location_rule():
    pt = np.array([[5, 2, 7]], np.int32)
    kv = PagedKVEmu(1, 8, 1, 4, pt)
    assert kv.locate(0, 0) == (5, 0)
    assert kv.locate(0, 15) == (5, 15)
    assert kv.locate(0, 16) == (2, 0)
    assert kv.locate(0, 47) == (7, 15)
    with pytest.raises(IndexError):
        kv.locate(0, 48)
    bad = PagedKVEmu(1, 8, 1, 4, np.array([[9]], np.int32))
    with pytest.raises(IndexError):
        bad.locate(0, 0)


def test_paged_attention_helper_matches_contiguous():
    rng = np.random.default_rng(14)
    B, nh, nkv, d = 2, 4, 2, 32
    lens = [19, 33]
    pt = np.array([[3, 0, -1], [4, 1, 2]], np.int32)
    # the documented page layout written out by hand: K token-major, V dim-major
    pool = np.full((2, 6, nkv, 16 * d), np.nan, F16)
    ks = [rng.standard_normal((L, nkv, d)).astype(F16) for L in lens]
    vs = [rng.standard_normal((L, nkv, d)).astype(F16) for L in lens]
    for b in range(B):
        for p in range(lens[b]):
            page, slot = pt[b, p // 16], p % 16
            for h in range(nkv):
                for e in range(d):
                    pool[0, page, h, slot * d + e] = ks[b][p, h, e]
                    pool[1, page, h, e * 16 + slot] = vs[b][p, h, e]
    q = rng.standard_normal((B, nh, d)).astype(F16)
    out = oracle.paged_attention(q, pool, pt, lens)
    for b in range(B):
        np.testing.assert_array_equal(out[b], attend(q[b], ks[b], vs[b]))


# ---------------------------------------------------------------- SwiGLU / argmax / GEMV

def test_swiglu_closed_forms():
    assert float(swiglu(1.0, 1.0)) == float(F16(0.7310585786300049))   # 1 / (1 + e^-1)
    assert float(swiglu(0.0, 123.0)) == 0.0
    x = np.linspace(-6, 6, 97)
    diff = swiglu(x, 1.0).astype(np.float64) - swiglu(-x, 1.0).astype(np.float64)
    np.testing.assert_allclose(diff, x, atol=8e-3)           # silu(x) - silu(-x) = x


def test_argmax_lowest_on_ties_and_nan():
    assert argmax_lowest([1.0, 3.0, 3.0, 2.0]) == 1
    assert argmax_lowest([-1.0]) == 0
    with pytest.raises(ValueError):
        argmax_lowest([0.0, np.nan])


def test_gemv_brute_force():
    rng = np.random.default_rng(15)
    w = (rng.standard_normal((3, 256)) * 0.02).astype(np.float32)
    q, s = quantize_w4(w)
    x = rng.standard_normal((2, 256)).astype(F16)
    b = rng.standard_normal(3).astype(F16)
    y = gemv_w4a16(q, s, x, b)
    for bi in range(2):
        for n in range(3):
            acc = 0.0
            for k in range(256):
                acc += int(q[n, k]) * float(s[n, k // 128]) * float(x[bi, k])
            assert abs(y[bi, n] - (acc + float(b[n]))) < 1e-12
