"""GPU parity of the INT8-activation (W4A8) variant against the oracle
(oracle/a8.py), called through the C ABI: the quantiser bit for bit (codes,
scale bits, code sums), the GEMV in both modes (separate quantise kernel, and
quantisation in the GEMV prologue) on every epilogue, and the two modes equal
to each other bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth
import w4a16_gemv_paged_amd as nq
from gpu_util import F16, dev, host, rel_inf, say, quantize_rows

pytestmark = pytest.mark.gpu

TOL_LAYER = 2e-3
# fp32 outputs: each group's exact integer sum times two scales (two fp32
# roundings), then at most 148 fp32 additions; the bound is ~(G + 2) 2^-24
# sqrt(G) relative for random signs, about 1e-4 at G = 148.
TOL_F32 = 1e-4
PERM = np.array([0, 4, 1, 5, 2, 6, 3, 7])   # stored byte p of each 8 holds input k0 + PERM[p]


def _decode_xq(buf, B, K):
    """Codes in natural order, scales and code sums from the device buffer."""
    raw = host(buf).view(np.uint8)
    G = K // 128
    stored = raw[:B * K].view(np.int8).reshape(B, K // 8, 8)
    codes = np.empty_like(stored)
    codes[:, :, PERM] = stored
    meta = raw[B * K:B * K + B * G * 8].view(np.int32).reshape(B, G, 2)
    return codes.reshape(B, K), meta[:, :, 0].view(np.float32), meta[:, :, 1]


def _activations(B, K, seed):
    """fp16 rows whose groups differ in magnitude, with a zero group and exact ties."""
    rng = np.random.default_rng(seed)
    mag = np.repeat(rng.uniform(0.01, 30, (B, K // 128)), 128, axis=1)
    x = (rng.standard_normal((B, K)) * mag).astype(F16)
    if K >= 256:
        x[:, 128:256] = 0
    x[0, :8] = [127, 2.5, -2.5, 3.5, 126.5, -127, 0.5, 1.5]      # group 0: scale 1, ties
    return x


@pytest.mark.parametrize("B,K", [(1, 128), (3, 384), (4, 3584), (2, 18944)])
def test_quantize_a8_bit_exact(B, K):
    say("a8 quantise", B, K)
    x = _activations(B, K, seed=K + B)
    buf = torch.zeros(nq.nq_a8_bytes(B, K), dtype=torch.uint8, device="cuda")
    nq.nq_quantize_a8(dev(x), B, K, buf)
    q, s, sm = _decode_xq(buf, B, K)
    qo, so = oracle.quantize_a8(x)
    np.testing.assert_array_equal(q, qo)
    np.testing.assert_array_equal(s.view(np.uint32), so.view(np.uint32))
    np.testing.assert_array_equal(sm, qo.reshape(B, K // 128, 128).astype(np.int64).sum(axis=2))


SHAPES = [(384, 768, nq.NQ_MAT_PLAIN), (3584, 4608, nq.NQ_MAT_PLAIN), (3584, 37888, nq.NQ_MAT_GATE_UP),
          (18944, 3584, nq.NQ_MAT_PLAIN)]


@pytest.mark.parametrize("K,N,kind", SHAPES)
@pytest.mark.parametrize("B", [1, 2, 4])
def test_gemv_w4a8_matches_oracle_both_modes(K, N, kind, B):
    say("w4a8 gemv", K, N, B)
    w = synth.gemv_weight(K, N, seed=3)
    qw, sw = quantize_rows(w)
    p = dev(nq.nq_pack_weights(w, kind))
    x = _activations(B, K, seed=7)
    qx, sx = oracle.quantize_a8(x)
    ref = oracle.gemv_w4a8(qw, sw, qx, sx)
    buf = torch.zeros(nq.nq_a8_bytes(B, K), dtype=torch.uint8, device="cuda")
    nq.nq_quantize_a8(dev(x), B, K, buf)
    xd = dev(x)
    outs = {}
    modes = ["quantised"] + (["fused"] if B * K * 3 <= 120 * 1024 else [])
    for mode in modes:
        xq = buf if mode == "quantised" else None
        if kind == nq.NQ_MAT_GATE_UP:
            I = N // 2
            y = torch.empty(B, I, dtype=torch.float16, device="cuda")
            nq.nq_gemv_w4a8(p, N, K, kind, 0, B, xd, xq, None, y, nq.NQ_EPI_SWIGLU_F16)
            got = host(y)
            assert rel_inf(got, oracle.swiglu(ref[:, :I], ref[:, I:])) < TOL_LAYER, mode
        else:
            y = torch.empty(B, N, dtype=torch.float32, device="cuda")
            nq.nq_gemv_w4a8(p, N, K, kind, 0, B, xd, xq, None, y, nq.NQ_EPI_STORE_F32)
            got = host(y)
            assert rel_inf(got, ref) < TOL_F32, mode
        outs[mode] = got
    if "fused" in outs:
        np.testing.assert_array_equal(outs["fused"].view(np.uint32 if outs["fused"].dtype == np.float32 else np.uint16),
                                      outs["quantised"].view(np.uint32 if outs["fused"].dtype == np.float32 else np.uint16))


@pytest.mark.parametrize("B", [1, 3])
def test_gemv_w4a8_bias_residual_f16(B):
    K, N = 3584, 3584
    w = synth.gemv_weight(K, N, seed=5)
    qw, sw = quantize_rows(w)
    p = dev(nq.nq_pack_weights(w))
    x = _activations(B, K, seed=9)
    qx, sx = oracle.quantize_a8(x)
    ref = oracle.gemv_w4a8(qw, sw, qx, sx)
    rng = np.random.default_rng(4)
    b = (0.05 * rng.standard_normal(N)).astype(F16)
    say("w4a8 bias", B)
    y = torch.empty(B, N, dtype=torch.float16, device="cuda")
    nq.nq_gemv_w4a8(p, N, K, 0, 0, B, dev(x), None, dev(b), y, nq.NQ_EPI_BIAS_F16)
    assert rel_inf(host(y), (ref + b.astype(np.float64)).astype(F16)) < TOL_LAYER
    r0 = (rng.standard_normal((B, N)) * 2).astype(F16)
    yr = dev(r0)
    say("w4a8 residual", B)
    nq.nq_gemv_w4a8(p, N, K, 0, 0, B, dev(x), None, None, yr, nq.NQ_EPI_RESIDUAL_F16)
    assert rel_inf(host(yr), (r0.astype(np.float64) + ref).astype(F16)) < TOL_LAYER


def test_w4a8_close_to_w4a16():
    """The activation quantisation error: W4A8 against the W4A16 oracle stays
    within the size of half an activation step (about 1/254 of the group
    maximum per input)."""
    K, N, B = 3584, 4608, 2
    w = synth.gemv_weight(K, N, seed=1)
    qw, sw = quantize_rows(w)
    x = synth.activations(B, K, seed=2)
    y = torch.empty(B, N, dtype=torch.float32, device="cuda")
    say("w4a8 vs w4a16")
    nq.nq_gemv_w4a8(dev(nq.nq_pack_weights(w)), N, K, 0, 0, B, dev(x), None, None, y, nq.NQ_EPI_STORE_F32)
    assert rel_inf(host(y), oracle.gemv_w4a16(qw, sw, x)) < 2e-2


def test_w4a8_rejects_bad_arguments():
    w = synth.gemv_weight(18944, 64, seed=9)
    p = dev(nq.nq_pack_weights(w))
    x = torch.zeros(5, 18944, dtype=torch.float16, device="cuda")
    y = torch.zeros(5, 64, dtype=torch.float32, device="cuda")
    with pytest.raises(nq.NQError) as e:
        nq.nq_gemv_w4a8(p, 64, 18944, 0, 0, 5, x, None, None, y, nq.NQ_EPI_STORE_F32)
    assert e.value.status == 1
    with pytest.raises(nq.NQError) as e:   # 4 rows of 18944 inputs do not fit LDS for in-kernel quantisation
        nq.nq_gemv_w4a8(p, 64, 18944, 0, 0, 4, x, None, None, y, nq.NQ_EPI_STORE_F32)
    assert e.value.status == 2
    with pytest.raises(nq.NQError) as e:
        nq.nq_quantize_a8(x, 5, 18944, y)
    assert e.value.status == 1
    assert torch.count_nonzero(y).item() == 0
