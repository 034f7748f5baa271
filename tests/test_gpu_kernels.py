"""GPU parity tests of libnq's kernels against the oracle (called through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import w4a16_gemv_paged_amd as nq
from gpu_util import F16, dev, host, rel_inf, say, exact_case_weights

pytestmark = pytest.mark.gpu

TOL_LAYER = 2e-3   # per-layer-output bar (infinity-norm relative)
# fp32 outputs (no fp16 rounding at the end): the kernels accumulate the biased
# fp16 codes (1024 + n, 16 * (72 + q)) against pre-scaled activations and
# subtract the bias products in fp32, so a group's partial sum carries terms up
# to ~1032 |x| before they cancel; with the unit roundoff 2^-24 that puts the
# relative error at a few 1e-5 (measured 1.4e-5 at K = 512), against ~1e-7
# for exact codes. The bar keeps a margin over that.
TOL_F32 = 1e-4


def _packed_dev(w, kind=nq.NQ_MAT_PLAIN, d=0):
    return dev(nq.nq_pack_weights(w, kind, d))


# ------------------------------------------------------------------ unpack

@pytest.mark.parametrize("n,k,kind,d", [(48, 512, 0, 0), (37, 384, 0, 0), (768, 512, 1, 64),
                                        (4608, 3584, 1, 128), (2816, 512, 2, 0), (4096, 512, 3, 0)])
def test_device_unpack_bit_exact(n, k, kind, d):
    say("unpack", n, k, kind)
    w = synth.normal_matrix(0, (n, k, 99), n, k)
    qo, so = oracle.quantize_w4(w)
    p = _packed_dev(w, kind, d)
    q = torch.empty(n, k, dtype=torch.int8, device="cuda")
    s = torch.empty(n, k // 128, dtype=torch.int16, device="cuda")
    nq.nq_unpack_weights_dev(p, n, k, kind, d, q, s)
    np.testing.assert_array_equal(host(q), qo)
    np.testing.assert_array_equal(host(s).view(np.uint16), so.view(np.uint16))


# ------------------------------------------------------------------ GEMV

GEMV_7B = synth.GEMV_SHAPES_7B


@pytest.mark.parametrize("k,n", [(512, 768), (1408, 512), (512, 4096)] + GEMV_7B)
@pytest.mark.parametrize("batch", [1, 4, 8])
def test_gemv_exact_arithmetic_bitwise(k, n, batch):
    """x in {-2..2} and power-of-two scales make every partial sum exact in
    fp32, so the GPU must equal the oracle bit for bit whatever the order."""
    say("gemv exact", k, n, batch)
    w, q, s = exact_case_weights(n, k, seed=k + n)
    rng = np.random.default_rng(batch)
    x = rng.integers(-2, 3, size=(batch, k)).astype(F16)
    ref = oracle.gemv_w4a16(q, s, x).astype(F16)
    y = torch.empty(batch, n, dtype=torch.float16, device="cuda")
    nq.nq_gemv_w4a16(_packed_dev(w), n, k, 0, 0, batch, dev(x), None, 1e-6, None, y, nq.NQ_EPI_STORE_F16)
    np.testing.assert_array_equal(host(y).view(np.uint16), ref.view(np.uint16))


@pytest.mark.parametrize("k", [640, 1280, 1408, 2560])
@pytest.mark.parametrize("batch", [1, 4])
def test_gemv_ring_windows_bitwise(k, batch):
    """Wide matrices (1024 tiles: one K-slice per tile from batch 4, two at
    batch 1) whose waves take 5, 10, 11 or 20 groups at batch 4 and 2-3, 5,
    5-6 or 10 at batch 1: a lone last window of the weight ring, exactly one
    or two full windows, full windows and a tail. Exact arithmetic as above,
    so bit for bit."""
    n = 16384
    say("gemv ring windows", k, n, batch)
    w, q, s = exact_case_weights(n, k, seed=k + 7)
    rng = np.random.default_rng(batch + 10)
    x = rng.integers(-2, 3, size=(batch, k)).astype(F16)
    ref = oracle.gemv_w4a16(q, s, x).astype(F16)
    y = torch.empty(batch, n, dtype=torch.float16, device="cuda")
    nq.nq_gemv_w4a16(_packed_dev(w), n, k, 0, 0, batch, dev(x), None, 1e-6, None, y, nq.NQ_EPI_STORE_F16)
    np.testing.assert_array_equal(host(y).view(np.uint16), ref.view(np.uint16))


def test_gemv_one_hot_columns():
    """x = e_k returns column k: y[n] = fp16(q[n,k] * s[n, k // 128])."""
    k, n = 1024, 64
    w = synth.normal_matrix(0, (7,), n, k)
    qo, so = oracle.quantize_w4(w)
    cols = [0, 1, 127, 128, 500, 1023]
    x = np.zeros((len(cols), k), F16)
    for i, c in enumerate(cols):
        x[i, c] = 1
    p = _packed_dev(w)
    for i0 in range(0, len(cols), 4):
        xb = x[i0:i0 + 4]
        say("gemv one-hot", i0)
        y = torch.empty(len(xb), n, dtype=torch.float16, device="cuda")
        nq.nq_gemv_w4a16(p, n, k, 0, 0, len(xb), dev(xb), None, 1e-6, None, y, nq.NQ_EPI_STORE_F16)
        for j, c in enumerate(cols[i0:i0 + 4]):
            ref = (qo[:, c].astype(np.float64) * so[:, c // 128].astype(np.float64)).astype(F16)
            np.testing.assert_array_equal(host(y)[j], ref)


@pytest.mark.parametrize("k,n", [(512, 768), (3584, 4608), (18944, 3584)])
@pytest.mark.parametrize("batch", [1, 2, 3, 5, 8])
def test_gemv_random_store_f16_and_f32(k, n, batch):
    say("gemv random", k, n, batch)
    w = synth.gemv_weight(k, n, seed=0)
    qo, so = oracle.quantize_w4(w)
    x = synth.activations(batch, k, seed=1)
    ref = oracle.gemv_w4a16(qo, so, x)
    p = _packed_dev(w)
    y = torch.empty(batch, n, dtype=torch.float16, device="cuda")
    nq.nq_gemv_w4a16(p, n, k, 0, 0, batch, dev(x), None, 1e-6, None, y, nq.NQ_EPI_STORE_F16)
    assert rel_inf(host(y), ref.astype(F16)) < TOL_LAYER
    yf = torch.empty(batch, n, dtype=torch.float32, device="cuda")
    nq.nq_gemv_w4a16(p, n, k, 0, 0, batch, dev(x), None, 1e-6, None, yf, nq.NQ_EPI_STORE_F32)
    assert rel_inf(host(yf), ref) < TOL_F32


@pytest.mark.parametrize("batch", [1, 4])
def test_gemv_norm_bias_residual_swiglu(batch):
    """Each fused epilogue and the RMSNorm prologue against the oracle."""
    H, I = 512, 1408
    rng = np.random.default_rng(3)
    h = (rng.standard_normal((batch, H)) * 3).astype(F16)
    g = (1 + 0.02 * rng.standard_normal(H)).astype(F16)
    xh = oracle.rmsnorm(h, g, 1e-6)
    # bias
    w = synth.gemv_weight(H, 768, seed=4)
    b = (0.02 * rng.standard_normal(768)).astype(F16)
    qo, so = oracle.quantize_w4(w)
    say("gemv bias+norm", batch)
    y = torch.empty(batch, 768, dtype=torch.float16, device="cuda")
    nq.nq_gemv_w4a16(_packed_dev(w), 768, H, 0, 0, batch, dev(h), dev(g), 1e-6, dev(b), y, nq.NQ_EPI_BIAS_F16)
    assert rel_inf(host(y), oracle.gemv_w4a16(qo, so, xh, b).astype(F16)) < TOL_LAYER
    # residual (in place)
    w = synth.gemv_weight(I, H, seed=5)
    qo, so = oracle.quantize_w4(w)
    a = synth.activations(batch, I, seed=6)
    r0 = (rng.standard_normal((batch, H)) * 2).astype(F16)
    say("gemv residual", batch)
    yr = dev(r0)
    nq.nq_gemv_w4a16(_packed_dev(w), H, I, 0, 0, batch, dev(a), None, 1e-6, None, yr, nq.NQ_EPI_RESIDUAL_F16)
    ref = (r0.astype(np.float64) + oracle.gemv_w4a16(qo, so, a)).astype(F16)
    assert rel_inf(host(yr), ref) < TOL_LAYER
    # SwiGLU on a fused [Wg; Wu]
    wg, wu = synth.gemv_weight(H, I, seed=7), synth.gemv_weight(H, I, seed=8)
    wgu = np.concatenate([wg, wu])
    qo, so = oracle.quantize_w4(wgu)
    say("gemv swiglu", batch)
    ya = torch.empty(batch, I, dtype=torch.float16, device="cuda")
    nq.nq_gemv_w4a16(_packed_dev(wgu, nq.NQ_MAT_GATE_UP), 2 * I, H, nq.NQ_MAT_GATE_UP, 0, batch, dev(h), dev(g),
                     1e-6, None, ya, nq.NQ_EPI_SWIGLU_F16)
    gu = oracle.gemv_w4a16(qo, so, xh)
    ref = oracle.swiglu(gu[:, :I], gu[:, I:])
    assert rel_inf(host(ya), ref) < TOL_LAYER


@pytest.mark.parametrize("batch", [4, 5, 8])
def test_gemv_norm_gain_multi_chunk(batch):
    """The RMSNorm prologue when the staged activation rows and the gain (B + 1
    rows of K = 18944) exceed the LDS budget and are staged in several chunks:
    each chunk reloads the gain, the sums of squares accumulate across chunks,
    and the last chunk is not a multiple of the K-slices."""
    K, N = 18944, 512
    rng = np.random.default_rng(31)
    h = (rng.standard_normal((batch, K)) * 3).astype(F16)
    g = (1 + 0.02 * rng.standard_normal(K)).astype(F16)
    w = synth.gemv_weight(K, N, seed=32)
    b = (0.02 * rng.standard_normal(N)).astype(F16)
    qo, so = oracle.quantize_w4(w)
    xh = oracle.rmsnorm(h, g, 1e-6)
    say("gemv norm gain multi-chunk", batch)
    y = torch.empty(batch, N, dtype=torch.float16, device="cuda")
    nq.nq_gemv_w4a16(_packed_dev(w), N, K, 0, 0, batch, dev(h), dev(g), 1e-6, dev(b), y, nq.NQ_EPI_BIAS_F16)
    assert rel_inf(host(y), oracle.gemv_w4a16(qo, so, xh, b).astype(F16)) < TOL_LAYER


@pytest.mark.parametrize("batch", [2, 3, 5, 6, 7])
def test_gemv_norm_prologue_odd_batches(batch):
    """The RMSNorm prologue at batch sizes that are not a power of two: the pass
    gives each thread one batch row (the row count rounded up to a power of two,
    the threads of the extra rows idle) and reduces every row's sum of squares
    at once. Checked in the per-tile GEMV and in the streaming GEMV (at least 16
    row tiles per workgroup, the LM head's kernel), against the oracle."""
    rng = np.random.default_rng(40 + batch)
    for k, n in ((3584, 768), (512, 65536)):
        h = (rng.standard_normal((batch, k)) * 3).astype(F16)
        g = (1 + 0.02 * rng.standard_normal(k)).astype(F16)
        w = synth.gemv_weight(k, n, seed=41)
        qo, so = oracle.quantize_w4(w)
        xh = oracle.rmsnorm(h, g, 1e-6)
        say("gemv norm prologue", batch, k, n)
        y = torch.empty(batch, n, dtype=torch.float32, device="cuda")
        nq.nq_gemv_w4a16(_packed_dev(w), n, k, 0, 0, batch, dev(h), dev(g), 1e-6, None, y, nq.NQ_EPI_STORE_F32)
        assert rel_inf(host(y), oracle.gemv_w4a16(qo, so, xh)) < TOL_LAYER


def test_gemv_rejects_bad_arguments():
    w = synth.gemv_weight(256, 32, seed=9)
    p = _packed_dev(w)
    x = torch.zeros(9, 256, dtype=torch.float16, device="cuda")
    y = torch.zeros(9, 32, dtype=torch.float16, device="cuda")
    for kwargs, code in [(dict(batch=9), 1), (dict(batch=0), 1), (dict(epi=3), 1), (dict(K=200), 1)]:
        a = dict(packed=p, N=32, K=256, kind=0, head_dim=0, batch=1, x=x, norm_gain=None, eps=1e-6, bias=None,
                 y=y, epi=0)
        a.update(kwargs)
        with pytest.raises(nq.NQError) as e:
            nq.nq_gemv_w4a16(*a.values())
        assert e.value.status == code
    assert torch.count_nonzero(y).item() == 0


# ------------------------------------------------------------------ KV pool

def _kv_handle(shape, num_pages, poison=True):
    cfg = nq.NQConfig.from_shape(shape, 8, 32768)
    nbytes = nq.nq_kv_pool_bytes(cfg, num_pages)
    pool = torch.full((nbytes // 2,), 0x7E00 if poison else 0, dtype=torch.int16, device="cuda")
    h = nq.nq_kv_alloc(cfg, pool, nbytes, num_pages)
    return cfg, pool, h


def test_kv_append_bit_exact_against_paged_emulation():
    shape = synth.ModelShape("kv", 2, 512, 1408, 8, 2, 64, 4096)
    B, max_pages, P = 3, 4, 14
    pt, _ = synth.decode_page_tables(B, max_pages, seed=3, spare_pages=2)
    cfg, pool, h = _kv_handle(shape, P)
    emu = oracle.PagedKVEmu(2, P, 2, 64, pt)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ptd = dev(pt)
    for layer in (0, 1):
        for step, positions in enumerate([[0, 5, 17], [1, 15, 16], [47, 33, 63]]):
            # values encode (layer, b, position, head, dim) exactly as fp16 integers
            k = np.zeros((B, 2, 64), F16)
            v = np.zeros((B, 2, 64), F16)
            for b in range(B):
                for hh in range(2):
                    k[b, hh] = (layer * 1000 + b * 300 + positions[b] * 4 + hh) % 2048 + np.arange(64) / 64
                    v[b, hh] = -k[b, hh]
                emu.append(layer, b, positions[b], k[b], v[b])
            say("kv append", layer, step)
            nq.nq_kv_append(h, layer, B, ptd, max_pages, dev(np.array(positions, np.int32)), dev(k), dev(v), err)
    got = host(pool).view(F16).reshape(emu.pool.shape)
    np.testing.assert_array_equal(got.view(np.uint16), emu.pool.view(np.uint16))
    nq.nq_check_device_error(err)
    nq.nq_kv_free(h)


def test_kv_append_flags_bad_page_without_writing():
    shape = synth.ModelShape("kv", 1, 512, 1408, 8, 2, 64, 4096)
    cfg, pool, h = _kv_handle(shape, 4)
    pt = np.array([[2, 9]], np.int32)         # page id 9 is outside the 4-page pool
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    k = np.ones((1, 2, 64), F16)
    say("kv append bad page")
    nq.nq_kv_append(h, 0, 1, dev(pt), 2, dev(np.array([20], np.int32)), dev(k), dev(k), err)
    with pytest.raises(nq.NQError) as e:
        nq.nq_check_device_error(err)
    assert e.value.status == 6
    assert np.all(host(pool) == 0x7E00)
    say("kv append position beyond table")
    nq.nq_kv_append(h, 0, 1, dev(pt), 2, dev(np.array([32], np.int32)), dev(k), dev(k), err)
    with pytest.raises(nq.NQError):
        nq.nq_check_device_error(err)
    nq.nq_kv_free(h)


# ------------------------------------------------------------------ attention

def _attn_setup(shape, lens, seed=5, perm_seed=3):
    inp = synth.attention_inputs(len(lens), shape.n_heads, shape.n_kv_heads, shape.head_dim, lens,
                                 seed=seed, perm_seed=perm_seed)
    cfg, pool, h = _kv_handle(shape, inp["num_pages"])
    emu = oracle.PagedKVEmu(1, inp["num_pages"], shape.n_kv_heads, shape.head_dim, inp["page_table"])
    for b, L in enumerate(lens):
        for p in range(L):
            emu.append(0, b, p, inp["k_tok"][b][p], inp["v_tok"][b][p])
    pool_np = emu.pool
    layer_elems = pool_np[0, 0].size
    flat = pool.view(torch.float16)
    flat[: 2 * layer_elems].copy_(dev(pool_np[0].reshape(-1)))
    return inp, cfg, pool, h, pool_np


def _attn_run(cfg, h, inp, batch):
    max_pages = inp["page_table"].shape[1]
    wsb = nq.nq_attn_workspace_bytes(cfg, batch, max_pages)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty(batch, cfg.n_heads, cfg.head_dim, dtype=torch.float16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    nq.nq_attn_decode(h, 0, batch, dev(inp["q"]), dev(inp["page_table"]), max_pages, dev(inp["lens"]), out, ws,
                      wsb, err)
    nq.nq_check_device_error(err)
    return host(out)


ATT7B = synth.ModelShape("att7b", 1, 3584, 18944, 28, 4, 128, 152064)
ATTTINY = synth.ModelShape("atttiny", 1, 512, 1408, 8, 2, 64, 4096)


@pytest.mark.parametrize("lens", [[1], [15], [16], [17], [47], [511], [4097], [3, 40, 16, 100, 1, 250, 33, 64]])
@pytest.mark.parametrize("shape", [ATT7B, ATTTINY], ids=["28x4x128", "8x2x64"])
def test_attention_matches_oracle_tail_pages(lens, shape):
    say("attention", shape.name, lens)
    inp, cfg, pool, h, pool_np = _attn_setup(shape, lens)
    got = _attn_run(cfg, h, inp, len(lens))
    ref = oracle.paged_attention(inp["q"], pool_np[0], inp["page_table"], inp["lens"])
    for b in range(len(lens)):
        assert rel_inf(got[b], ref[b]) < TOL_LAYER, (b, lens[b])
    if lens == [1]:
        np.testing.assert_array_equal(got[0], np.repeat(inp["v_tok"][0][0], shape.n_heads // shape.n_kv_heads, 0))
    nq.nq_kv_free(h)


def test_attention_independent_of_page_placement():
    """Two different permutations of the same logical cache give bit-identical output."""
    lens = [700, 33, 129]
    a_inp, cfg, pool_a, ha, _ = _attn_setup(ATT7B, lens, perm_seed=3)
    b_inp, cfg2, pool_b, hb, _ = _attn_setup(ATT7B, lens, perm_seed=11)   # both pools stay alive
    assert not np.array_equal(a_inp["page_table"], b_inp["page_table"])
    say("attention placement")
    ga = _attn_run(cfg, ha, a_inp, 3)
    gb = _attn_run(cfg2, hb, b_inp, 3)
    np.testing.assert_array_equal(ga.view(np.uint16), gb.view(np.uint16))
    nq.nq_kv_free(ha)
    nq.nq_kv_free(hb)


def test_attention_split_merge_reuses_workspace():
    """Split partials merged with the log-sum-exp rule: three calls on one
    workspace give bit-identical outputs. The workspace starts as NaN bit
    patterns: an empty split's output rows (a zero length, and the pages past
    each short sequence) are never written and must never be used."""
    lens = [3, 700, 0, 2000]
    inp, cfg, pool, h, pool_np = _attn_setup(ATT7B, lens, seed=8)
    batch, max_pages = len(lens), inp["page_table"].shape[1]
    wsb = nq.nq_attn_workspace_bytes(cfg, batch, max_pages)
    ws = torch.full((wsb,), 0xFF, dtype=torch.uint8, device="cuda")
    live = [b for b, L in enumerate(lens) if L > 0]
    ref = dict(zip(live, oracle.paged_attention(inp["q"][live], pool_np[0], inp["page_table"][live],
                                                inp["lens"][live])))
    outs = []
    for call in range(3):
        say("attention split reuse", call)
        out = torch.empty(batch, cfg.n_heads, cfg.head_dim, dtype=torch.float16, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        nq.nq_attn_decode(h, 0, batch, dev(inp["q"]), dev(inp["page_table"]), max_pages, dev(inp["lens"]), out,
                          ws, wsb, err)
        nq.nq_check_device_error(err)
        outs.append(host(out))
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(outs[0][b] == 0)
        else:
            assert rel_inf(outs[0][b], ref[b]) < TOL_LAYER, (b, L)
    for o in outs[1:]:
        np.testing.assert_array_equal(o.view(np.uint16), outs[0].view(np.uint16))
    nq.nq_kv_free(h)


@pytest.mark.parametrize("lens", [[511, 4097, 32767]])
def test_attention_full_context_lengths(lens):
    """The attention sweep lengths of the 7B shape (tails of 15, 1 and 15 tokens)."""
    for L in lens:
        say("attention full", L)
        inp, cfg, pool, h, pool_np = _attn_setup(ATT7B, [L], seed=5)
        got = _attn_run(cfg, h, inp, 1)
        ref = oracle.paged_attention(inp["q"], pool_np[0], inp["page_table"], inp["lens"])
        assert rel_inf(got[0], ref[0]) < TOL_LAYER
        nq.nq_kv_free(h)
        del pool


def test_attention_batch8_ragged_full_range():
    lens = synth.ragged_lengths(8, 1, 32767, seed=6)
    say("attention ragged", lens.tolist())
    inp, cfg, pool, h, pool_np = _attn_setup(ATT7B, lens.tolist())
    got = _attn_run(cfg, h, inp, 8)
    ref = oracle.paged_attention(inp["q"], pool_np[0], inp["page_table"], inp["lens"])
    for b in range(8):
        assert rel_inf(got[b], ref[b]) < TOL_LAYER, (b, lens[b])
    nq.nq_kv_free(h)


@pytest.mark.parametrize("batch,hi,seed", [(3, 3000, 21), (16, 1200, 22), (64, 300, 23)])
def test_attention_split_by_length_large_batch(batch, hi, seed):
    """Batches above one split every sequence's pages by the current lengths
    over a fixed grid: ragged lengths (zeros included) up to 64 sequences,
    against the oracle; a zero length gives a zero row."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, hi, size=batch)
    lens[0], lens[-1] = 0, hi                      # an empty sequence and the longest one
    shape = ATTTINY if batch > 8 else ATT7B
    say("attention by length", batch, int(lens.sum()))
    inp, cfg, pool, h, pool_np = _attn_setup(shape, lens.tolist(), seed=seed)
    got = _attn_run(cfg, h, inp, batch)
    live = [b for b in range(batch) if lens[b] > 0]
    ref = oracle.paged_attention(inp["q"][live], pool_np[0], inp["page_table"][live], inp["lens"][live])
    for i, b in enumerate(live):
        assert rel_inf(got[b], ref[i]) < TOL_LAYER, (b, lens[b])
    assert np.all(got[0] == 0)
    nq.nq_kv_free(h)


def test_attention_rejects_batch_beyond_split_grid():
    """64 sequences of 32768-page tables need more than 1024 workgroups of 512
    pages per KV head: refused before any launch, and the workspace size is 0."""
    cfg, pool, h = _kv_handle(ATTTINY, 8)
    assert nq.nq_attn_workspace_bytes(cfg, 64, 32768) == 0
    q = torch.zeros(64, cfg.n_heads, cfg.head_dim, dtype=torch.float16, device="cuda")
    pt = torch.zeros(64, 32768, dtype=torch.int32, device="cuda")
    lens = torch.ones(64, dtype=torch.int32, device="cuda")
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    say("attention oversized batch refused")
    with pytest.raises(nq.NQError) as e:
        nq.nq_attn_decode(h, 0, 64, q, pt, 32768, lens, torch.empty_like(q), ws, ws.numel(), None)
    assert e.value.status == 3  # NQ_ERR_OUT_OF_RANGE
    nq.nq_kv_free(h)


def test_attention_bad_page_id_sets_flag():
    lens = [40]
    inp, cfg, pool, h, _ = _attn_setup(ATTTINY, lens)
    inp["page_table"] = inp["page_table"].copy()
    inp["page_table"][0, 1] = inp["num_pages"] + 5
    say("attention bad page")
    with pytest.raises(nq.NQError) as e:
        _attn_run(cfg, h, inp, 1)
    assert e.value.status == 6
    nq.nq_kv_free(h)
