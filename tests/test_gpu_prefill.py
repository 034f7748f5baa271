"""GPU parity of the chunked prefill against the oracle, called through the C ABI:
the W4A16 GEMM (every epilogue, ragged row counts, odd group counts), the
causal paged prefill attention (tail pages, a prefix from an earlier chunk,
NaN-poisoned unwritten slots), and whole prompts through the tiny model
(teacher-forced layers, last-token logits and greedy token, chunk-size
invariance, continuation by decode steps)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.model import OracleModel, Dims, layer_causal, head_logits
import w4a16_gemv_paged_amd as nq
from w4a16_gemv_paged_amd.engine import DeviceModel, KVCache, Stepper, Prefill, run_greedy
from gpu_util import F16, dev, host, rel_inf, say, exact_case_weights

pytestmark = pytest.mark.gpu

TOL_LAYER, TOL_LOGITS, MARGIN = 2e-3, 5e-3, 1e-2
TOL_F32 = 1e-4     # fp32 outputs: see the note on biased codes in test_gpu_kernels.py


def _pk(w, kind=nq.NQ_MAT_PLAIN, d=0):
    return dev(nq.nq_pack_weights(w, kind, d))


# ------------------------------------------------------------------ GEMM

@pytest.mark.parametrize("k,n", [(384, 768), (640, 200), (3584, 4608), (18944, 3584)])
@pytest.mark.parametrize("m", [1, 5, 16, 17, 40, 100, 257])
def test_gemm_exact_arithmetic_bitwise(k, n, m):
    """x in {-2..2} and power-of-two scales make every partial sum exact in
    fp32, so each output must equal the oracle's bit for bit (N = 200 ends in a
    partial tile; K = 384 and 640 give odd group counts)."""
    say("gemm exact", k, n, m)
    w, q, s = exact_case_weights(n, k, seed=k + n)
    x = np.random.default_rng(m).integers(-2, 3, size=(m, k)).astype(F16)
    ref = oracle.gemv_w4a16(q, s, x).astype(F16)
    y = torch.empty(m, n, dtype=torch.float16, device="cuda")
    nq.nq_gemm_w4a16(_pk(w), n, k, 0, 0, m, dev(x), None, y, nq.NQ_EPI_STORE_F16)
    np.testing.assert_array_equal(host(y).view(np.uint16), ref.view(np.uint16))


@pytest.mark.parametrize("m", [3, 64, 200])
def test_gemm_random_every_epilogue(m):
    H, I = 512, 1408
    rng = np.random.default_rng(m)
    x = synth.activations(m, H, seed=11)
    # store f16 / f32 and bias
    w = synth.gemv_weight(H, 768, seed=4)
    b = (0.02 * rng.standard_normal(768)).astype(F16)
    qo, so = oracle.quantize_w4(w)
    p = _pk(w)
    say("gemm store/bias", m)
    y = torch.empty(m, 768, dtype=torch.float16, device="cuda")
    nq.nq_gemm_w4a16(p, 768, H, 0, 0, m, dev(x), None, y, nq.NQ_EPI_STORE_F16)
    ref = oracle.gemv_w4a16(qo, so, x)
    assert rel_inf(host(y), ref.astype(F16)) < TOL_LAYER
    yf = torch.empty(m, 768, dtype=torch.float32, device="cuda")
    nq.nq_gemm_w4a16(p, 768, H, 0, 0, m, dev(x), None, yf, nq.NQ_EPI_STORE_F32)
    assert rel_inf(host(yf), ref) < TOL_F32
    nq.nq_gemm_w4a16(p, 768, H, 0, 0, m, dev(x), dev(b), y, nq.NQ_EPI_BIAS_F16)
    assert rel_inf(host(y), oracle.gemv_w4a16(qo, so, x, b).astype(F16)) < TOL_LAYER
    # residual, in place, on a K = 1408 (11 groups) matrix
    w = synth.gemv_weight(I, H, seed=5)
    qo, so = oracle.quantize_w4(w)
    a = synth.activations(m, I, seed=6)
    r0 = (rng.standard_normal((m, H)) * 2).astype(F16)
    say("gemm residual", m)
    yr = dev(r0)
    nq.nq_gemm_w4a16(_pk(w), H, I, 0, 0, m, dev(a), None, yr, nq.NQ_EPI_RESIDUAL_F16)
    ref = (r0.astype(np.float64) + oracle.gemv_w4a16(qo, so, a)).astype(F16)
    assert rel_inf(host(yr), ref) < TOL_LAYER
    # SwiGLU on a fused [Wg; Wu]
    wgu = np.concatenate([synth.gemv_weight(H, I, seed=7), synth.gemv_weight(H, I, seed=8)])
    qo, so = oracle.quantize_w4(wgu)
    say("gemm swiglu", m)
    ya = torch.empty(m, I, dtype=torch.float16, device="cuda")
    nq.nq_gemm_w4a16(_pk(wgu, nq.NQ_MAT_GATE_UP), 2 * I, H, nq.NQ_MAT_GATE_UP, 0, m, dev(x), None, ya,
                     nq.NQ_EPI_SWIGLU_F16)
    gu = oracle.gemv_w4a16(qo, so, x)
    assert rel_inf(host(ya), oracle.swiglu(gu[:, :I], gu[:, I:])) < TOL_LAYER


def test_gemm_rows_are_independent_of_the_chunk():
    """Row m of a GEMM over M rows is bit-identical to the same row computed in
    a GEMM over fewer rows (the rows are separate MFMA columns)."""
    k, n = 3584, 4608
    w = synth.gemv_weight(k, n, seed=1)
    p = _pk(w)
    x = synth.activations(300, k, seed=2)
    outs = {}
    for m in (300, 37, 1):
        say("gemm chunk", m)
        y = torch.empty(m, n, dtype=torch.float16, device="cuda")
        nq.nq_gemm_w4a16(p, n, k, 0, 0, m, dev(x[:m]), None, y, nq.NQ_EPI_STORE_F16)
        outs[m] = host(y).view(np.uint16)
    np.testing.assert_array_equal(outs[37], outs[300][:37])
    np.testing.assert_array_equal(outs[1], outs[300][:1])


def test_gemm_rejects_bad_arguments():
    w = synth.gemv_weight(256, 32, seed=9)
    p = _pk(w)
    x = torch.zeros(8, 256, dtype=torch.float16, device="cuda")
    y = torch.zeros(8, 32, dtype=torch.float16, device="cuda")
    for kwargs in [dict(M=0), dict(M=4097), dict(epi=3), dict(K=200), dict(epi=1)]:
        a = dict(packed=p, N=32, K=256, kind=0, head_dim=0, M=8, x=x, bias=None, y=y, epi=0)
        a.update(kwargs)
        with pytest.raises(nq.NQError) as e:
            nq.nq_gemm_w4a16(*a.values())
        assert e.value.status == 1
    assert torch.count_nonzero(y).item() == 0


# ------------------------------------------------------------------ prefill attention

ATT7B = synth.ModelShape("att7b", 1, 3584, 18944, 28, 4, 128, 152064)
ATTTINY = synth.ModelShape("atttiny", 1, 512, 1408, 8, 2, 64, 4096)


def _prefill_attn_case(shape, start, n_q, seed=5):
    """A sequence whose positions 0..start+n_q-1 are cached in permuted pages
    (the rest of the pool NaN), and n_q queries at positions start.."""
    nkv, d, nh = shape.n_kv_heads, shape.head_dim, shape.n_heads
    total = start + n_q
    max_pages = (total + 15) // 16 + 1          # one table entry past the last page
    num_pages = max_pages + 3
    pt = synth.page_permutation(num_pages, seed)[:max_pages].reshape(1, -1)
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((total, nkv, d), dtype=np.float32).astype(F16)
    v = rng.standard_normal((total, nkv, d), dtype=np.float32).astype(F16)
    q = rng.standard_normal((n_q, nh, d), dtype=np.float32).astype(F16)
    emu = oracle.PagedKVEmu(1, num_pages, nkv, d, pt)
    for p in range(total):
        emu.append(0, 0, p, k[p], v[p])
    cfg = nq.NQConfig.from_shape(shape, 8, 32768)
    nbytes = nq.nq_kv_pool_bytes(cfg, num_pages)
    pool = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda")
    pool.view(torch.float16).copy_(dev(emu.pool.reshape(-1)))
    h = nq.nq_kv_alloc(cfg, pool, nbytes, num_pages)
    return dict(q=q, emu=emu, pt=pt, pool=pool, h=h, max_pages=max_pages)


def _prefill_attn_run(c, start, n_q, shape):
    out = torch.empty(n_q, shape.n_heads, shape.head_dim, dtype=torch.float16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    nq.nq_attn_prefill(c["h"], 0, n_q, start, dev(c["q"]), dev(c["pt"][0]), c["max_pages"], out, err)
    nq.nq_check_device_error(err)
    return host(out)


@pytest.mark.parametrize("start,n_q", [(0, 1), (0, 15), (0, 16), (0, 17), (0, 100), (37, 50), (512, 64),
                                       (4000, 33)])
@pytest.mark.parametrize("shape", [ATT7B, ATTTINY], ids=["28x4x128", "8x2x64"])
def test_prefill_attention_matches_oracle(start, n_q, shape):
    say("prefill attention", shape.name, start, n_q)
    c = _prefill_attn_case(shape, start, n_q)
    got = _prefill_attn_run(c, start, n_q, shape)
    K, V = c["emu"].get(0, 0, start + n_q)
    for i in range(n_q):
        p = start + i
        ref = oracle.attend(c["q"][i], K[:p + 1], V[:p + 1])
        assert rel_inf(got[i], ref) < TOL_LAYER, (i, p)
    if start == 0:   # the first query sees only itself: its output is v_0 exactly
        rep = shape.n_heads // shape.n_kv_heads
        np.testing.assert_array_equal(got[0], np.repeat(V[0], rep, 0))
    nq.nq_kv_free(c["h"])


def test_prefill_attention_rejects_positions_past_the_table():
    c = _prefill_attn_case(ATTTINY, 0, 20)
    out = torch.empty(40, 8, 64, dtype=torch.float16, device="cuda")
    with pytest.raises(nq.NQError) as e:
        nq.nq_attn_prefill(c["h"], 0, 40, c["max_pages"] * 16 - 20, dev(c["q"]), dev(c["pt"][0]), c["max_pages"],
                           out)
    assert e.value.status == 3
    nq.nq_kv_free(c["h"])


# ------------------------------------------------------------------ whole prompts (tiny model)

SHAPE = synth.TINY
PROMPT = 45            # 2 full chunks of 16 + a ragged 13


@pytest.fixture(scope="module")
def tiny():
    layers = [synth.layer_params(SHAPE, i, seed=0) for i in range(SHAPE.layers)]
    head = synth.head_params(SHAPE, seed=0)
    om = OracleModel.build(SHAPE, layers, head)
    say("build tiny device model")
    dm = DeviceModel(SHAPE, lambda i: layers[i], head, max_batch=8, max_pos=4096)
    yield om, dm
    dm.close()


def _prefill(dm, prompt, chunk, split=None, max_pages=None):
    """Prefill one sequence (in two calls at ``split`` if given); returns the
    layer outputs, last-token logits, next token, position and KV pool."""
    n = len(prompt)
    max_pages = max_pages or (n + 15) // 16 + 2
    pt, total = synth.decode_page_tables(1, max_pages, seed=3, spare_pages=3)
    kv = KVCache(dm, total, poison=True)
    pf = Prefill(dm, kv, chunk)
    cfg = dm.cfg
    lo = torch.empty(cfg.layers, n, cfg.hidden, dtype=torch.float16, device="cuda")
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    nt = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    po = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    row = dev(pt[0])
    if split is None:
        pf.run(prompt, row, 0, nt, po, logits, lo)
    else:
        lo1 = torch.empty(cfg.layers, split, cfg.hidden, dtype=torch.float16, device="cuda")
        lo2 = torch.empty(cfg.layers, n - split, cfg.hidden, dtype=torch.float16, device="cuda")
        pf.run(prompt[:split], row, 0, None, None, None, lo1)
        pf.run(prompt[split:], row, split, nt, po, logits, lo2)
        lo = torch.cat([lo1, lo2], dim=1)
    pf.check()
    out = dict(layer_out=host(lo), logits=host(logits), next=int(host(nt)[0]), pos=int(host(po)[0]),
               pool=host(kv.pool), pt=pt)
    kv.close()
    return out


@pytest.fixture(scope="module")
def tiny_prefill(tiny):
    om, dm = tiny
    prompt = synth.prompt_ids(PROMPT, SHAPE.vocab, seed=2)
    say("tiny prefill chunk 16")
    return prompt, _prefill(dm, prompt, 16)


def test_prefill_layers_teacher_forced(tiny, tiny_prefill):
    om, _ = tiny
    prompt, gpu = tiny_prefill
    d = om.dims
    for li, layer in enumerate(om.layers):
        x = om.head.embed[np.array(prompt)] if li == 0 else gpu["layer_out"][li - 1]
        ref = layer_causal(layer, d, x)
        errs = [rel_inf(gpu["layer_out"][li, t], ref[t]) for t in range(PROMPT)]
        assert max(errs) < TOL_LAYER, (li, int(np.argmax(errs)), max(errs))


def test_prefill_last_token_logits_and_greedy_token(tiny, tiny_prefill):
    om, _ = tiny
    prompt, gpu = tiny_prefill
    z = head_logits(om, gpu["layer_out"][-1, -1])
    assert rel_inf(gpu["logits"], z) < TOL_LOGITS
    top2 = np.sort(z)[-2:]
    if top2[1] - top2[0] > MARGIN:
        assert gpu["next"] == oracle.argmax_lowest(z)
    assert gpu["next"] == int(np.argmax(gpu["logits"]))       # the device argmax of its own logits
    assert gpu["pos"] == PROMPT


def test_prefill_writes_only_the_prompt_positions(tiny_prefill):
    """Every slot of the prompt's positions holds a finite value; every other
    slot of the pool keeps its NaN poison."""
    prompt, gpu = tiny_prefill
    pool = gpu["pool"].view(F16).reshape(SHAPE.layers, 2, -1, SHAPE.n_kv_heads, 16 * SHAPE.head_dim)
    written = np.zeros(pool.shape[2:4] + (16,), bool)
    for p in range(PROMPT):
        written[gpu["pt"][0, p // 16], :, p % 16] = True
    d = SHAPE.head_dim
    k = pool[:, 0].reshape(SHAPE.layers, -1, SHAPE.n_kv_heads, 16, d)
    v = pool[:, 1].reshape(SHAPE.layers, -1, SHAPE.n_kv_heads, d, 16).transpose(0, 1, 2, 4, 3)
    for arr in (k, v):
        fin = np.isfinite(arr).all(axis=-1)                      # [L, page, head, slot]
        assert np.array_equal(fin, np.broadcast_to(written, fin.shape))
        assert np.isnan(arr[:, ~written]).all()


@pytest.mark.parametrize("chunk", [1, 7, 45, 4096])
def test_prefill_chunk_size_does_not_change_a_bit(tiny, tiny_prefill, chunk):
    """Rows are independent GEMM columns and each query walks the same pages in
    the same order, so the chunking changes nothing, bit for bit."""
    om, dm = tiny
    prompt, ref = tiny_prefill
    say("tiny prefill chunk", chunk)
    got = _prefill(dm, prompt, chunk)
    np.testing.assert_array_equal(got["layer_out"].view(np.uint16), ref["layer_out"].view(np.uint16))
    np.testing.assert_array_equal(got["pool"], ref["pool"])
    assert got["next"] == ref["next"]


def test_prefill_in_two_calls_equals_one(tiny, tiny_prefill):
    """A second call continues at start_pos over the pages the first wrote."""
    om, dm = tiny
    prompt, ref = tiny_prefill
    say("tiny prefill split at 30")
    got = _prefill(dm, prompt, 16, split=30)
    np.testing.assert_array_equal(got["layer_out"].view(np.uint16), ref["layer_out"].view(np.uint16))
    np.testing.assert_array_equal(got["pool"], ref["pool"])
    np.testing.assert_array_equal(got["logits"].view(np.uint32), ref["logits"].view(np.uint32))


def test_prefill_rejects_positions_past_the_table_or_rope(tiny):
    om, dm = tiny
    kv = KVCache(dm, 8, poison=True)
    pf = Prefill(dm, kv, 16)
    row = dev(np.arange(2, dtype=np.int32))
    with pytest.raises(nq.NQError) as e:
        pf.run(list(range(40)), row, 0)               # 40 positions, 2 pages
    assert e.value.status == 3
    with pytest.raises(nq.NQError) as e:
        pf.run([1, 2], row, 4095)                    # max_pos is 4096
    assert e.value.status == 3
    kv.close()


def test_prefill_then_decode_matches_oracle(tiny):
    """Prompt by prefill, then 24 decode steps (graph replays), against the
    oracle's token-by-token run teacher-forced with the GPU's tokens."""
    om, dm = tiny
    prompt = synth.prompt_ids(PROMPT, SHAPE.vocab, seed=2)
    n_gen = 24
    max_pages = (PROMPT + n_gen + 15) // 16
    pt, total = synth.decode_page_tables(1, max_pages, seed=3, spare_pages=3)
    kv = KVCache(dm, total, poison=True)
    st = Stepper(dm, kv, pt, want_logits=True)
    stream = torch.cuda.Stream()
    say("tiny prefill + decode")
    with torch.cuda.stream(stream):
        gpu = run_greedy(st, [prompt], n_gen, use_graph=True, stream=stream, record_logits=True,
                         prefill_chunk=16)
    torch.cuda.synchronize()
    st.close()
    kv.close()
    orc = oracle.generate(om, prompt, n_gen, forced=gpu["tokens"][0])
    ok = orc["margins"] > MARGIN
    assert ok.sum() >= n_gen // 2
    np.testing.assert_array_equal(gpu["tokens"][0][ok], orc["tokens"][ok])
    errs = [rel_inf(gpu["logits"][i, 0], orc["logits"][i + 1]) for i in range(n_gen - 1)]
    assert max(errs) < TOL_LOGITS
