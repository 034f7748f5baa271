"""Pins for the oracle's whole decode step (CPU only).

The incremental decode step (cache, one token at a time) must agree with the
layer-major causal forward over the whole sequence, the paged cache must give
the same run as the contiguous one, and the run convention must leave the
cache at P + G - 1 positions."""
import numpy as np
import pytest

import synth
import oracle
from oracle.model import OracleModel, layer_decode, ContiguousKV

MICRO = synth.ModelShape("micro", 2, 256, 384, 4, 2, 64, 512)


@pytest.fixture(scope="module")
def micro():
    layers = [synth.layer_params(MICRO, i, seed=0) for i in range(MICRO.layers)]
    head = synth.head_params(MICRO, seed=0)
    return OracleModel.build(MICRO, layers, head)


def test_incremental_equals_causal_forward(micro):
    toks = synth.prompt_ids(21, MICRO.vocab, seed=2)
    cf = oracle.causal_forward(micro, toks)
    cache = ContiguousKV(MICRO.layers, MICRO.n_kv_heads, MICRO.head_dim)
    for p, t in enumerate(toks):
        r = oracle.decode_step(micro, [cache], [t], [p])
        for li in range(MICRO.layers):
            np.testing.assert_array_equal(r["layer_out"][li, 0], cf["layer_out"][li][p])
        np.testing.assert_allclose(r["logits"][0], cf["logits"][p], rtol=1e-12, atol=1e-12)


def test_paged_run_equals_contiguous_run(micro):
    prompt = synth.prompt_ids(16, MICRO.vocab, seed=2)
    a = oracle.generate(micro, prompt, 8)
    pt, total = synth.decode_page_tables(1, 2, seed=3, spare_pages=3)
    kv = oracle.PagedKVEmu(MICRO.layers, total, MICRO.n_kv_heads, MICRO.head_dim, pt)
    b = oracle.generate(micro, prompt, 8, paged=(kv, 0))
    np.testing.assert_array_equal(a["tokens"], b["tokens"])
    np.testing.assert_array_equal(a["logits"], b["logits"])
    # 16 + 8 - 1 = 23 positions written: page 0 full, page 1 has slots 0..6
    p1 = pt[0, 1]
    d = MICRO.head_dim
    kpage = kv.pool[:, 0, p1].reshape(MICRO.layers, MICRO.n_kv_heads, 16, d).astype(np.float32)
    vpage = kv.pool[:, 1, p1].reshape(MICRO.layers, MICRO.n_kv_heads, d, 16).astype(np.float32)
    assert not np.any(np.isnan(kpage[:, :, :7])) and np.all(np.isnan(kpage[:, :, 7:]))
    assert not np.any(np.isnan(vpage[..., :7])) and np.all(np.isnan(vpage[..., 7:]))


def test_run_convention_and_forcing(micro):
    prompt = synth.prompt_ids(5, MICRO.vocab, seed=4)
    r = oracle.generate(micro, prompt, 4)
    assert len(r["tokens"]) == 4 and r["layer_out"].shape[0] == 5 + 4 - 1
    # generated token i is the argmax of the logits at position P - 1 + i
    full = list(prompt) + list(r["tokens"][:-1])
    cf = oracle.causal_forward(micro, full)
    np.testing.assert_array_equal(np.argmax(cf["logits"][4:], axis=1), r["tokens"])
    assert np.all(r["margins"] >= 0)
    forced = (r["tokens"] + 1) % MICRO.vocab
    f = oracle.generate(micro, prompt, 4, forced=forced)
    assert f["tokens"][0] == r["tokens"][0]
    cf2 = oracle.causal_forward(micro, list(prompt) + list(forced[:-1]))
    np.testing.assert_array_equal(np.argmax(cf2["logits"][4:], axis=1), f["tokens"])


def test_layer_trace_boundaries_are_fp16(micro):
    cache = ContiguousKV(MICRO.layers, MICRO.n_kv_heads, MICRO.head_dim)
    tr = {}
    h = micro.head.embed[3]
    layer_decode(micro.layers[0], micro.dims, h, 0, lambda k, v: cache.append(0, 0, k, v),
                 lambda n: cache.get(0, n), tr)
    for key in ("x", "qkv", "q", "k", "v", "o", "h_mid", "x2", "a", "h_out"):
        assert tr[key].dtype == np.float16, key
    # at position 0 attention returns v of the only token, per GQA group
    o = tr["o"].reshape(MICRO.n_heads, MICRO.head_dim)
    for h_ in range(MICRO.n_heads):
        np.testing.assert_array_equal(o[h_], tr["v"][h_ // 2])
