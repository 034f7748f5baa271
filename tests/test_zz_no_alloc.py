"""nq_attn_decode_static (split-K paged decode attention with its partials in
the library's own device scratch, no workspace, no allocation) against
nq_attn_decode on the same inputs, and against the oracle.

Three calls in a row on one GPU: a ragged batch of 3 (split by length, 192
splits per KV head), then a smaller batch-1 call (11 fixed splits) that
leaves the first call's partials in the scratch beyond its own, then the first
call again. Every output must equal nq_attn_decode's bit for bit (the same
kernels on the same split plan) and be within the per-layer tolerance of the
oracle's fp64 attention."""
import numpy as np
import pytest
import torch

import oracle
import synth
import w4a16_gemv_paged_amd as nq
from gpu_util import F16, dev, host, rel_inf, say

pytestmark = pytest.mark.gpu

SHAPE = synth.ModelShape("att7b", 1, 3584, 18944, 28, 4, 128, 152064)
TOL = 2e-3


def _problem(lens, seed):
    """Inputs of one call: q, the page table and lengths, and a device pool
    holding one layer's pages (NaN in every slot no token was written to)."""
    inp = synth.attention_inputs(len(lens), SHAPE.n_heads, SHAPE.n_kv_heads, SHAPE.head_dim, lens, seed=seed)
    cfg = nq.NQConfig.from_shape(SHAPE, 8, 32768)
    emu = oracle.PagedKVEmu(1, inp["num_pages"], SHAPE.n_kv_heads, SHAPE.head_dim, inp["page_table"])
    for b, L in enumerate(lens):
        for p in range(L):
            emu.append(0, b, p, inp["k_tok"][b][p], inp["v_tok"][b][p])
    nbytes = nq.nq_kv_pool_bytes(cfg, inp["num_pages"])
    pool = torch.full((nbytes // 2,), 0x7E00, dtype=torch.int16, device="cuda")
    pool.view(torch.float16)[: emu.pool[0].size].copy_(dev(emu.pool[0].reshape(-1)))
    kv = nq.nq_kv_alloc(cfg, pool, nbytes, inp["num_pages"])
    ref = oracle.paged_attention(inp["q"], emu.pool[0], inp["page_table"], inp["lens"])
    return dict(inp=inp, cfg=cfg, pool=pool, kv=kv, ref=ref, q=dev(inp["q"]), pt=dev(inp["page_table"]),
                lens=dev(inp["lens"]))


def _with_workspace(pr):
    inp, cfg = pr["inp"], pr["cfg"]
    B, max_pages = inp["page_table"].shape
    wsb = nq.nq_attn_workspace_bytes(cfg, B, max_pages)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty(B, cfg.n_heads, cfg.head_dim, dtype=torch.float16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    nq.nq_attn_decode(pr["kv"], 0, B, pr["q"], pr["pt"], max_pages, pr["lens"], out, ws, wsb, err)
    nq.nq_check_device_error(err)
    return host(out)


def _static(pr):
    inp, cfg = pr["inp"], pr["cfg"]
    B, max_pages = inp["page_table"].shape
    assert nq.nq_attn_workspace_bytes(cfg, B, max_pages) <= nq.NQ_ATTN_SCRATCH_BYTES
    out = torch.full((B, cfg.n_heads, cfg.head_dim), float("nan"), dtype=torch.float16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    nq.nq_attn_decode_static(pr["kv"], 0, B, pr["q"], pr["pt"], max_pages, pr["lens"], out, err)
    nq.nq_check_device_error(err)
    return host(out)


def test_static_attention_matches_workspace_attention_on_consecutive_calls():
    big = _problem([511, 4097, 300], seed=5)
    small = _problem([700], seed=6)
    try:
        say("static attention: batch 3, lengths 511/4097/300")
        a1 = _static(big)
        say("static attention: batch 1, length 700 (second call, smaller)")
        a2 = _static(small)
        say("static attention: batch 3 again")
        a3 = _static(big)
        say("workspace attention on the same inputs")
        w1 = _with_workspace(big)
        w2 = _with_workspace(small)
        np.testing.assert_array_equal(a1.view(np.uint16), w1.view(np.uint16))
        np.testing.assert_array_equal(a2.view(np.uint16), w2.view(np.uint16))
        np.testing.assert_array_equal(a3.view(np.uint16), a1.view(np.uint16))
        for got, pr in ((a1, big), (a2, small)):
            assert np.all(np.isfinite(got.astype(np.float32)))
            for b in range(got.shape[0]):
                assert rel_inf(got[b], pr["ref"][b]) < TOL, (b, rel_inf(got[b], pr["ref"][b]))
    finally:
        nq.nq_kv_free(big["kv"])
        nq.nq_kv_free(small["kv"])
