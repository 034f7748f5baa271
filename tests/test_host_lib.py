"""CPU tests of libnq's host side: the library loads and exports every symbol
include/nq.h declares, the packer is bit-exact with the oracle's quantiser,
the packed bytes follow the documented layout, and bad arguments are refused
without side effects. No GPU call is made here."""
import ctypes
import json
import os

import numpy as np
import pytest

import oracle
import w4a16_gemv_paged_amd as nq

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _w(n, k, seed=0, std=0.02):
    return np.random.default_rng(seed).standard_normal((n, k), dtype=np.float32) * np.float32(std)


def test_library_exports_every_header_symbol():
    syms = nq.header_symbols()
    assert len(syms) >= 30
    L = ctypes.CDLL(nq.LIB_PATH)
    missing = [s for s in syms if not hasattr(L, s)]
    assert not missing, missing


def test_status_strings_and_version():
    assert nq.nq_status_str(0) == "NQ_OK"
    assert nq.nq_status_str(6) == "NQ_ERR_DEVICE_FAULT"
    assert nq.nq_layout_version() == 1


@pytest.mark.parametrize("n,k,kind,d", [(48, 512, nq.NQ_MAT_PLAIN, 0), (37, 256, nq.NQ_MAT_PLAIN, 0),
                                        (768, 512, nq.NQ_MAT_QKV, 64), (1536, 256, nq.NQ_MAT_QKV, 128),
                                        (64, 384, nq.NQ_MAT_GATE_UP, 0), (80, 128, nq.NQ_MAT_LM_HEAD, 0)])
def test_packer_matches_oracle_quantiser_bitwise(n, k, kind, d):
    w = _w(n, k, seed=n + k)
    packed, q, s = nq.nq_pack_weights(w, kind, d, want_codes=True)
    qo, so = oracle.quantize_w4(w)
    np.testing.assert_array_equal(q, qo)
    np.testing.assert_array_equal(s, so.view(np.uint16))
    q2, s2 = nq.nq_unpack_weights(packed, n, k, kind, d)
    np.testing.assert_array_equal(q2, qo)
    np.testing.assert_array_equal(s2, so.view(np.uint16))
    assert packed.size == nq.nq_packed_size(n, k) == ((n + 15) // 16 * 16) * (k // 2 + k // 64)


def test_packer_edge_values_match_oracle():
    """Ties, zeros, tiny (subnormal-scale) and large groups."""
    w = np.zeros((16, 768), np.float32)
    w[0, :128] = np.linspace(-7, 7, 128, dtype=np.float32)            # exact half-steps appear
    w[1, 128:256] = np.float32(3e-7)                                   # scale in fp16 subnormal range
    w[2, 256:384] = np.float32(-1e-9)                                  # scale rounds to 0 -> codes 0
    w[3, 384:512] = _w(1, 128, 5, std=1000.0)[0]                       # large
    w[4, 512:640] = np.float32(65504 * 7)                              # scale exactly at fp16 max
    w[5] = _w(1, 768, 6)[0]
    _, q, s = nq.nq_pack_weights(w, want_codes=True)
    qo, so = oracle.quantize_w4(w)
    np.testing.assert_array_equal(q, qo)
    np.testing.assert_array_equal(s, so.view(np.uint16))


def test_golden_hand_groups_through_packer():
    g = json.load(open(os.path.join(GOLD, "quant_hand.json")))
    G = g["group"]
    w = np.zeros((1, G * len(g["groups"])), np.float32)
    for gi, grp in enumerate(g["groups"]):
        for i, v in grp["values"].items():
            w[0, gi * G + int(i)] = np.float32(v)
    _, q, s = nq.nq_pack_weights(w, want_codes=True)
    for gi, grp in enumerate(g["groups"]):
        assert s[0, gi] == int(grp["scale_bits"], 16)
        for i, c in grp["codes"].items():
            assert q[0, gi * G + int(i)] == c


def _decode_documented_layout(packed, n_rows, K, kind, d):
    """Independent reading of the layout documented in include/nq.h."""
    T = (n_rows + 15) // 16
    G = K // 128
    codes = packed[: T * G * 1024]
    scales = packed[T * G * 1024:].view(np.uint16)
    q = np.zeros((n_rows, K), np.int8)
    s = np.zeros((n_rows, G), np.uint16)
    for t in range(T):
        for r in range(16):
            if kind == nq.NQ_MAT_QKV:
                hb, u = divmod(t, d // 16)
                n = hb * d + (8 * u + r if r < 8 else d // 2 + 8 * u + r - 8)
            elif kind == nq.NQ_MAT_GATE_UP:
                n = 8 * t + r if r < 8 else n_rows // 2 + 8 * t + r - 8
            else:
                n = 16 * t + r
            if n >= n_rows:
                continue
            for g in range(G):
                s[n, g] = scales[(t * G + g) * 16 + r]
                blk = (t * G + g) * 1024
                for c in range(64):
                    if c % 16 != r:
                        continue
                    k0 = 128 * g + 32 * (c // 16)
                    words = codes[blk + 16 * c: blk + 16 * c + 16].view("<u4")
                    for j in range(4):
                        for m in range(8):
                            k = k0 + 8 * j + (2 * m if m < 4 else 2 * (m - 4) + 1)
                            q[n, k] = ((int(words[j]) >> (4 * m)) & 15) - 8
    return q, s


@pytest.mark.parametrize("n,k,kind,d", [(24, 256, nq.NQ_MAT_PLAIN, 0), (128, 128, nq.NQ_MAT_QKV, 64),
                                        (32, 256, nq.NQ_MAT_GATE_UP, 0)])
def test_packed_bytes_follow_documented_layout(n, k, kind, d):
    w = _w(n, k, seed=11)
    packed = nq.nq_pack_weights(w, kind, d)
    q, s = _decode_documented_layout(packed, n, k, kind, d)
    qo, so = oracle.quantize_w4(w)
    np.testing.assert_array_equal(q, qo)
    np.testing.assert_array_equal(s, so.view(np.uint16))


def test_padding_rows_are_zero():
    w = _w(20, 128, seed=12)
    packed = nq.nq_pack_weights(w)
    T, G = 2, 1
    scales = packed[T * G * 1024:].view(np.uint16)
    assert np.all(scales[16 + 4:32] == 0)                  # tile 1 rows 4..15 are padding
    blk = packed[1024:2048]
    for c in range(64):
        if c % 16 >= 4:
            assert np.all(blk[16 * c:16 * c + 16] == 0x88)   # code 0 = nibble 8


def test_every_nibble_value_at_every_slot():
    """All 15 used codes (and -8) at every in-tile position round-trip."""
    q = np.zeros((16, 128), np.int8)
    for r in range(16):
        q[r] = (np.arange(128) + r) % 16 - 8
    q[:, 0] = 7                                              # one |q| = 7 per group fixes s
    w = (q.astype(np.float32) * np.float32(0.25))
    packed, q2, s2 = nq.nq_pack_weights(w, want_codes=True)
    # -8 * 0.25 = -2 would need |q| = 8 > 7: the quantiser maps it to -7 (clamped by rounding -8 * 7/8)
    qo, so = oracle.quantize_w4(w)
    np.testing.assert_array_equal(q2, qo)
    qu, su = nq.nq_unpack_weights(packed, 16, 128)
    np.testing.assert_array_equal(qu, qo)


@pytest.mark.parametrize("args", [
    dict(N=16, K=100, group=128, kind=0, d=0),     # K not a multiple of 128
    dict(N=16, K=128, group=64, kind=0, d=0),      # group != 128
    dict(N=0, K=128, group=128, kind=0, d=0),      # empty
    dict(N=100, K=128, group=128, kind=1, d=64),   # QKV with N % d != 0
    dict(N=24, K=128, group=128, kind=2, d=0),     # GATE_UP with N % 16 != 0
    dict(N=16, K=128, group=128, kind=9, d=0),     # unknown kind
])
def test_pack_rejects_bad_args(args):
    w = np.zeros((max(args["N"], 1), args["K"]), np.float32)
    out = np.full(1 << 16, 0xAB, np.uint8)
    st = nq.lib().nq_pack_weights(w.ctypes.data, args["N"], args["K"], args["group"], args["kind"], args["d"],
                                  out.ctypes.data, None, None)
    assert st == 1, nq.nq_last_error()
    assert nq.nq_last_error()
    assert np.all(out == 0xAB)


def test_pack_rejects_non_finite():
    w = _w(16, 128)
    w[3, 7] = np.nan
    with pytest.raises(nq.NQError) as e:
        nq.nq_pack_weights(w)
    assert e.value.status == 3


def test_config_check_and_sizes():
    import synth
    cfg = nq.NQConfig.from_shape(synth.QWEN7B, 8, 32768)
    nq.nq_config_check(cfg)
    geo = json.load(open(os.path.join(GOLD, "geometry.json")))
    # one page of one KV head, K or V: 16 tokens x 128 x fp16 = 4 KiB
    per_page = nq.nq_kv_pool_bytes(cfg, 1) // (cfg.layers * 2 * cfg.n_kv_heads)
    assert per_page == geo["page_bytes"] and cfg.page_tokens == geo["page_tokens"]
    assert cfg.layers == geo["layers_7b"] and cfg.group == geo["group"]
    bad = nq.NQConfig.from_shape(synth.QWEN7B, 8, 32768)
    bad.page_tokens = 32
    with pytest.raises(nq.NQError):
        nq.nq_config_check(bad)
    bad = nq.NQConfig.from_shape(synth.QWEN7B, 9, 32768)
    with pytest.raises(nq.NQError):
        nq.nq_config_check(bad)
    assert nq.nq_workspace_bytes(cfg, 1, 48) > 0
    assert nq.nq_workspace_bytes(cfg, 9, 48) == 0
    assert nq.nq_attn_workspace_bytes(cfg, 8, 2048) > 0
    # every decode-step batch covers the widest table; 64 sequences of it do not
    assert nq.nq_workspace_bytes(cfg, 8, 32768) > 0
    assert nq.nq_attn_workspace_bytes(cfg, 64, 4096) > 0
    assert nq.nq_attn_workspace_bytes(cfg, 64, 32768) == 0


def test_attention_split_plan_sizes():
    """The split plan behind nq_attn_workspace_bytes (partials are
    [B][n_heads][S][d] and [B][n_heads][S][2] floats, each 256-byte aligned):
    batch 1 takes fixed splits of 4 pages (one per wave) while they number at
    most 768 / n_kv; larger batches split by length over min(256 / n_kv,
    B * ceil(pages / 4)) workgroups per KV head, at least B + 1; beyond 1024
    workgroups of 512 pages, or 64 sequences, nothing."""
    import synth
    cfg = nq.NQConfig.from_shape(synth.QWEN7B, 8, 32768)
    nh, d = cfg.n_heads, cfg.head_dim
    a256 = lambda n: (n + 255) // 256 * 256

    def ws(batch, S):
        return a256(batch * nh * S * d * 4) + a256(batch * nh * S * 2 * 4)

    assert nq.nq_attn_workspace_bytes(cfg, 1, 4) == ws(1, 1)
    assert nq.nq_attn_workspace_bytes(cfg, 1, 52) == ws(1, 13)
    assert nq.nq_attn_workspace_bytes(cfg, 1, 768) == ws(1, 192)
    assert nq.nq_attn_workspace_bytes(cfg, 1, 769) == ws(1, 192)    # past 192 fixed splits: by length
    assert nq.nq_attn_workspace_bytes(cfg, 1, 2048) == ws(1, 192)
    assert nq.nq_attn_workspace_bytes(cfg, 2, 8) == ws(2, 4)        # 2 * ceil(8 / 4) splits
    assert nq.nq_attn_workspace_bytes(cfg, 8, 3) == ws(8, 1)        # tables of at most 4 pages: unsplit
    assert nq.nq_attn_workspace_bytes(cfg, 8, 2048) == ws(8, 64)     # one workgroup per CU over the 4 KV heads
    assert nq.nq_attn_workspace_bytes(cfg, 8, 32768) == ws(8, 520)  # 8 * 32768 / 512 + 8: no split over 512 pages
    assert nq.nq_attn_workspace_bytes(cfg, 65, 64) == 0
    assert nq.nq_attn_workspace_bytes(cfg, 64, 32768) == 0


def test_rope_table_matches_definition():
    import synth
    cfg = nq.NQConfig.from_shape(synth.QWEN7B, 1, 40000)
    tab = nq.nq_rope_table_fill(cfg)
    for pos in (0, 1, 511, 32767, 39999):
        phi = oracle.model.rope_angles(pos, 128, 1e6)
        np.testing.assert_allclose(tab[pos, :, 0], np.cos(phi).astype(np.float32), rtol=0, atol=1.2e-7)
        np.testing.assert_allclose(tab[pos, :, 1], np.sin(phi).astype(np.float32), rtol=0, atol=1.2e-7)


def test_model_state_errors_without_gpu():
    import synth
    cfg = nq.NQConfig.from_shape(synth.TINY, 1, 64)
    m = nq.nq_model_create(cfg)
    try:
        io = nq.NQStepIO(1, 4, 16, 16, 16, None, None, None, 0, None)
        st = nq.lib().nq_decode_step(m, None, ctypes.byref(io), None)
        assert st == 1  # null kv
        with pytest.raises(nq.NQError) as e:
            nq.nq_model_bind_layer(m, 5, nq.NQLayerPtrs())
        assert e.value.status == 3
    finally:
        nq.nq_model_destroy(m)


def test_step_mode_and_trace_arguments_without_gpu():
    """nq_model_set_step_mode takes the two modes only; nq_model_set_step_trace
    takes NULL (off) or a buffer of at least 256 * (layers + 1) * 16 uint64,
    8-byte aligned. The buffer is only recorded here, never touched."""
    import synth
    cfg = nq.NQConfig.from_shape(synth.TINY, 1, 64)
    m = nq.nq_model_create(cfg)
    try:
        for mode in (nq.NQ_STEP_AUTO, nq.NQ_STEP_KERNELS):
            nq.nq_model_set_step_mode(m, mode)
        with pytest.raises(nq.NQError) as e:
            nq.nq_model_set_step_mode(m, 7)
        assert e.value.status == 1
        need = 256 * (synth.TINY.layers + 1) * 16 * 8
        fake = 1 << 20
        nq.nq_model_set_step_trace(m, fake, need)
        nq.nq_model_set_step_trace(m, None, 0)
        for buf, nbytes in ((fake, need - 8), (fake + 4, need)):
            with pytest.raises(nq.NQError) as e:
                nq.nq_model_set_step_trace(m, buf, nbytes)
            assert e.value.status == 1
        assert nq.lib().nq_model_set_step_trace(None, None, 0) == 1
    finally:
        nq.nq_model_destroy(m)


def test_static_attention_refuses_beyond_its_scratch_without_gpu():
    """nq_attn_decode_static checks the split partials against its fixed
    library scratch (NQ_ATTN_SCRATCH_BYTES) before it looks up or touches any
    device memory: a batch and table width whose partials need more is
    refused with NQ_ERR_OUT_OF_RANGE, as are shapes beyond the kernels. The
    pointers are never dereferenced on these paths."""
    import synth
    cfg = nq.NQConfig.from_shape(synth.QWEN7B, 8, 32768)
    fake = 1 << 20                                   # 16-byte aligned, never used
    num_pages = 4096
    kv = nq.nq_kv_alloc(cfg, fake, nq.nq_kv_pool_bytes(cfg, num_pages), num_pages)
    try:
        assert nq.NQ_ATTN_SCRATCH_BYTES == 24 << 20
        assert nq.nq_attn_workspace_bytes(cfg, 8, 2048) <= nq.NQ_ATTN_SCRATCH_BYTES      # batch 8, 64 splits fit
        for batch, pages in ((32, 2048), (64, 512), (64, 32768)):
            need = nq.nq_attn_workspace_bytes(cfg, batch, pages)
            assert need == 0 or need > nq.NQ_ATTN_SCRATCH_BYTES
            with pytest.raises(nq.NQError) as e:
                nq.nq_attn_decode_static(kv, 0, batch, fake, fake, pages, fake, fake, stream=0)
            assert e.value.status == 3, (batch, pages)
        with pytest.raises(nq.NQError) as e:             # argument checks as for nq_attn_decode
            nq.nq_attn_decode_static(kv, 0, 1, fake + 8, fake, 4, fake, fake, stream=0)
        assert e.value.status == 1
        with pytest.raises(nq.NQError) as e:
            nq.nq_attn_decode_static(kv, 28, 1, fake, fake, 4, fake, fake, stream=0)
        assert e.value.status == 3
    finally:
        nq.nq_kv_free(kv)
