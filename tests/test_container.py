"""Packed-weight container (host only, no GPU): a tiny model written with
write_container reads back byte for byte, and damaged or foreign files are
refused (magic, header checksum, layout version, truncation, tensor bytes)."""
import os
import struct

import numpy as np
import pytest

import synth
import w4a16_gemv_paged_amd as nq
from w4a16_gemv_paged_amd.engine import write_container, _pack_layer, LAYER_TENSORS

SHAPE = synth.TINY


def fnv1a(data: bytes) -> int:
    """FNV-1a 64 (offset basis 0xcbf29ce484222325, prime 0x100000001b3)."""
    h = 0xcbf29ce484222325
    for b in data:
        h = ((h ^ b) * 0x100000001b3) & 0xFFFFFFFFFFFFFFFF
    return h


@pytest.fixture(scope="module")
def tiny_file(tmp_path_factory):
    path = str(tmp_path_factory.mktemp("c") / "tiny.nqpack")
    head = synth.head_params(SHAPE, seed=0)
    write_container(path, SHAPE, lambda l: synth.layer_params(SHAPE, l, seed=0), head)
    return path, head


def test_round_trip(tiny_file):
    path, head = tiny_file
    c = nq.nq_container_open(path)
    try:
        assert nq.nq_container_count(c) == 7 * SHAPE.layers + 3
        cfg = nq.nq_container_config(c)
        assert (cfg.layers, cfg.hidden, cfg.intermediate, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.vocab) == \
               (SHAPE.layers, SHAPE.hidden, SHAPE.intermediate, SHAPE.n_heads, SHAPE.n_kv_heads, SHAPE.head_dim,
                SHAPE.vocab)
        assert cfg.rope_theta == np.float32(SHAPE.rope_theta) and cfg.rms_eps == np.float32(SHAPE.rms_eps)
        for li in range(SHAPE.layers):
            t = _pack_layer(synth.layer_params(SHAPE, li, seed=0), SHAPE.head_dim)
            for name in LAYER_TENSORS:
                d, view = nq.nq_container_tensor(c, f"layer.{li}.{name}")
                np.testing.assert_array_equal(view, np.ascontiguousarray(t[name]).view(np.uint8).reshape(-1))
        d, view = nq.nq_container_tensor(c, "lm_head")
        np.testing.assert_array_equal(view, nq.nq_pack_weights(head["lm_head"], nq.NQ_MAT_LM_HEAD))
        assert d.role == nq.NQ_TENSOR_PACKED and d.mat_kind == nq.NQ_MAT_LM_HEAD and d.N == SHAPE.vocab
        d, view = nq.nq_container_tensor(c, "embed")
        np.testing.assert_array_equal(view.view(np.float16).reshape(SHAPE.vocab, SHAPE.hidden), head["embed"])
        d0, _ = nq.nq_container_tensor_at(c, 0)
        assert d0.name == b"layer.0.qkv"
        nq.nq_container_verify(c)
        with pytest.raises(nq.NQError) as e:
            nq.nq_container_tensor(c, "no.such.tensor")
        assert e.value.status == 3
    finally:
        nq.nq_container_close(c)


def _damaged(path, tmp_path, edit):
    raw = bytearray(open(path, "rb").read())
    raw = edit(raw)
    out = str(tmp_path / "damaged.nqpack")
    open(out, "wb").write(bytes(raw))
    return out


def _refused(path):
    with pytest.raises(nq.NQError) as e:
        nq.nq_container_open(path)
    assert e.value.status == 7
    return str(e.value)


def test_bad_magic_checksum_version_and_truncation_are_refused(tiny_file, tmp_path):
    path, _ = tiny_file

    def magic(r):
        r[0] ^= 0xFF
        return r

    def cfg_byte(r):
        r[20] ^= 1            # inside the stored configuration: the header checksum no longer matches
        return r

    def layout(r):
        r[12:16] = struct.pack("<I", 99)   # layout version, with the header checksum recomputed
        off = 88   # magic, 2 versions, 11 config words, count, reserved, 4 padding bytes, 2 x 8-byte table fields
        r[off:off + 8] = struct.pack("<Q", fnv1a(bytes(r[:off])))
        return r

    def truncate(r):
        return r[:len(r) - 96]

    assert "magic" in _refused(_damaged(path, tmp_path, magic))
    assert "checksum" in _refused(_damaged(path, tmp_path, cfg_byte))
    assert "layout" in _refused(_damaged(path, tmp_path, layout))
    assert "table" in _refused(_damaged(path, tmp_path, truncate))
    assert _refused(str(tmp_path / "missing.nqpack"))


def test_damaged_tensor_fails_verify(tiny_file, tmp_path):
    path, _ = tiny_file
    c = nq.nq_container_open(path)
    _, view = nq.nq_container_tensor(c, "layer.1.down")
    off = view.ctypes.data - nq.nq_container_tensor_at(c, 0)[1].ctypes.data + 4096
    nq.nq_container_close(c)

    def flip(r):
        r[off + 100] ^= 0x10
        return r

    c = nq.nq_container_open(_damaged(path, tmp_path, flip))
    try:
        with pytest.raises(nq.NQError) as e:
            nq.nq_container_verify(c)
        assert e.value.status == 7 and "layer.1.down" in str(e.value)
    finally:
        nq.nq_container_close(c)


def test_writer_rejects_bad_tensors(tmp_path):
    cfg = nq.NQConfig.from_shape(SHAPE, 1, 1)
    w = nq.nq_container_create(str(tmp_path / "w.nqpack"), cfg, 2)
    g = np.ones(512, np.float16)
    nq.nq_container_add(w, "a", nq.NQ_TENSOR_F16, 512, 1, g)
    for args, code in [(("a", nq.NQ_TENSOR_F16, 512, 1, g), 1),          # duplicate name
                       (("b", nq.NQ_TENSOR_F16, 513, 1, g), 1),          # size does not match the shape
                       (("b", nq.NQ_TENSOR_PACKED, 16, 100, g), 1),      # K not a multiple of 128
                       (("x" * 48, nq.NQ_TENSOR_F16, 512, 1, g), 1)]:    # name too long
        with pytest.raises(nq.NQError) as e:
            nq.nq_container_add(w, *args)
        assert e.value.status == code
    with pytest.raises(nq.NQError) as e:                                 # one tensor short of the count
        nq.nq_container_finish(w)
    assert e.value.status == 5
