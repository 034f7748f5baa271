"""Python binding of libnq, the MI355X W4A16 paged greedy-decode library.

Thin ctypes layer over the C ABI declared in ``include/nq.h``: every function
here has the name of the C entry point it calls and only marshals arguments
(device pointers from torch tensors, host arrays from NumPy, streams from
torch). All computation happens in libnq (host packer in C++, everything on
the device in HIP kernels). There is no fallback: if libnq.so is not built,
every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

__all__ = [
    "NQError", "NQConfig", "NQLayerPtrs", "NQStepIO", "lib", "LIB_PATH",
    "NQ_MAT_PLAIN", "NQ_MAT_QKV", "NQ_MAT_GATE_UP", "NQ_MAT_LM_HEAD",
    "NQ_EPI_STORE_F16", "NQ_EPI_BIAS_F16", "NQ_EPI_RESIDUAL_F16", "NQ_EPI_SWIGLU_F16", "NQ_EPI_STORE_F32",
    "nq_status_str", "nq_last_error", "nq_layout_version", "nq_packed_size", "nq_pack_weights",
    "nq_unpack_weights", "nq_unpack_weights_dev", "nq_gemv_w4a16", "nq_config_check",
    "nq_kv_pool_bytes", "nq_kv_alloc", "nq_kv_append", "nq_kv_free", "nq_attn_workspace_bytes",
    "nq_attn_decode", "nq_attn_decode_static", "NQ_ATTN_SCRATCH_BYTES", "nq_model_create",
    "nq_model_set_step_mode", "nq_step_kernels", "nq_model_set_step_trace", "NQ_STEP_AUTO", "NQ_STEP_KERNELS", "nq_model_bind_layer", "nq_model_bind_head",
    "nq_rope_table_bytes", "nq_rope_table_fill", "nq_model_bind_rope", "nq_workspace_bytes",
    "nq_model_bind_workspace", "nq_model_destroy", "nq_decode_step", "nq_graph_capture",
    "nq_graph_launch", "nq_graph_kernel_count", "nq_graph_destroy", "nq_check_device_error",
    "nq_gemm_w4a16", "nq_attn_prefill", "NQPrefillIO", "nq_prefill_workspace_bytes", "nq_prefill",
    "nq_a8_bytes", "nq_quantize_a8", "nq_gemv_w4a8",
    "NQTensorDesc", "NQ_TENSOR_PACKED", "NQ_TENSOR_F16", "nq_container_create", "nq_container_add",
    "nq_container_finish", "nq_container_open", "nq_container_config", "nq_container_count",
    "nq_container_tensor", "nq_container_tensor_at", "nq_container_verify", "nq_container_close",
    "header_symbols",
]

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libnq.so")
HEADER = os.path.join(os.path.dirname(PKG_DIR), "include", "nq.h")

NQ_OK = 0
NQ_MAT_PLAIN, NQ_MAT_QKV, NQ_MAT_GATE_UP, NQ_MAT_LM_HEAD = 0, 1, 2, 3
NQ_EPI_STORE_F16, NQ_EPI_BIAS_F16, NQ_EPI_RESIDUAL_F16, NQ_EPI_SWIGLU_F16, NQ_EPI_STORE_F32 = 0, 1, 2, 3, 4
STATUS_NAMES = {0: "NQ_OK", 1: "NQ_ERR_INVALID_ARG", 2: "NQ_ERR_UNSUPPORTED", 3: "NQ_ERR_OUT_OF_RANGE",
                4: "NQ_ERR_HIP", 5: "NQ_ERR_STATE", 6: "NQ_ERR_DEVICE_FAULT", 7: "NQ_ERR_IO"}
NQ_TENSOR_PACKED, NQ_TENSOR_F16 = 1, 2


class NQError(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        super().__init__(f"{func}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class NQConfig(ctypes.Structure):
    _fields_ = [("layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("group", ctypes.c_int32), ("page_tokens", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("max_pos", ctypes.c_int32)]

    @staticmethod
    def from_shape(shape, max_batch: int, max_pos: int) -> "NQConfig":
        return NQConfig(shape.layers, shape.hidden, shape.intermediate, shape.n_heads, shape.n_kv_heads,
                        shape.head_dim, shape.vocab, shape.rms_eps, shape.rope_theta, 128, 16,
                        max_batch, max_pos)


class NQLayerPtrs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("qkv_packed", "qkv_bias", "o_packed", "gate_up_packed",
                                                 "down_packed", "attn_norm", "mlp_norm")]


class NQStepIO(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("max_pages", ctypes.c_int32), ("page_table", ctypes.c_void_p),
                ("tokens", ctypes.c_void_p), ("pos", ctypes.c_void_p), ("logits", ctypes.c_void_p),
                ("layer_out", ctypes.c_void_p), ("token_hist", ctypes.c_void_p), ("hist_len", ctypes.c_int32),
                ("err_flag", ctypes.c_void_p)]


class NQTensorDesc(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("role", ctypes.c_int32), ("mat_kind", ctypes.c_int32),
                ("N", ctypes.c_int32), ("K", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("bytes", ctypes.c_uint64)]


class NQPrefillIO(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int32), ("start_pos", ctypes.c_int32), ("tokens", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("next_token", ctypes.c_void_p), ("pos_out", ctypes.c_void_p), ("logits", ctypes.c_void_p),
                ("layer_out", ctypes.c_void_p), ("err_flag", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("ws_bytes", ctypes.c_size_t)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_S = ctypes.c_size_t
_F = ctypes.c_float
_CFG = ctypes.POINTER(NQConfig)

_SIGS = {
    "nq_status_str": (ctypes.c_char_p, [_I]),
    "nq_last_error": (ctypes.c_char_p, []),
    "nq_layout_version": (_I, []),
    "nq_packed_size": (_S, [_I, _I, _I]),
    "nq_pack_weights": (_I, [_P, _I, _I, _I, _I, _I, _P, _P, _P]),
    "nq_unpack_weights": (_I, [_P, _I, _I, _I, _I, _I, _P, _P]),
    "nq_unpack_weights_dev": (_I, [_P, _I, _I, _I, _I, _I, _P, _P, _P]),
    "nq_gemv_w4a16": (_I, [_P, _I, _I, _I, _I, _I, _P, _P, _F, _P, _P, _I, _P]),
    "nq_config_check": (_I, [_CFG]),
    "nq_kv_pool_bytes": (_S, [_CFG, _I]),
    "nq_kv_alloc": (_I, [_CFG, _P, _S, _I, ctypes.POINTER(_P)]),
    "nq_kv_append": (_I, [_P, _I, _I, _P, _I, _P, _P, _P, _P, _P]),
    "nq_kv_free": (None, [_P]),
    "nq_attn_workspace_bytes": (_S, [_CFG, _I, _I]),
    "nq_attn_decode": (_I, [_P, _I, _I, _P, _P, _I, _P, _P, _P, _S, _P, _P]),
    "nq_attn_decode_static": (_I, [_P, _I, _I, _P, _P, _I, _P, _P, _P, _P]),
    "nq_model_create": (_I, [_CFG, ctypes.POINTER(_P)]),
    "nq_model_bind_layer": (_I, [_P, _I, ctypes.POINTER(NQLayerPtrs)]),
    "nq_model_bind_head": (_I, [_P, _P, _P, _P]),
    "nq_rope_table_bytes": (_S, [_CFG]),
    "nq_rope_table_fill": (_I, [_CFG, _P]),
    "nq_model_bind_rope": (_I, [_P, _P]),
    "nq_workspace_bytes": (_S, [_CFG, _I, _I]),
    "nq_model_bind_workspace": (_I, [_P, _P, _S]),
    "nq_model_destroy": (None, [_P]),
    "nq_model_set_step_mode": (_I, [_P, _I]),
    "nq_step_kernels": (_I, [_P, _I, _I]),
    "nq_model_set_step_trace": (_I, [_P, _P, ctypes.c_int64]),
    "nq_decode_step": (_I, [_P, _P, ctypes.POINTER(NQStepIO), _P]),
    "nq_graph_capture": (_I, [_P, _P, ctypes.POINTER(NQStepIO), _P, ctypes.POINTER(_P)]),
    "nq_graph_launch": (_I, [_P, _P]),
    "nq_graph_kernel_count": (_I, [_P]),
    "nq_graph_destroy": (None, [_P]),
    "nq_check_device_error": (_I, [_P, _P]),
    "nq_gemm_w4a16": (_I, [_P, _I, _I, _I, _I, _I, _P, _P, _P, _I, _P]),
    "nq_attn_prefill": (_I, [_P, _I, _I, _I, _P, _P, _I, _P, _P, _P]),
    "nq_prefill_workspace_bytes": (_S, [_CFG, _I]),
    "nq_prefill": (_I, [_P, _P, ctypes.POINTER(NQPrefillIO), _P]),
    "nq_a8_bytes": (_S, [_I, _I]),
    "nq_quantize_a8": (_I, [_P, _I, _I, _P, _P]),
    "nq_gemv_w4a8": (_I, [_P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P]),
    "nq_container_create": (_I, [ctypes.c_char_p, _CFG, _I, ctypes.POINTER(_P)]),
    "nq_container_add": (_I, [_P, ctypes.POINTER(NQTensorDesc), _P]),
    "nq_container_finish": (_I, [_P]),
    "nq_container_open": (_I, [ctypes.c_char_p, ctypes.POINTER(_P)]),
    "nq_container_config": (_I, [_P, _CFG]),
    "nq_container_count": (_I, [_P]),
    "nq_container_tensor": (_I, [_P, ctypes.c_char_p, ctypes.POINTER(NQTensorDesc), ctypes.POINTER(_P)]),
    "nq_container_tensor_at": (_I, [_P, _I, ctypes.POINTER(NQTensorDesc), ctypes.POINTER(_P)]),
    "nq_container_verify": (_I, [_P]),
    "nq_container_close": (None, [_P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libnq.so. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libnq.so not found at {LIB_PATH}; build it with "
                               "`python -m w4a16_gemv_paged_amd.build` (there is no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def header_symbols() -> list:
    """Names of the functions include/nq.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(nq_[a-z0-9_]+)\s*\(", text)))


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    return x.data_ptr()  # torch tensor


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(st: int, func: str) -> None:
    if st != NQ_OK:
        raise NQError(st, func, lib().nq_last_error().decode())


# ------------------------------------------------------------------ basics

def nq_status_str(s: int) -> str:
    return lib().nq_status_str(s).decode()


def nq_last_error() -> str:
    return lib().nq_last_error().decode()


def nq_layout_version() -> int:
    return lib().nq_layout_version()


def nq_packed_size(N: int, K: int, group: int = 128) -> int:
    return lib().nq_packed_size(N, K, group)


def nq_pack_weights(w: np.ndarray, kind: int = NQ_MAT_PLAIN, head_dim: int = 0, want_codes: bool = False,
                    group: int = 128):
    """Host packer. Returns the packed bytes (uint8), plus the logical codes and
    scale bits when ``want_codes``."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    size = lib().nq_packed_size(N, K, group)
    if size == 0:
        _check(lib().nq_pack_weights(_ptr(w), N, K, group, kind, head_dim, None, None, None), "nq_pack_weights")
    out = np.empty(size, np.uint8)
    q = np.empty((N, K), np.int8) if want_codes else None
    s = np.empty((N, K // group), np.uint16) if want_codes else None
    _check(lib().nq_pack_weights(_ptr(w), N, K, group, kind, head_dim, _ptr(out), _ptr(q), _ptr(s)),
           "nq_pack_weights")
    return (out, q, s) if want_codes else out


def nq_unpack_weights(packed: np.ndarray, N: int, K: int, kind: int = NQ_MAT_PLAIN, head_dim: int = 0,
                      group: int = 128):
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    q = np.empty((N, K), np.int8)
    s = np.empty((N, K // group), np.uint16)
    _check(lib().nq_unpack_weights(_ptr(packed), N, K, group, kind, head_dim, _ptr(q), _ptr(s)),
           "nq_unpack_weights")
    return q, s


def nq_unpack_weights_dev(packed, N, K, kind, head_dim, q_out, s_out, stream=None, group: int = 128):
    _check(lib().nq_unpack_weights_dev(_ptr(packed), N, K, group, kind, head_dim, _ptr(q_out), _ptr(s_out),
                                       _stream(stream)), "nq_unpack_weights_dev")


def nq_gemv_w4a16(packed, N, K, kind, head_dim, batch, x, norm_gain, eps, bias, y, epi, stream=None):
    _check(lib().nq_gemv_w4a16(_ptr(packed), N, K, kind, head_dim, batch, _ptr(x), _ptr(norm_gain), eps,
                               _ptr(bias), _ptr(y), epi, _stream(stream)), "nq_gemv_w4a16")


def nq_gemm_w4a16(packed, N, K, kind, head_dim, M, x, bias, y, epi, stream=None):
    _check(lib().nq_gemm_w4a16(_ptr(packed), N, K, kind, head_dim, M, _ptr(x), _ptr(bias), _ptr(y), epi,
                               _stream(stream)), "nq_gemm_w4a16")


def nq_a8_bytes(batch: int, K: int) -> int:
    return lib().nq_a8_bytes(batch, K)


def nq_quantize_a8(x, batch, K, xq, stream=None):
    _check(lib().nq_quantize_a8(_ptr(x), batch, K, _ptr(xq), _stream(stream)), "nq_quantize_a8")


def nq_gemv_w4a8(packed, N, K, kind, head_dim, batch, x, xq, bias, y, epi, stream=None):
    _check(lib().nq_gemv_w4a8(_ptr(packed), N, K, kind, head_dim, batch, _ptr(x), _ptr(xq), _ptr(bias), _ptr(y),
                              epi, _stream(stream)), "nq_gemv_w4a8")


def nq_config_check(cfg: NQConfig) -> None:
    _check(lib().nq_config_check(ctypes.byref(cfg)), "nq_config_check")


# ------------------------------------------------------------------ KV cache and attention

def nq_kv_pool_bytes(cfg: NQConfig, num_pages: int) -> int:
    return lib().nq_kv_pool_bytes(ctypes.byref(cfg), num_pages)


def nq_kv_alloc(cfg: NQConfig, pool, nbytes: int, num_pages: int) -> int:
    h = _P()
    _check(lib().nq_kv_alloc(ctypes.byref(cfg), _ptr(pool), nbytes, num_pages, ctypes.byref(h)), "nq_kv_alloc")
    return h.value


def nq_kv_append(kv, layer, batch, page_table, max_pages, pos, k, v, err_flag=None, stream=None):
    _check(lib().nq_kv_append(kv, layer, batch, _ptr(page_table), max_pages, _ptr(pos), _ptr(k), _ptr(v),
                              _ptr(err_flag), _stream(stream)), "nq_kv_append")


def nq_kv_free(kv) -> None:
    lib().nq_kv_free(kv)


def nq_attn_workspace_bytes(cfg: NQConfig, batch: int, max_pages: int) -> int:
    return lib().nq_attn_workspace_bytes(ctypes.byref(cfg), batch, max_pages)


def nq_attn_decode(kv, layer, batch, q, page_table, max_pages, lens, out, workspace, ws_bytes, err_flag=None,
                   stream=None):
    _check(lib().nq_attn_decode(kv, layer, batch, _ptr(q), _ptr(page_table), max_pages, _ptr(lens), _ptr(out),
                                _ptr(workspace), ws_bytes, _ptr(err_flag), _stream(stream)), "nq_attn_decode")


NQ_ATTN_SCRATCH_BYTES = 24 << 20


def nq_attn_decode_static(kv, layer, batch, q, page_table, max_pages, lens, out, err_flag=None, stream=None):
    _check(lib().nq_attn_decode_static(kv, layer, batch, _ptr(q), _ptr(page_table), max_pages, _ptr(lens), _ptr(out),
                                       _ptr(err_flag), _stream(stream)), "nq_attn_decode_static")


def nq_attn_prefill(kv, layer, n_q, start_pos, q, page_table, max_pages, out, err_flag=None, stream=None):
    _check(lib().nq_attn_prefill(kv, layer, n_q, start_pos, _ptr(q), _ptr(page_table), max_pages, _ptr(out),
                                 _ptr(err_flag), _stream(stream)), "nq_attn_prefill")


# ------------------------------------------------------------------ model, step, graph

NQ_STEP_AUTO, NQ_STEP_KERNELS = 0, 1


def nq_model_set_step_trace(model, buf, nbytes: int) -> None:
    _check(lib().nq_model_set_step_trace(model, _ptr(buf), nbytes), "nq_model_set_step_trace")


def nq_model_set_step_mode(model, mode: int) -> None:
    _check(lib().nq_model_set_step_mode(model, mode), "nq_model_set_step_mode")


def nq_step_kernels(model, batch: int, max_pages: int) -> int:
    return lib().nq_step_kernels(model, batch, max_pages)


def nq_model_create(cfg: NQConfig) -> int:
    h = _P()
    _check(lib().nq_model_create(ctypes.byref(cfg), ctypes.byref(h)), "nq_model_create")
    return h.value


def nq_model_bind_layer(m, layer: int, ptrs: NQLayerPtrs) -> None:
    _check(lib().nq_model_bind_layer(m, layer, ctypes.byref(ptrs)), "nq_model_bind_layer")


def nq_model_bind_head(m, embed, final_norm, lm_packed) -> None:
    _check(lib().nq_model_bind_head(m, _ptr(embed), _ptr(final_norm), _ptr(lm_packed)), "nq_model_bind_head")


def nq_rope_table_bytes(cfg: NQConfig) -> int:
    return lib().nq_rope_table_bytes(ctypes.byref(cfg))


def nq_rope_table_fill(cfg: NQConfig) -> np.ndarray:
    out = np.empty(cfg.max_pos * (cfg.head_dim // 2) * 2, np.float32)
    _check(lib().nq_rope_table_fill(ctypes.byref(cfg), _ptr(out)), "nq_rope_table_fill")
    return out.reshape(cfg.max_pos, cfg.head_dim // 2, 2)


def nq_model_bind_rope(m, table) -> None:
    _check(lib().nq_model_bind_rope(m, _ptr(table)), "nq_model_bind_rope")


def nq_workspace_bytes(cfg: NQConfig, batch: int, max_pages: int) -> int:
    return lib().nq_workspace_bytes(ctypes.byref(cfg), batch, max_pages)


def nq_model_bind_workspace(m, ws, nbytes: int) -> None:
    _check(lib().nq_model_bind_workspace(m, _ptr(ws), nbytes), "nq_model_bind_workspace")


def nq_model_destroy(m) -> None:
    lib().nq_model_destroy(m)


def nq_decode_step(m, kv, io: NQStepIO, stream=None) -> None:
    _check(lib().nq_decode_step(m, kv, ctypes.byref(io), _stream(stream)), "nq_decode_step")


def nq_graph_capture(m, kv, io: NQStepIO, stream=None) -> int:
    h = _P()
    _check(lib().nq_graph_capture(m, kv, ctypes.byref(io), _stream(stream), ctypes.byref(h)), "nq_graph_capture")
    return h.value


def nq_graph_launch(g, stream=None) -> None:
    _check(lib().nq_graph_launch(g, _stream(stream)), "nq_graph_launch")


def nq_graph_kernel_count(g) -> int:
    return lib().nq_graph_kernel_count(g)


def nq_graph_destroy(g) -> None:
    lib().nq_graph_destroy(g)


def nq_check_device_error(err_flag, stream=None) -> None:
    _check(lib().nq_check_device_error(_ptr(err_flag), _stream(stream)), "nq_check_device_error")


# ------------------------------------------------------------------ chunked prefill

def nq_prefill_workspace_bytes(cfg: NQConfig, chunk: int) -> int:
    return lib().nq_prefill_workspace_bytes(ctypes.byref(cfg), chunk)


def nq_prefill(m, kv, io: NQPrefillIO, stream=None) -> None:
    _check(lib().nq_prefill(m, kv, ctypes.byref(io), _stream(stream)), "nq_prefill")


# ------------------------------------------------------------------ packed-weight container

def nq_container_create(path: str, cfg: NQConfig, n_tensors: int):
    h = _P()
    _check(lib().nq_container_create(os.fsencode(path), ctypes.byref(cfg), n_tensors, ctypes.byref(h)),
           "nq_container_create")
    return h.value


def nq_container_add(w, name: str, role: int, N: int, K: int, data: np.ndarray, mat_kind: int = 0,
                     head_dim: int = 0) -> None:
    data = np.ascontiguousarray(data)
    d = NQTensorDesc(name.encode(), role, mat_kind, N, K, head_dim, data.nbytes)
    _check(lib().nq_container_add(w, ctypes.byref(d), _ptr(data)), "nq_container_add")


def nq_container_finish(w) -> None:
    _check(lib().nq_container_finish(w), "nq_container_finish")


def nq_container_open(path: str):
    h = _P()
    _check(lib().nq_container_open(os.fsencode(path), ctypes.byref(h)), "nq_container_open")
    return h.value


def nq_container_config(c) -> NQConfig:
    cfg = NQConfig()
    _check(lib().nq_container_config(c, ctypes.byref(cfg)), "nq_container_config")
    return cfg


def nq_container_count(c) -> int:
    return lib().nq_container_count(c)


def _tensor_view(d: NQTensorDesc, p: int) -> np.ndarray:
    return np.ctypeslib.as_array(ctypes.cast(p, ctypes.POINTER(ctypes.c_uint8)), shape=(d.bytes,))


def nq_container_tensor(c, name: str):
    """(description, read-only uint8 view of the mapped bytes) of a tensor."""
    d, p = NQTensorDesc(), _P()
    _check(lib().nq_container_tensor(c, name.encode(), ctypes.byref(d), ctypes.byref(p)), "nq_container_tensor")
    return d, _tensor_view(d, p.value)


def nq_container_tensor_at(c, index: int):
    d, p = NQTensorDesc(), _P()
    _check(lib().nq_container_tensor_at(c, index, ctypes.byref(d), ctypes.byref(p)), "nq_container_tensor_at")
    return d, _tensor_view(d, p.value)


def nq_container_verify(c) -> None:
    _check(lib().nq_container_verify(c), "nq_container_verify")


def nq_container_close(c) -> None:
    lib().nq_container_close(c)
