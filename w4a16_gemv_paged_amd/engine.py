"""Device-memory plumbing around libnq for a whole model.

Packs host parameters with ``nq_pack_weights`` (C++), uploads them into torch
tensors, binds them to an ``nq_model``, owns the KV pool, the workspace and the
per-step buffers, and drives decode steps (eager or as graph replays). PyTorch
is used only to allocate device memory, copy host data in and out and pick the
stream; every arithmetic step runs in libnq.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from . import (NQConfig, NQLayerPtrs, NQStepIO, NQ_MAT_PLAIN, NQ_MAT_QKV, NQ_MAT_GATE_UP, NQ_MAT_LM_HEAD,
               NQ_TENSOR_PACKED, NQ_TENSOR_F16, nq_container_create, nq_container_add, nq_container_finish,
               nq_container_open, nq_container_config, nq_container_tensor, nq_container_close,
               nq_pack_weights, nq_model_create, nq_model_bind_layer, nq_model_bind_head, nq_model_bind_rope,
               nq_rope_table_fill, nq_workspace_bytes, nq_model_bind_workspace, nq_model_destroy,
               nq_kv_pool_bytes, nq_kv_alloc, nq_kv_free, nq_decode_step, nq_graph_capture, nq_graph_launch,
               nq_graph_destroy, nq_graph_kernel_count, nq_check_device_error, NQPrefillIO,
               nq_prefill_workspace_bytes, nq_prefill, nq_model_set_step_mode, nq_step_kernels, nq_model_set_step_trace,
               NQ_STEP_AUTO, NQ_STEP_KERNELS)

STEP_MODES = {"auto": NQ_STEP_AUTO, "kernels": NQ_STEP_KERNELS}


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device, non_blocking=False)


# Per-layer tensors of a model, in the order of nq_layer_ptrs, and the head's.
LAYER_TENSORS = ("qkv", "qkv_bias", "o", "gate_up", "down", "attn_norm", "mlp_norm")
HEAD_TENSORS = ("embed", "final_norm", "lm_head")


def _pack_layer(p: dict, head_dim: int) -> dict:
    """Host tensors of one layer: the four packed projections (uint8) and the
    fp16 bias and norm gains."""
    return {
        "qkv": nq_pack_weights(np.concatenate([p["wq"], p["wk"], p["wv"]]), NQ_MAT_QKV, head_dim),
        "qkv_bias": np.concatenate([p["bq"], p["bk"], p["bv"]]).astype(np.float16),
        "o": nq_pack_weights(p["wo"], NQ_MAT_PLAIN),
        "gate_up": nq_pack_weights(np.concatenate([p["wg"], p["wu"]]), NQ_MAT_GATE_UP),
        "down": nq_pack_weights(p["wd"], NQ_MAT_PLAIN),
        "attn_norm": np.asarray(p["g1"], np.float16),
        "mlp_norm": np.asarray(p["g2"], np.float16),
    }


def _dev_bytes(a: np.ndarray, device) -> torch.Tensor:
    """Upload host bytes (packed uint8, or fp16 kept as int16 bits)."""
    a = np.ascontiguousarray(a)
    return to_device(a.view(np.int16) if a.dtype == np.float16 else a, device)


class DeviceModel:
    """A Qwen2-style decoder bound to libnq.

    ``layer_params(l)`` returns the parameter dict of layer l (float32
    wq/wk/wv/wo/wg/wu/wd, float16 bq/bk/bv/g1/g2); ``head`` holds float16
    embed/g_final and float32 lm_head. The weights are packed on the host and
    uploaded layer by layer; host copies are dropped after upload.
    ``DeviceModel.load`` builds the same model from a packed-weight container
    instead, with no repacking."""

    def __init__(self, shape, layer_params, head: dict, max_batch: int, max_pos: int, device="cuda"):
        self._setup(shape, max_batch, max_pos, device)
        # draw and pack layer l+1 on a helper thread while layer l is uploaded
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(1) as ex:
            nxt = ex.submit(lambda l: _pack_layer(layer_params(l), shape.head_dim), 0)
            for li in range(shape.layers):
                t = nxt.result()
                if li + 1 < shape.layers:
                    nxt = ex.submit(lambda l: _pack_layer(layer_params(l), shape.head_dim), li + 1)
                self._bind_layer(li, [t[n] for n in LAYER_TENSORS])
                del t
        self._bind_head(head["embed"], head["g_final"], nq_pack_weights(head["lm_head"], NQ_MAT_LM_HEAD))

    @classmethod
    def load(cls, path: str, max_batch: int, max_pos: int, device="cuda") -> "DeviceModel":
        """The model stored in a packed-weight container (``write_container``)."""
        from types import SimpleNamespace
        c = nq_container_open(path)
        try:
            cfg = nq_container_config(c)
            shape = SimpleNamespace(name=os.path.basename(path), layers=cfg.layers, hidden=cfg.hidden,
                                    intermediate=cfg.intermediate, n_heads=cfg.n_heads,
                                    n_kv_heads=cfg.n_kv_heads, head_dim=cfg.head_dim, vocab=cfg.vocab,
                                    rms_eps=cfg.rms_eps, rope_theta=cfg.rope_theta)
            self = cls.__new__(cls)
            self._setup(shape, max_batch, max_pos, device)

            def get(name):
                d, view = nq_container_tensor(c, name)
                return view.view(np.float16) if d.role == NQ_TENSOR_F16 else view

            for li in range(cfg.layers):
                self._bind_layer(li, [get(f"layer.{li}.{n}") for n in LAYER_TENSORS])
            self._bind_head(*[get(n) for n in HEAD_TENSORS])
        finally:
            nq_container_close(c)   # the device copies are complete (synchronous uploads)
        return self

    def _setup(self, shape, max_batch, max_pos, device):
        self.shape = shape
        self.device = device
        self.cfg = NQConfig.from_shape(shape, max_batch, max_pos)
        self.handle = nq_model_create(self.cfg)
        self._keep = []
        self.layers = []
        self.ws = None

    def _bind_layer(self, li: int, host: list):
        ts = [_dev_bytes(a, self.device) for a in host]
        names = ("qkv", "bias", "o", "gate_up", "down", "g1", "g2")
        self._keep.extend(ts)
        self.layers.append(dict(zip(names, ts)))
        nq_model_bind_layer(self.handle, li, NQLayerPtrs(*[t.data_ptr() for t in ts]))

    def _bind_head(self, embed, g_final, lm_packed):
        self.embed = _dev_bytes(np.asarray(embed, np.float16), self.device)
        self.g_final = _dev_bytes(np.asarray(g_final, np.float16), self.device)
        self.lm = _dev_bytes(lm_packed, self.device)
        nq_model_bind_head(self.handle, self.embed, self.g_final, self.lm)
        self.rope = to_device(nq_rope_table_fill(self.cfg), self.device)
        nq_model_bind_rope(self.handle, self.rope)

    def set_step_mode(self, mode: str) -> None:
        """"auto": the persistent whole-step kernel at batch 1 where supported;
        "kernels": the kernel-per-stage step at every batch."""
        nq_model_set_step_mode(self.handle, STEP_MODES[mode])

    def step_kernels(self, batch: int, max_pages: int) -> int:
        return nq_step_kernels(self.handle, batch, max_pages)

    def set_step_trace(self, buf) -> None:
        """Stage stamps of the persistent step into ``buf`` (a device tensor of
        at least 256 * (layers + 1) * 16 int64), or off with None."""
        if buf is None:
            nq_model_set_step_trace(self.handle, None, 0)
        else:
            nq_model_set_step_trace(self.handle, buf, buf.numel() * buf.element_size())

    def weight_bytes(self) -> int:
        n = sum(t.numel() * t.element_size() for t in self._keep)
        return n + self.lm.numel() + self.embed.numel() * 2 + self.g_final.numel() * 2

    def close(self):
        if self.handle:
            nq_model_destroy(self.handle)
            self.handle = None


class KVCache:
    """A caller-owned KV pool of ``num_pages`` pages (optionally NaN-poisoned)."""

    def __init__(self, model: DeviceModel, num_pages: int, poison: bool = True):
        self.num_pages = num_pages
        nbytes = nq_kv_pool_bytes(model.cfg, num_pages)
        self.pool = torch.empty(nbytes // 2, dtype=torch.int16, device=model.device)
        self.pool.fill_(0x7E00 if poison else 0)  # fp16 NaN bits
        self.handle = nq_kv_alloc(model.cfg, self.pool, nbytes, num_pages)

    def view(self, cfg: NQConfig) -> torch.Tensor:
        """The pool as fp16 [layer][2][page][kv_head][16 * head_dim] (bit view); K pages
        are token-major ([16][head_dim]) and V pages dim-major ([head_dim][16])."""
        return self.pool.view(torch.float16).view(cfg.layers, 2, self.num_pages, cfg.n_kv_heads, 16 * cfg.head_dim)

    def close(self):
        if self.handle:
            nq_kv_free(self.handle)
            self.handle = None


class Stepper:
    """Per-step device buffers for a batch and the io struct that points at them."""

    def __init__(self, model: DeviceModel, kv: KVCache, page_table: np.ndarray, hist_len: int = 0,
                 want_logits: bool = False, want_layers: bool = False):
        dev = model.device
        cfg = model.cfg
        self.model, self.kv = model, kv
        self.batch, self.max_pages = page_table.shape
        self.page_table = to_device(page_table.astype(np.int32), dev)
        self.tokens = torch.zeros(self.batch, dtype=torch.int32, device=dev)
        self.pos = torch.zeros(self.batch, dtype=torch.int32, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.logits = torch.empty(self.batch, cfg.vocab, dtype=torch.float32, device=dev) if want_logits else None
        self.layer_out = (torch.empty(cfg.layers, self.batch, cfg.hidden, dtype=torch.float16, device=dev)
                          if want_layers else None)
        self.hist = torch.full((self.batch, hist_len), -1, dtype=torch.int32, device=dev) if hist_len else None
        self.ws_bytes = nq_workspace_bytes(cfg, self.batch, self.max_pages)
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=dev)
        p = lambda t: t.data_ptr() if t is not None else None
        self.io = NQStepIO(self.batch, self.max_pages, p(self.page_table), p(self.tokens), p(self.pos),
                           p(self.logits), p(self.layer_out), p(self.hist), hist_len, p(self.err))
        self.graph = None

    def set_tokens(self, toks, stream=None):
        self.tokens.copy_(torch.as_tensor(np.asarray(toks, np.int32)), non_blocking=False)

    def set_pos(self, pos):
        self.pos.copy_(torch.as_tensor(np.asarray(pos, np.int32)), non_blocking=False)

    def step(self, stream=None):
        nq_model_bind_workspace(self.model.handle, self.ws, self.ws_bytes)
        nq_decode_step(self.model.handle, self.kv.handle, self.io, stream)

    def capture(self, stream):
        nq_model_bind_workspace(self.model.handle, self.ws, self.ws_bytes)
        self.graph = nq_graph_capture(self.model.handle, self.kv.handle, self.io, stream)
        return nq_graph_kernel_count(self.graph)

    def replay(self, stream):
        nq_graph_launch(self.graph, stream)

    def check(self, stream=None):
        nq_check_device_error(self.err, stream)

    def close(self):
        if self.graph:
            nq_graph_destroy(self.graph)
            self.graph = None


class Prefill:
    """Workspace and buffers of the chunked prefill (``nq_prefill``) at one chunk size."""

    def __init__(self, model: DeviceModel, kv: KVCache, chunk: int):
        self.model, self.kv, self.chunk = model, kv, chunk
        dev = model.device
        self.ws_bytes = nq_prefill_workspace_bytes(model.cfg, chunk)
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)

    def run(self, tokens, page_row, start_pos: int = 0, next_token=None, pos_out=None, logits=None,
            layer_out=None, stream=None):
        """Prefills ``tokens`` (positions start_pos..) of the sequence whose page-table row is ``page_row``
        (a device int32 tensor). Outputs go to the given device tensors (each optional)."""
        toks = torch.as_tensor(np.asarray(tokens, np.int32)).to(self.model.device)
        p = lambda t: t.data_ptr() if t is not None else None
        io = NQPrefillIO(len(tokens), start_pos, p(toks), p(page_row), page_row.numel(), self.chunk, p(next_token),
                         p(pos_out), p(logits), p(layer_out), p(self.err), p(self.ws), self.ws_bytes)
        nq_prefill(self.model.handle, self.kv.handle, io, stream)
        self._toks = toks  # alive until the stream has used it

    def check(self, stream=None):
        nq_check_device_error(self.err, stream)


def write_container(path: str, shape, layer_params, head: dict) -> None:
    """Packs a model (``layer_params(l)`` and ``head`` as for DeviceModel) into a
    packed-weight container file, one layer at a time."""
    cfg = NQConfig.from_shape(shape, 1, 1)
    w = nq_container_create(path, cfg, len(LAYER_TENSORS) * shape.layers + len(HEAD_TENSORS))
    try:
        for li in range(shape.layers):
            t = _pack_layer(layer_params(li), shape.head_dim)
            H, I, d = shape.hidden, shape.intermediate, shape.head_dim
            qkv_n = (shape.n_heads + 2 * shape.n_kv_heads) * d
            packed = {"qkv": (qkv_n, H, NQ_MAT_QKV, d), "o": (H, shape.n_heads * d, NQ_MAT_PLAIN, 0),
                      "gate_up": (2 * I, H, NQ_MAT_GATE_UP, 0), "down": (H, I, NQ_MAT_PLAIN, 0)}
            for name in LAYER_TENSORS:
                a = t[name]
                if name in packed:
                    N, K, kind, hd = packed[name]
                    nq_container_add(w, f"layer.{li}.{name}", NQ_TENSOR_PACKED, N, K, a, kind, hd)
                else:
                    nq_container_add(w, f"layer.{li}.{name}", NQ_TENSOR_F16, a.size, 1, a)
        nq_container_add(w, "embed", NQ_TENSOR_F16, shape.vocab, shape.hidden, np.asarray(head["embed"], np.float16))
        nq_container_add(w, "final_norm", NQ_TENSOR_F16, shape.hidden, 1, np.asarray(head["g_final"], np.float16))
        nq_container_add(w, "lm_head", NQ_TENSOR_PACKED, shape.vocab, shape.hidden,
                         nq_pack_weights(head["lm_head"], NQ_MAT_LM_HEAD), NQ_MAT_LM_HEAD)
    except BaseException:
        try:
            nq_container_finish(w)   # frees the writer; the count check fails, which is expected here
        except Exception:
            pass
        raise
    nq_container_finish(w)


def run_greedy(st: Stepper, prompts, n_gen: int, use_graph: bool = False, stream=None,
               record_logits: bool = False, record_layers: bool = False, prefill_chunk: int | None = None):
    """Greedy decode of ``batch`` sequences in lockstep, one token per step.

    prompts: list of int sequences (ragged allowed). Sequence b goes through its
    prompt at positions 0..P_b-1, then generates n_gen tokens, feeding each
    back (the cache ends at P_b + n_gen - 1 positions). Sequences whose prompt
    is shorter start generating earlier and stop after n_gen tokens; they keep
    stepping (their extra tokens are ignored) until every sequence is done.
    Returns generated tokens [B][n_gen] and, if asked, the logits / layer
    outputs seen at every step.

    With ``prefill_chunk``, each prompt goes through ``nq_prefill`` instead
    (chunks of that many tokens), which yields its first generated token and
    position; the remaining n_gen - 1 tokens come from decode steps. Logits and
    layer outputs of the decode steps are recorded as above; ``record_layers``
    also returns each sequence's prefill layer outputs [L][P_b][H]
    (``prefill_layer_out``) and ``record_logits`` the logits of the prompt's
    last row (``prefill_logits`` [B][V])."""
    if prefill_chunk:
        return _run_prefilled(st, prompts, n_gen, use_graph, stream, record_logits, record_layers, prefill_chunk)
    B = st.batch
    P = [len(p) for p in prompts]
    total = max(P) + n_gen - 1
    if stream is None:
        stream = torch.cuda.current_stream()
    gen = [[] for _ in range(B)]
    logits, layers = [], []
    cur = np.array([p[0] for p in prompts], np.int32)
    st.set_pos(np.zeros(B, np.int32))
    st.set_tokens(cur)
    if use_graph and st.graph is None:
        st.capture(stream)
    for s in range(total):
        if use_graph:
            st.replay(stream)
        else:
            st.step(stream)
        nxt = st.tokens.cpu().numpy()
        if record_logits:
            logits.append(st.logits.cpu().numpy().copy())
        if record_layers:
            layers.append(st.layer_out.cpu().numpy().copy())
        for b in range(B):
            if s >= P[b] - 1 and len(gen[b]) < n_gen:
                gen[b].append(int(nxt[b]))
            cur[b] = prompts[b][s + 1] if s + 1 < P[b] else nxt[b]
        st.set_tokens(cur)
    st.check(stream)
    out = {"tokens": np.array(gen, np.int64)}
    if record_logits:
        out["logits"] = np.array(logits)
    if record_layers:
        out["layer_out"] = np.array(layers)
    return out


def _run_prefilled(st: Stepper, prompts, n_gen, use_graph, stream, record_logits, record_layers, chunk):
    B = st.batch
    if stream is None:
        stream = torch.cuda.current_stream()
    pf = Prefill(st.model, st.kv, chunk)
    cfg = st.model.cfg
    pf_layers, pf_logits = [], []
    for b in range(B):
        lo = (torch.empty(cfg.layers, len(prompts[b]), cfg.hidden, dtype=torch.float16, device=st.model.device)
              if record_layers else None)
        lg = torch.empty(cfg.vocab, dtype=torch.float32, device=st.model.device) if record_logits else None
        pf.run(prompts[b], st.page_table[b], 0, next_token=st.tokens[b:b + 1], pos_out=st.pos[b:b + 1],
               logits=lg, layer_out=lo, stream=stream)
        if record_layers:
            pf_layers.append(lo.cpu().numpy())
        if record_logits:
            pf_logits.append(lg.cpu().numpy())
    pf.check(stream)
    gen = [[int(t)] for t in st.tokens.cpu().numpy()]
    logits, layers = [], []
    if use_graph and st.graph is None:
        st.capture(stream)
    for _ in range(n_gen - 1):
        if use_graph:
            st.replay(stream)
        else:
            st.step(stream)
        nxt = st.tokens.cpu().numpy()
        if record_logits:
            logits.append(st.logits.cpu().numpy().copy())
        if record_layers:
            layers.append(st.layer_out.cpu().numpy().copy())
        for b in range(B):
            gen[b].append(int(nxt[b]))
    st.check(stream)
    out = {"tokens": np.array(gen, np.int64)}
    if record_logits:
        out["logits"] = np.array(logits)
        out["prefill_logits"] = np.array(pf_logits)
    if record_layers:
        out["layer_out"] = np.array(layers)
        out["prefill_layer_out"] = pf_layers
    return out
