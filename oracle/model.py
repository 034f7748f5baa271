"""Decode-step oracle: Qwen2-style decoder with INT4 weights and fp16 activations.

TEST INFRASTRUCTURE ONLY (see the package docstring). Everything is computed
in float64 from the stored inputs and rounded to float16 (round-half-even)
only where the method defines an fp16 tensor ("W4A16": fp16 activations):
the hidden state after the embedding gather and after each residual add, the
normalised inputs of the projections, q/k/v after the QKV bias, q and k after
RoPE (and so the K/V cache), the attention output and the SwiGLU output.
Logits stay float64.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from .quant import quantize_w4, dequantize_w4, GROUP

F16 = np.float16
F64 = np.float64


# --------------------------------------------------------------------------
# Elementary operations
# --------------------------------------------------------------------------

def softmax(x) -> np.ndarray:
    """Numerically stable softmax along the last axis, as the "Inference Zero
    To Hero" preface defines it (section "How each chapter works"): subtract
    the maximum, exponentiate, divide by the sum of the exponentials."""
    x = np.asarray(x, dtype=F64)
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def rmsnorm(x16, g16, eps: float) -> np.ndarray:
    """RMSNorm of an fp16 row: y = fp16( x / sqrt(mean(x^2) + eps) * g ).

    READING: the pages name no normalisation; Qwen2 uses RMSNorm with a gain
    and eps 1e-6. One rounding, at the end."""
    x = np.asarray(x16, dtype=F16).astype(F64)
    g = np.asarray(g16, dtype=F16).astype(F64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return (x * r * g).astype(F16)


def rope_angles(pos, d: int, theta: float) -> np.ndarray:
    """phi[..., i] = pos * theta^(-2i/d) for i < d/2 (float64)."""
    i = np.arange(d // 2, dtype=F64)
    inv = np.power(F64(theta), -2.0 * i / d)
    return np.asarray(pos, dtype=F64)[..., None] * inv


def rope(x16, pos, theta: float) -> np.ndarray:
    """Rotary position embedding, rotate-half pairing (READING: Qwen2's
    convention; the pages are silent). Pairs (i, i + d/2) are rotated by
    phi_i = pos * theta^(-2i/d):

      x'_i       = x_i cos phi - x_{i+d/2} sin phi
      x'_{i+d/2} = x_{i+d/2} cos phi + x_i sin phi

    ``x16`` is [..., heads, d]; ``pos`` is a scalar or has the leading shape
    ``[...]``. Returns fp16."""
    x = np.asarray(x16, dtype=F16).astype(F64)
    d = x.shape[-1]
    h = d // 2
    phi = rope_angles(pos, d, theta)
    c = np.cos(phi)[..., None, :]
    s = np.sin(phi)[..., None, :]
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1).astype(F16)


def attend(q16, k16, v16) -> np.ndarray:
    """Single-query attention over a contiguous cache (float64 result).

    Scores s_t = q . k_t / sqrt(d), softmax, o = sum_t p_t v_t ("Build Crude
    Implementations for Learning", section "nanoGPT level"; in decode the
    current token is the last row, so the causal mask keeps every cached row).
    q16 [nh, d]; k16, v16 [T, nkv, d]. READING (grouped-query attention with
    28 query and 4 KV heads): query head h reads KV head h // (nh / nkv)."""
    q = np.asarray(q16, dtype=F16).astype(F64)
    K = np.asarray(k16, dtype=F16).astype(F64)
    V = np.asarray(v16, dtype=F16).astype(F64)
    nh, d = q.shape
    nkv = K.shape[1]
    rep = nh // nkv
    out = np.empty((nh, d), dtype=F64)
    for h in range(nh):
        kv = h // rep
        s = (K[:, kv, :] @ q[h]) / math.sqrt(d)
        out[h] = softmax(s) @ V[:, kv, :]
    return out


def attend_splitk(q16, k16, v16, splits: int) -> np.ndarray:
    """Same result as :func:`attend`, computed from per-chunk partials.

    The cache is cut into ``splits`` contiguous chunks; each chunk c gives
    (m_c, l_c, o_c) = (max score, sum exp(s - m_c), sum exp(s - m_c) v). They
    combine as m = max m_c, o = sum e^{m_c - m} o_c / sum e^{m_c - m} l_c,
    which is exactly the softmax over the whole cache."""
    q = np.asarray(q16, dtype=F16).astype(F64)
    K = np.asarray(k16, dtype=F16).astype(F64)
    V = np.asarray(v16, dtype=F16).astype(F64)
    nh, d = q.shape
    T, nkv, _ = K.shape
    rep = nh // nkv
    bounds = np.linspace(0, T, splits + 1).round().astype(int)
    out = np.empty((nh, d), dtype=F64)
    for h in range(nh):
        kv = h // rep
        parts = []
        for c in range(splits):
            t0, t1 = bounds[c], bounds[c + 1]
            if t1 <= t0:
                continue
            s = (K[t0:t1, kv, :] @ q[h]) / math.sqrt(d)
            m = np.max(s)
            e = np.exp(s - m)
            parts.append((m, np.sum(e), e @ V[t0:t1, kv, :]))
        m = max(p[0] for p in parts)
        num = sum(math.exp(p[0] - m) * p[2] for p in parts)
        den = sum(math.exp(p[0] - m) * p[1] for p in parts)
        out[h] = num / den
    return out


def swiglu(g, u) -> np.ndarray:
    """a = fp16( silu(g) * u ) with silu(g) = g / (1 + e^-g), from float64 g, u.
    READING: Qwen2's MLP; the pages only name the gate/up/down projections."""
    g = np.asarray(g, dtype=F64)
    u = np.asarray(u, dtype=F64)
    return (g / (1.0 + np.exp(-g)) * u).astype(F16)


def argmax_lowest(z) -> int:
    """Greedy choice: index of the largest logit, lowest index on ties
    (READING). NaN logits are an error."""
    z = np.asarray(z, dtype=F64)
    if np.any(np.isnan(z)):
        raise ValueError("NaN in logits")
    return int(np.argmax(z))


def gemv_w4a16(q, s16, x16, bias16=None) -> np.ndarray:
    """y[b] = W^ x[b] (+ bias) in float64, W^ = dequantize(q, s16); x fp16 [B, K]."""
    w = dequantize_w4(q, s16)
    x = np.asarray(x16, dtype=F16).astype(F64)
    y = x @ w.T
    if bias16 is not None:
        y = y + np.asarray(bias16, dtype=F16).astype(F64)
    return y


# --------------------------------------------------------------------------
# KV caches
# --------------------------------------------------------------------------

class ContiguousKV:
    """Unpaged cache of one sequence: per layer, K and V as [T, nkv, d] fp16."""

    def __init__(self, layers: int, n_kv: int, d: int):
        self.k = [np.zeros((0, n_kv, d), F16) for _ in range(layers)]
        self.v = [np.zeros((0, n_kv, d), F16) for _ in range(layers)]

    def append(self, layer: int, pos: int, k16, v16) -> None:
        if pos != self.k[layer].shape[0]:
            raise ValueError("contiguous cache is append-only")
        self.k[layer] = np.concatenate([self.k[layer], np.asarray(k16, F16)[None]], axis=0)
        self.v[layer] = np.concatenate([self.v[layer], np.asarray(v16, F16)[None]], axis=0)

    def get(self, layer: int, length: int):
        return self.k[layer][:length], self.v[layer][:length]


class PagedKVEmu:
    """Paged cache ("What it actually builds": 16 tokens per page, pages are
    non-contiguous blocks found through a page table).

    Pool layout [layer][K=0 / V=1][page][kv_head][16 * d] fp16: one page of one
    KV head holds 16 tokens x d fp16 (4 KiB at d = 128). The pages fix only the
    page size, so the order inside a page is a reading: K is token-major
    (element slot * d + e) and V is dim-major (element e * 16 + slot). Token p
    of sequence b lives in page page_table[b][p // 16], slot p % 16. The pool
    starts filled with NaN so that a read of a slot never written shows up."""

    def __init__(self, layers: int, num_pages: int, n_kv: int, d: int,
                 page_table, page_tokens: int = 16, pool=None):
        self.page_tokens = page_tokens
        self.d = d
        self.pt = np.asarray(page_table, dtype=np.int32)
        if pool is None:
            pool = np.full((layers, 2, num_pages, n_kv, page_tokens * d), np.nan, dtype=F16)
        if pool.shape[-1] != page_tokens * d:
            raise ValueError("pool pages must hold page_tokens * d elements per KV head")
        self.pool = pool

    def locate(self, b: int, pos: int):
        j = pos // self.page_tokens
        if j >= self.pt.shape[1]:
            raise IndexError("position beyond the page table")
        page = int(self.pt[b, j])
        if page < 0 or page >= self.pool.shape[2]:
            raise IndexError(f"page id {page} out of range")
        return page, pos % self.page_tokens

    def append(self, layer: int, b: int, pos: int, k16, v16) -> None:
        """k16, v16 [n_kv, d] of token ``pos``."""
        page, slot = self.locate(b, pos)
        d, T = self.d, self.page_tokens
        self.pool[layer, 0, page, :, slot * d:(slot + 1) * d] = k16
        self.pool[layer, 1, page, :, slot::T] = v16

    def get(self, layer: int, b: int, length: int):
        """K and V of positions 0..length-1 as [length, n_kv, d]."""
        T, d = self.page_tokens, self.d
        npages = (length + T - 1) // T
        ids = self.pt[b, :npages]
        if np.any(ids < 0) or np.any(ids >= self.pool.shape[2]):
            raise IndexError("page table entry out of range")
        nkv = self.pool.shape[3]
        k = self.pool[layer, 0, ids].reshape(npages, nkv, T, d).transpose(0, 2, 1, 3)
        v = self.pool[layer, 1, ids].reshape(npages, nkv, d, T).transpose(0, 3, 1, 2)
        return (k.reshape(npages * T, nkv, d)[:length], v.reshape(npages * T, nkv, d)[:length])


def paged_attention(q16, pool_layer, page_table, lens) -> np.ndarray:
    """Decode attention of B sequences over one layer's page pool.

    q16 [B, nh, d]; pool_layer [2][P][nkv][16 * d] (PagedKVEmu layout);
    lens[b] = number of cached tokens of sequence b. Returns float64 [B, nh, d]."""
    q16 = np.asarray(q16, dtype=F16)
    pool = np.asarray(pool_layer, dtype=F16)[None]
    d = q16.shape[-1]
    kv = PagedKVEmu(1, pool.shape[2], pool.shape[3], d, page_table,
                    page_tokens=pool.shape[4] // d, pool=pool)
    out = np.empty(q16.shape, dtype=F64)
    for b in range(q16.shape[0]):
        k, v = kv.get(0, b, int(lens[b]))
        out[b] = attend(q16[b], k, v)
    return out


# --------------------------------------------------------------------------
# Model
# --------------------------------------------------------------------------

@dataclass
class Dims:
    hidden: int
    intermediate: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    vocab: int
    rms_eps: float = 1e-6
    rope_theta: float = 1e6


class OracleLayer:
    """One decoder layer: quantised fused QKV [Wq; Wk; Wv] with bias, O,
    fused gate/up [Wg; Wu], down, and the two RMSNorm gains."""

    def __init__(self, p: dict, quant=quantize_w4):
        """``quant`` maps a float32 [N, K] matrix to (codes, scales); any
        replacement must equal quantize_w4 (e.g. it applied to row blocks)."""
        self.q_qkv, self.s_qkv = quant(np.concatenate([p["wq"], p["wk"], p["wv"]], axis=0))
        self.b_qkv = np.concatenate([p["bq"], p["bk"], p["bv"]]).astype(F16)
        self.q_o, self.s_o = quant(p["wo"])
        self.q_gu, self.s_gu = quant(np.concatenate([p["wg"], p["wu"]], axis=0))
        self.q_d, self.s_d = quant(p["wd"])
        self.g1 = np.asarray(p["g1"], F16)
        self.g2 = np.asarray(p["g2"], F16)
        self._w = {}

    def w(self, name: str) -> np.ndarray:
        """Dequantised float64 matrix, cached."""
        if name not in self._w:
            q, s = {"qkv": (self.q_qkv, self.s_qkv), "o": (self.q_o, self.s_o),
                    "gu": (self.q_gu, self.s_gu), "d": (self.q_d, self.s_d)}[name]
            self._w[name] = dequantize_w4(q, s)
        return self._w[name]

    def drop_cache(self) -> None:
        self._w = {}


class OracleHead:
    """Embedding (fp16, untied), final RMSNorm gain and quantised LM head."""

    def __init__(self, h: dict, quant=quantize_w4):
        self.embed = np.asarray(h["embed"], F16)
        self.g_final = np.asarray(h["g_final"], F16)
        self.q_lm, self.s_lm = quant(h["lm_head"])
        self._w = None

    def w_lm(self) -> np.ndarray:
        if self._w is None:
            self._w = dequantize_w4(self.q_lm, self.s_lm)
        return self._w


@dataclass
class OracleModel:
    dims: Dims
    layers: list
    head: OracleHead = None
    layer_ids: list = field(default=None)

    @staticmethod
    def build(shape, layer_params: list, head_params: dict | None) -> "OracleModel":
        dims = Dims(shape.hidden, shape.intermediate, shape.n_heads, shape.n_kv_heads,
                    shape.head_dim, shape.vocab, shape.rms_eps, shape.rope_theta)
        layers = [OracleLayer(p) for p in layer_params]
        head = OracleHead(head_params) if head_params is not None else None
        return OracleModel(dims, layers, head, list(range(len(layers))))


def _split_qkv(qkv16, dims: Dims):
    nh, nkv, d = dims.n_heads, dims.n_kv_heads, dims.head_dim
    q = qkv16[..., : nh * d].reshape(*qkv16.shape[:-1], nh, d)
    k = qkv16[..., nh * d: (nh + nkv) * d].reshape(*qkv16.shape[:-1], nkv, d)
    v = qkv16[..., (nh + nkv) * d:].reshape(*qkv16.shape[:-1], nkv, d)
    return q, k, v


def layer_decode(layer: OracleLayer, dims: Dims, h16, pos: int, cache_append, cache_get,
                 trace: dict | None = None) -> np.ndarray:
    """One layer of the single-token decode step (fp16 in, fp16 out).

    x = rmsnorm(h, g1); qkv = W_qkv x + b; q, k = rope(q, k, pos); append k, v
    at ``pos``; o = attention over positions [0, pos]; h = h + W_o o;
    x2 = rmsnorm(h, g2); a = silu(W_g x2) * (W_u x2); h = h + W_d a."""
    h16 = np.asarray(h16, F16)
    x = rmsnorm(h16, layer.g1, dims.rms_eps)
    qkv = (layer.w("qkv") @ x.astype(F64) + layer.b_qkv.astype(F64)).astype(F16)
    q, k, v = _split_qkv(qkv, dims)
    q = rope(q, pos, dims.rope_theta)
    k = rope(k, pos, dims.rope_theta)
    cache_append(k, v)
    K, V = cache_get(pos + 1)
    o = attend(q, K, V).astype(F16).reshape(-1)
    h = (h16.astype(F64) + layer.w("o") @ o.astype(F64)).astype(F16)
    x2 = rmsnorm(h, layer.g2, dims.rms_eps)
    gu = layer.w("gu") @ x2.astype(F64)
    a = swiglu(gu[: dims.intermediate], gu[dims.intermediate:])
    out = (h.astype(F64) + layer.w("d") @ a.astype(F64)).astype(F16)
    if trace is not None:
        trace.update(x=x, qkv=qkv, q=q, k=k, v=v, o=o, h_mid=h, x2=x2, a=a, h_out=out)
    return out


def layer_causal(layer: OracleLayer, dims: Dims, h16) -> np.ndarray:
    """The same layer over positions 0..T-1 at once (causal), fp16 [T, H] in
    and out. Each position attends to positions <= itself."""
    h16 = np.asarray(h16, F16)
    T = h16.shape[0]
    x = rmsnorm(h16, layer.g1, dims.rms_eps)
    qkv = (x.astype(F64) @ layer.w("qkv").T + layer.b_qkv.astype(F64)).astype(F16)
    q, k, v = _split_qkv(qkv, dims)
    pos = np.arange(T)
    q = rope(q, pos, dims.rope_theta)
    k = rope(k, pos, dims.rope_theta)
    o = np.empty((T, dims.n_heads * dims.head_dim), F16)
    for t in range(T):
        o[t] = attend(q[t], k[: t + 1], v[: t + 1]).astype(F16).reshape(-1)
    h = (h16.astype(F64) + o.astype(F64) @ layer.w("o").T).astype(F16)
    x2 = rmsnorm(h, layer.g2, dims.rms_eps)
    gu = x2.astype(F64) @ layer.w("gu").T
    a = swiglu(gu[:, : dims.intermediate], gu[:, dims.intermediate:])
    return (h.astype(F64) + a.astype(F64) @ layer.w("d").T).astype(F16)


def head_logits(model: OracleModel, h16) -> np.ndarray:
    """Final RMSNorm then the LM head: z = W_lm x (float64)."""
    x = rmsnorm(np.asarray(h16, F16), model.head.g_final, model.dims.rms_eps)
    return x.astype(F64) @ model.head.w_lm().T


def causal_forward(model: OracleModel, tokens) -> dict:
    """Layer-major forward over a whole token sequence. Returns the fp16
    hidden state after every layer ([L][T, H]) and float64 logits [T, V]."""
    tokens = np.asarray(tokens, dtype=np.int64)
    h = model.head.embed[tokens]
    outs = []
    for layer in model.layers:
        h = layer_causal(layer, model.dims, h)
        outs.append(h)
    return {"layer_out": outs, "logits": head_logits(model, h)}


def decode_step(model: OracleModel, caches, tokens, pos, trace: list | None = None) -> dict:
    """One greedy decode step for a batch.

    ``caches[b]`` is a ContiguousKV, or a (PagedKVEmu, b) pair; ``tokens[b]``
    is the input token at position ``pos[b]``. Returns float64 logits [B, V],
    next tokens (argmax, lowest index on ties) and the fp16 hidden state after
    every layer [L, B, H]."""
    B = len(tokens)
    L = len(model.layers)
    H = model.dims.hidden
    layer_out = np.empty((L, B, H), F16)
    logits = np.empty((B, model.dims.vocab), F64)
    nxt = np.empty(B, np.int64)
    for b in range(B):
        p = int(pos[b])
        h = model.head.embed[int(tokens[b])]
        cache = caches[b]
        for li, layer in enumerate(model.layers):
            if isinstance(cache, ContiguousKV):
                app = lambda k, v, li=li: cache.append(li, p, k, v)
                get = lambda n, li=li: cache.get(li, n)
            else:
                kv, bb = cache
                app = lambda k, v, li=li: kv.append(li, bb, p, k, v)
                get = lambda n, li=li: kv.get(li, bb, n)
            tr = {} if trace is not None else None
            h = layer_decode(layer, model.dims, h, p, app, get, tr)
            if trace is not None:
                trace.append(tr)
            layer_out[li, b] = h
        logits[b] = head_logits(model, h)
        nxt[b] = argmax_lowest(logits[b])
    return {"logits": logits, "next": nxt, "layer_out": layer_out}


def generate(model: OracleModel, prompt, n_gen: int, forced=None, paged=None) -> dict:
    """Greedy generation of one sequence, one token per step.

    Run convention (READING): the P prompt tokens go through the step one at a
    time at positions 0..P-1; the argmax at position P-1 is generated token 1;
    each generated token is fed back, so the cache ends at P + n_gen - 1
    positions. If ``forced`` is given, those tokens are fed back instead of the
    oracle's own choices (token teacher forcing); the oracle's own argmax and
    top-1 margin are still reported. ``paged`` = (PagedKVEmu, b) uses that
    cache instead of a contiguous one."""
    prompt = [int(t) for t in prompt]
    d = model.dims
    cache = paged if paged is not None else ContiguousKV(len(model.layers), d.n_kv_heads, d.head_dim)
    toks, logits, margins, layer_out = [], [], [], []
    feed = prompt[0]
    for step in range(len(prompt) + n_gen - 1):
        r = decode_step(model, [cache], [feed], [step])
        layer_out.append(r["layer_out"][:, 0])
        if step >= len(prompt) - 1:
            z = r["logits"][0]
            top2 = np.sort(z)[-2:]
            toks.append(int(r["next"][0]))
            logits.append(z)
            margins.append(float(top2[1] - top2[0]))
            g = len(toks)
            feed = int(forced[g - 1]) if forced is not None else toks[-1]
        else:
            feed = prompt[step + 1]
    return {"tokens": np.array(toks, np.int64), "logits": np.array(logits),
            "margins": np.array(margins), "layer_out": np.array(layer_out)}
