"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers and lays them out in the shapes of the
workloads. It holds none of the decode method's arithmetic (no quantisation, no
normalisation, no attention): both the HIP path and the CPU oracle take what it
returns and do their own work on it.

Determinism: every tensor is drawn from its own ``numpy.random.Generator``
(PCG64) seeded with the integer list ``[seed, *key, chunk]`` (NumPy builds a
SeedSequence from that list). Large matrices are drawn in row chunks of
``ROW_CHUNK`` rows, each chunk from its own key, so they can be drawn on several
threads and the values do not depend on the thread count, and any one layer can
be drawn without drawing the others.

Parameter storage formats (the model is "W4A16"): projection matrices come out
as float32 (each side quantises them to INT4 itself); the embedding, norm gains
and QKV biases come out as float16, which is how the model stores them.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

ROW_CHUNK = 1024
WEIGHT_STD = np.float32(0.02)

# tensor codes used in the seed key
_CODES = {
    "wq": 1, "wk": 2, "wv": 3, "bq": 4, "bk": 5, "bv": 6, "wo": 7,
    "wg": 8, "wu": 9, "wd": 10, "g1": 11, "g2": 12,
    "embed": 20, "lm_head": 21, "g_final": 22,
}


@dataclass(frozen=True)
class ModelShape:
    """Dimensions of a Qwen2-style decoder."""
    name: str
    layers: int
    hidden: int
    intermediate: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    vocab: int
    rms_eps: float = 1e-6
    rope_theta: float = 1e6


TINY = ModelShape("tiny-qwen2-2L-h512", 2, 512, 1408, 8, 2, 64, 4096)
QWEN7B = ModelShape("qwen2.5-coder-7b-shape", 28, 3584, 18944, 28, 4, 128, 152064)

# (K, N) of the fused projections of the 7B shape: QKV, O, gate/up, down
GEMV_SHAPES_7B = [(3584, 4608), (3584, 3584), (3584, 37888), (18944, 3584)]


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_matrix(seed: int, key: tuple, rows: int, cols: int,
                  std: np.float32 = WEIGHT_STD, pool: ThreadPoolExecutor | None = None) -> np.ndarray:
    """float32 [rows, cols] ~ N(0, std^2), drawn in row chunks keyed by ``key``."""
    out = np.empty((rows, cols), dtype=np.float32)
    nchunks = (rows + ROW_CHUNK - 1) // ROW_CHUNK

    def fill(c: int) -> None:
        r0 = c * ROW_CHUNK
        r1 = min(rows, r0 + ROW_CHUNK)
        rng = np.random.default_rng([seed, *key, c])
        blk = out[r0:r1]
        rng.standard_normal(out=blk, dtype=np.float32)
        np.multiply(blk, std, out=blk)

    if pool is None and nchunks > 1:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    elif pool is not None:
        list(pool.map(fill, range(nchunks)))
    else:
        fill(0)
    return out


def _vec(seed: int, key: tuple, n: int, std=WEIGHT_STD) -> np.ndarray:
    rng = np.random.default_rng([seed, *key, 0])
    return (rng.standard_normal(n, dtype=np.float32) * np.float32(std))


def layer_params(shape: ModelShape, layer: int, seed: int = 0) -> dict:
    """Parameters of one decoder layer.

    Keys: wq [nh*d, H], wk [nkv*d, H], wv [nkv*d, H], wo [H, nh*d], wg [I, H],
    wu [I, H], wd [H, I] (float32, torch Linear [out, in] layout);
    bq, bk, bv (float16); g1, g2 (float16 gains = 1 + N(0, 0.02)).
    """
    H, I, nh, nkv, d = shape.hidden, shape.intermediate, shape.n_heads, shape.n_kv_heads, shape.head_dim
    k = lambda name: (layer, _CODES[name])
    p = {
        "wq": normal_matrix(seed, k("wq"), nh * d, H),
        "wk": normal_matrix(seed, k("wk"), nkv * d, H),
        "wv": normal_matrix(seed, k("wv"), nkv * d, H),
        "bq": _vec(seed, k("bq"), nh * d).astype(np.float16),
        "bk": _vec(seed, k("bk"), nkv * d).astype(np.float16),
        "bv": _vec(seed, k("bv"), nkv * d).astype(np.float16),
        "wo": normal_matrix(seed, k("wo"), H, nh * d),
        "wg": normal_matrix(seed, k("wg"), I, H),
        "wu": normal_matrix(seed, k("wu"), I, H),
        "wd": normal_matrix(seed, k("wd"), H, I),
        "g1": (np.float32(1) + _vec(seed, k("g1"), H)).astype(np.float16),
        "g2": (np.float32(1) + _vec(seed, k("g2"), H)).astype(np.float16),
    }
    return p


def head_params(shape: ModelShape, seed: int = 0) -> dict:
    """Embedding E [V, H] float16, LM head W_lm [V, H] float32 (untied), final gain float16."""
    k = lambda name: (10_000, _CODES[name])
    emb = normal_matrix(seed, k("embed"), shape.vocab, shape.hidden).astype(np.float16)
    lm = normal_matrix(seed, k("lm_head"), shape.vocab, shape.hidden)
    gf = (np.float32(1) + _vec(seed, k("g_final"), shape.hidden)).astype(np.float16)
    return {"embed": emb, "lm_head": lm, "g_final": gf}


def prompt_ids(n: int, vocab: int, seed: int = 2, batch: int | None = None) -> np.ndarray:
    """Prompt token ids uniform in [0, vocab) (int32, shape [n] or [batch, n])."""
    rng = np.random.default_rng(seed)
    shape = (n,) if batch is None else (batch, n)
    return rng.integers(0, vocab, size=shape, dtype=np.int64).astype(np.int32)


def ragged_lengths(batch: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Lengths uniform in [lo, hi] inclusive (int32)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=batch, dtype=np.int64).astype(np.int32)


def activations(batch: int, k: int, seed: int = 1) -> np.ndarray:
    """GEMV activations: float16 [batch, k] ~ N(0, 1)."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((batch, k), dtype=np.float32).astype(np.float16)


def gemv_weight(k: int, n: int, seed: int = 0, copy: int = 0) -> np.ndarray:
    """GEMV weight float32 [n, k] ~ N(0, 0.02); ``copy`` picks an independent draw."""
    return normal_matrix(seed, (20_000 + copy, n, k), n, k)


def page_permutation(num_pages: int, seed: int = 3) -> np.ndarray:
    """A random permutation of physical page ids (int32)."""
    rng = np.random.default_rng(seed)
    return rng.permutation(num_pages).astype(np.int32)


def attention_inputs(batch: int, n_heads: int, n_kv: int, head_dim: int, lens,
                     page_tokens: int = 16, spare_pages: int = 4, seed: int = 5,
                     perm_seed: int = 3):
    """Synthetic decode-attention problem over a shared, permuted page pool.

    Returns dict with q [B, nh, d] f16, k_tok/v_tok: lists of [L_b, nkv, d] f16
    (per-sequence logical token order), page_table [B, max_pages] int32 (-1 =
    unused), num_pages (pool size, including ``spare_pages`` never referenced).
    """
    lens = np.asarray(lens, dtype=np.int64)
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((batch, n_heads, head_dim), dtype=np.float32).astype(np.float16)
    k_tok, v_tok = [], []
    for b in range(batch):
        k_tok.append(rng.standard_normal((int(lens[b]), n_kv, head_dim), dtype=np.float32).astype(np.float16))
        v_tok.append(rng.standard_normal((int(lens[b]), n_kv, head_dim), dtype=np.float32).astype(np.float16))
    pages = [(int(L) + page_tokens - 1) // page_tokens for L in lens]
    max_pages = max(pages) if pages else 1
    total = int(sum(pages)) + spare_pages
    perm = page_permutation(total, perm_seed)
    pt = np.full((batch, max_pages), -1, dtype=np.int32)
    i = 0
    for b in range(batch):
        pt[b, :pages[b]] = perm[i:i + pages[b]]
        i += pages[b]
    return {"q": q, "k_tok": k_tok, "v_tok": v_tok, "page_table": pt,
            "num_pages": total, "lens": lens.astype(np.int32)}


def decode_page_tables(batch: int, max_pages: int, seed: int = 3, spare_pages: int = 0):
    """Page tables for a decode run: each sequence owns ``max_pages`` pages drawn
    from a randomly permuted pool of ``batch * max_pages + spare_pages`` pages."""
    total = batch * max_pages + spare_pages
    perm = page_permutation(total, seed)
    pt = perm[: batch * max_pages].reshape(batch, max_pages).astype(np.int32)
    return pt, total


def fill_device_normal(t, seed: int) -> None:
    """Fills a device float16 tensor in place with N(0, 1) values from torch's
    seeded device generator (stand-in contents for a pre-filled KV cache)."""
    import torch
    g = torch.Generator(device=t.device)
    g.manual_seed(int(seed))
    flat = t.view(-1)
    step = 1 << 28
    for i in range(0, flat.numel(), step):
        blk = flat[i:i + step]
        blk.copy_(torch.randn(blk.numel(), generator=g, device=t.device, dtype=torch.float32))
