#!/usr/bin/env python3
"""Decode benchmark of libnq on one MI355X: a Qwen2.5-Coder-7B-shaped model
with symmetric group-128 INT4 weights (fp16 scales) and fp16 activations,
random-init (synthetic) weights and prompts.

Headline (the printed JSON line): batch-1 greedy decode, 512-token random
prompt fed through the chunked prefill (timed: the time to first token), then
the step replayed as one HIP graph per token; ``value`` = tokens/s over exactly
--steps timed replays (after --warmup). At batch 1 the step is the persistent
whole-step kernel; the same tokens are then timed with one kernel per stage.
The same line also carries the persistent step's per-stage GEMV rates from its
own stage stamps (16 replays with the stamps on), batch 1 at contexts 4097 and
32767 in both step modes, the batch-8 decode (ragged contexts uniform in [128, 16384], 128 steps),
the attention sweep (the attention and combine kernels at batch 1 over 511,
4097 and 32767 tokens and at batch 8 over ragged lengths in [1, 32767]), the
W4A16 GEMV sweep at the 7B projection shapes (timed as graph replays: GB/s and
fraction of the 8 TB/s HBM peak; beside each, the INT8-activation variant with its quantisation fused
into the GEMV and as a separate kernel), the roofline of the dominant kernel
(at batch 1 the persistent step kernel, the only kernel of the timed graph),
the gate/up GEMV + SwiGLU (the largest kernel of the one-kernel-per-stage step)
and the CPU oracle timed on bounded samples.

Modes (for profiling runs): --mode steproof runs only the headline's batch-1
phase (the prefill, then --warmup and --steps replays of the persistent step);
--mode roofline launches only the gate/up GEMV of 28 distinct weight copies;
--mode limits measures the cost of a kernel boundary inside a graph and the
reuse of weights across consecutive GEMV launches; --mode copy runs a 1 GiB
device copy (the calibration for the FETCH_SIZE / WRITE_SIZE counters);
--mode stepkern runs a few batch-1 steps at context 520 with one kernel per
stage and as the persistent kernel, then the attention sweep (for per-kernel
counters); --mode stagetrace runs the batch-1 configuration's persistent step
with its stage stamps on and prints the per-stage timeline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode ms/token & tok/s (7B INT4, B=1/8); GEMV HBM GB/s as % of peak"
PEAK_HBM = 8.0e12
GEMV_ROTATION = {(3584, 4608): 64, (3584, 3584): 82, (3584, 37888): 8, (18944, 3584): 16}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_gate_up_swiglu_7b_b1_pmc.md")
KERNEL_SRC = os.path.join(ROOT, "w4a16_gemv_paged_amd", "csrc", "kernels.hip")
DEVICE_HDR = os.path.join(ROOT, "w4a16_gemv_paged_amd", "csrc", "device.hpp")
ATTN_MARK = b"// ============================================================== attention"
STEP_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_step_7b_b1_persistent_pmc.md")
STEP_SRCS = [os.path.join(ROOT, "w4a16_gemv_paged_amd", "csrc", n) for n in ("step.hip", "device.hpp", "common.hpp")]
STEP_KERNEL = "decode_step_kernel<128, 7> (persistent whole step, batch 1)"


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def gemv_bytes(k: int, n: int, b: int) -> int:
    """Algorithmic bytes of one W4A16 GEMV: INT4 codes + fp16 scales + fp16 in/out."""
    return k * n // 2 + k * n // 64 + 2 * b * (k + n)


def step_weight_bytes(shape) -> int:
    """Bytes one B=1 decode step must stream: packed weights, biases and norm
    gains of every layer, the LM head, the final gain and one embedding row."""
    H, I, nh, nkv, d, V = (shape.hidden, shape.intermediate, shape.n_heads, shape.n_kv_heads, shape.head_dim,
                           shape.vocab)
    qkv_n = (nh + 2 * nkv) * d
    pk = lambda n, k: n * k // 2 + n * (k // 128) * 2
    layer = pk(qkv_n, H) + 2 * qkv_n + pk(H, nh * d) + pk(2 * I, H) + pk(H, I) + 2 * 2 * H
    return shape.layers * layer + pk(V, H) + 2 * H + 2 * H


def kernel_sha() -> str:
    """Hash of the source the gate/up GEMV is built from: the GEMV part of
    kernels.hip (everything before the attention section) and device.hpp."""
    src = open(KERNEL_SRC, "rb").read()
    cut = src.find(ATTN_MARK)
    h = hashlib.sha256(src[:cut] if cut > 0 else src)
    h.update(open(DEVICE_HDR, "rb").read())
    return h.hexdigest()[:16]


def step_sha() -> str:
    """Hash of the source the persistent step kernel is built from."""
    h = hashlib.sha256()
    for path in STEP_SRCS:
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def read_traffic(path: str = TRAFFIC_FILE, sha=kernel_sha):
    """HBM traffic per launch from a committed PMC summary, if it was taken on
    the current kernel source."""
    if not os.path.exists(path):
        return None
    m = re.search(r"TRAFFIC_JSON:\s*(\{.*\})", open(path).read())
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("kernel_sha") != sha():
        return None
    return d.get("traffic_bytes_per_launch")


def time_launches(fn, launches: int, stream, reps: int = 1):
    """Per-launch durations from HIP events recorded around each launch on
    ``stream``; returns (mean seconds per launch, back-to-back seconds per launch)."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(launches * reps)]
    stream.synchronize()
    i = 0
    for _ in range(reps):
        for j in range(launches):
            evs[i][0].record(stream)
            fn(j)
            evs[i][1].record(stream)
            i += 1
    stream.synchronize()
    per = [a.elapsed_time(b) * 1e-3 for a, b in evs]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        for j in range(launches):
            fn(j)
    e1.record(stream)
    stream.synchronize()
    return sum(per) / len(per), e0.elapsed_time(e1) * 1e-3 / (launches * reps)


def time_graph(fn, launches: int, stream, reps: int = 1) -> float:
    """Seconds per launch of ``reps`` x ``launches`` calls captured in one HIP
    graph and replayed twice (HIP events on ``stream``): the kernels' own
    time, without the host's per-call overhead."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(reps):
            for j in range(launches):
                fn(j)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e-3 / (2 * reps * launches)


PEAK_MFMA_F16 = 2.5e15   # MI355X dense fp16 matrix peak


def ttft_block(shape, prompt: int, ms: float, ms_per_token: float) -> dict:
    """Time to first token of the chunked prefill (one chunk of ``prompt`` rows)
    beside feeding the same prompt through the decode step one token at a time.
    The projections of a prompt row cost 2 flops per weight; the attention adds
    4 * d flops per (query head, earlier position) pair."""
    H, I, nh, nkv, d = shape.hidden, shape.intermediate, shape.n_heads, shape.n_kv_heads, shape.head_dim
    weights = H * (nh + 2 * nkv) * d + nh * d * H + 2 * H * I + I * H
    gemm_flop = 2 * weights * prompt * shape.layers
    attn_flop = 4 * d * nh * shape.layers * prompt * (prompt + 1) / 2
    return {"prompt_tokens": prompt, "chunk": prompt, "ms": round(ms, 3),
            "prefill_tok_s": round(prompt / ms * 1e3, 1),
            "kernels": 7 * shape.layers + 2,
            "flop": int(gemm_flop + attn_flop),
            "tflops": round((gemm_flop + attn_flop) / (ms * 1e-3) / 1e12, 1),
            "mfma_frac": round((gemm_flop + attn_flop) / (ms * 1e-3) / PEAK_MFMA_F16, 4),
            "token_by_token_ms": round(prompt * ms_per_token, 2)}


def gate_up_roofline(layers, hidden: int, inter: int, stream, reps: int = 10):
    """Times the gate/up GEMV + SwiGLU launch of the decode step (B=1, RMSNorm
    prologue) over the given per-layer (packed, gain) pairs."""
    import numpy as np
    import torch
    import synth
    import w4a16_gemv_paged_amd as nq
    x = torch.from_numpy(synth.activations(1, hidden, seed=1).view(np.int16)).cuda()
    y = torch.empty(1, inter, dtype=torch.float16, device="cuda")
    sid = stream.cuda_stream

    def launch(j):
        packed, gain = layers[j % len(layers)]
        nq.nq_gemv_w4a16(packed, 2 * inter, hidden, nq.NQ_MAT_GATE_UP, 0, 1, x, gain, 1e-6, None, y,
                         nq.NQ_EPI_SWIGLU_F16, sid)

    for j in range(len(layers)):
        launch(j)
    mean_s, b2b_s = time_launches(launch, len(layers), stream, reps)
    unit_bytes = gemv_bytes(hidden, 2 * inter, 1)
    traffic = read_traffic()
    return {
        "kernel": "gemv_w4a16_kernel<1, SWIGLU> (gate/up GEMV + SwiGLU, RMSNorm prologue), K=3584 N=37888 B=1",
        "bound": "hbm", "achieved": round(unit_bytes / b2b_s / 1e9, 1), "peak": 8000.0, "unit": "GB/s",
        "frac": round(unit_bytes / b2b_s / PEAK_HBM, 4),
        "traffic": traffic,
        "algorithmic_bytes_per_launch": unit_bytes,
        "mean_launch_us": round(mean_s * 1e6, 3),
        "back_to_back_us": round(b2b_s * 1e6, 3),
        "launches_timed": len(layers) * reps,
    }


def gemv_sweep(stream):
    import numpy as np
    import torch
    import synth
    import w4a16_gemv_paged_amd as nq
    out = []
    sid = stream.cuda_stream
    for (k, n), copies in GEMV_ROTATION.items():
        packed = nq.nq_pack_weights(synth.gemv_weight(k, n, seed=0))
        bufs = [torch.from_numpy(packed).cuda() for _ in range(copies)]  # >= 512 MB of distinct addresses
        for b in (1, 4):
            x = torch.from_numpy(synth.activations(b, k, seed=1).view(np.int16)).cuda()
            y = torch.empty(b, n, dtype=torch.float16, device="cuda")
            fn = lambda j: nq.nq_gemv_w4a16(bufs[j], n, k, 0, 0, b, x, None, 1e-6, None, y, 0, sid)
            for j in range(copies):
                fn(j)
            mean_s, eager_s = time_launches(fn, copies, stream, reps=max(1, 256 // copies))
            b2b_s = time_graph(fn, copies, stream, reps=max(1, 256 // copies))
            nb = gemv_bytes(k, n, b)
            row = {"K": k, "N": n, "B": b, "bytes": nb, "us": round(b2b_s * 1e6, 2),
                   "GBs": round(nb / b2b_s / 1e9, 1), "frac": round(nb / b2b_s / PEAK_HBM, 4),
                   "eager_us": round(eager_s * 1e6, 2), "event_pair_us": round(mean_s * 1e6, 2)}
            # the INT8-activation variant on the same weights: a separate quantise
            # kernel before each GEMV, and quantisation in the GEMV prologue
            xq = torch.empty(nq.nq_a8_bytes(b, k), dtype=torch.uint8, device="cuda")
            yf = torch.empty(b, n, dtype=torch.float16, device="cuda")
            fq = lambda j: nq.nq_quantize_a8(x, b, k, xq, sid)
            f2 = lambda j: (nq.nq_quantize_a8(x, b, k, xq, sid),
                            nq.nq_gemv_w4a8(bufs[j], n, k, 0, 0, b, x, xq, None, yf, 0, sid))
            reps = max(1, 256 // copies)
            row["w4a8_quantize_us"] = round(time_launches(fq, copies, stream, reps=reps)[1] * 1e6, 2)
            row["w4a8_two_kernels_us"] = round(time_launches(f2, copies, stream, reps=reps)[1] * 1e6, 2)
            row["w4a8_fused_us"] = None
            try:
                ff = lambda j: nq.nq_gemv_w4a8(bufs[j], n, k, 0, 0, b, x, None, None, yf, 0, sid)
                ff(0)
                row["w4a8_fused_us"] = round(time_launches(ff, copies, stream, reps=reps)[1] * 1e6, 2)
            except nq.NQError:
                pass   # the batch's K does not fit LDS for in-kernel quantisation
            out.append(row)
            log(f"gemv K={k} N={n} B={b}: {b2b_s * 1e6:.2f} us {nb / b2b_s / 1e9:.0f} GB/s; W4A8 fused "
                f"{row['w4a8_fused_us']} us, quantise + W4A8 {row['w4a8_two_kernels_us']} us")
        del bufs
    agg = {}
    for b in (1, 4):
        rows = [r for r in out if r["B"] == b]
        tb = sum(r["bytes"] for r in rows)
        tt = sum(r["bytes"] / (r["GBs"] * 1e9) for r in rows)
        agg[f"B{b}"] = {"GBs": round(tb / tt / 1e9, 1), "frac": round(tb / tt / PEAK_HBM, 4)}
    return out, agg


def attn_bytes(shape, lens) -> int:
    """Algorithmic bytes of one layer's decode attention: the K and V rows of
    every cached token (fp16), q in and the output out (fp16)."""
    kv = 2 * shape.n_kv_heads * shape.head_dim * 2 * int(sum(int(x) for x in lens))
    return kv + 2 * 2 * len(lens) * shape.n_heads * shape.head_dim


def attention_sweep(dm, shape, stream, reps: int = 4):
    """The decode attention and combine kernels of one layer (nq_attn_decode),
    timed back to back over the 28 layers of a random-filled pool (every call a
    different layer's pages, as in the step): batch 1 at 511, 4097 and 32767
    cached tokens, and batch 8 over lengths uniform in [1, 32767] (seed 6)."""
    import numpy as np
    import torch
    import synth
    import w4a16_gemv_paged_amd as nq
    from w4a16_gemv_paged_amd.engine import KVCache
    cases = [("B1_511", [511]), ("B1_4097", [4097]), ("B1_32767", [32767]),
             ("B8_ragged_1_32767_seed6", synth.ragged_lengths(8, 1, 32767, seed=6).tolist())]
    sid = stream.cuda_stream
    out = []
    for name, lens in cases:
        B = len(lens)
        max_pages = max((int(x) + 15) // 16 for x in lens)
        pt, total = synth.decode_page_tables(B, max_pages, seed=3)
        kv = KVCache(dm, total, poison=False)
        synth.fill_device_normal(kv.pool.view(torch.float16), seed=7)
        q = torch.randn(B, shape.n_heads, shape.head_dim, dtype=torch.float16, device="cuda")
        o = torch.empty_like(q)
        ptd = torch.from_numpy(pt).cuda()
        ld = torch.tensor(lens, dtype=torch.int32, device="cuda")
        wsb = nq.nq_attn_workspace_bytes(dm.cfg, B, max_pages)
        ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        fn = lambda j: nq.nq_attn_decode(kv.handle, j % shape.layers, B, q, ptd, max_pages, ld, o, ws, wsb, err,
                                         stream=stream)
        for j in range(shape.layers):
            fn(j)
        mean_s, b2b_s = time_launches(fn, shape.layers, stream, reps=reps)
        nq.nq_check_device_error(err)
        nb = attn_bytes(shape, lens)
        out.append({"case": name, "batch": B, "lens": [int(x) for x in lens], "max_pages": max_pages,
                    "bytes": nb, "us": round(b2b_s * 1e6, 2), "GBs": round(nb / b2b_s / 1e9, 1),
                    "frac": round(nb / b2b_s / PEAK_HBM, 4), "event_pair_us": round(mean_s * 1e6, 2)})
        log(f"attention {name}: {b2b_s * 1e6:.2f} us, {nb / b2b_s / 1e9:.0f} GB/s")
        kv.close()
        del kv, ws
        torch.cuda.empty_cache()
    return out


def context_sweep(dm, shape, stream, contexts=(4097, 32700), steps: int = 32):
    """Batch-1 decode at long contexts over a random-filled pool (timing only:
    the tokens are not a real continuation), in both step modes: ms per token
    over ``steps`` graph replays."""
    import torch
    import synth
    from w4a16_gemv_paged_amd.engine import KVCache, Stepper
    out = []
    for ctx in contexts:
        max_pages = (ctx + steps + 8 + 15) // 16
        pt, total = synth.decode_page_tables(1, max_pages, seed=3)
        kv = KVCache(dm, total, poison=False)
        synth.fill_device_normal(kv.pool.view(torch.float16), seed=7)
        row = {"context": ctx}
        for mode in ("auto", "kernels"):
            dm.set_step_mode(mode)
            st = Stepper(dm, kv, pt)
            with torch.cuda.stream(stream):
                st.set_pos([ctx])
                st.set_tokens([17])
                n = st.capture(stream)
                for _ in range(4):
                    st.replay(stream)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(steps):
                    st.replay(stream)
                e1.record(stream)
                torch.cuda.synchronize()
                st.check(stream)
            row[mode] = {"ms_per_token": round(e0.elapsed_time(e1) / steps, 4), "kernels_per_step": n}
            st.close()
            del st
        dm.set_step_mode("auto")
        log(f"B=1 at context {ctx}: persistent {row['auto']['ms_per_token']} ms, "
            f"kernels {row['kernels']['ms_per_token']} ms")
        out.append(row)
        kv.close()
        del kv
        torch.cuda.empty_cache()
    return out


STAGE_EVENTS = ["QKV partials in", "QKV hand-off: arrive", "QKV hand-off: all arrived", "attention partials in",
                "attention hand-off: arrive", "attention hand-off: all arrived", "O partials in", "O hand-off: arrive",
                "O hand-off: all arrived", "gate/up partials in", "gate/up hand-off: arrive",
                "gate/up hand-off: all arrived", "down partials in", "down hand-off: arrive", "down hand-off: all arrived",
                "next stage's input staged"]


# (stage, event that starts it: the hand-off before it; None = the previous
# layer's last hand-off, event that ends it: its partial sums in LDS)
GEMV_STAGES = [("QKV", None, 0, "qkv"), ("O", 5, 6, "o"), ("gate/up", 8, 9, "gate_up"), ("down", 11, 12, "down")]


def stage_trace(shape, stream, steps: int = 16, dm=None):
    """The batch-1 configuration (512-token prompt through the prefill, 52-page
    table) stepped with the persistent kernel's stage stamps on: per event, the
    time since the layer's start (the previous layer's last event), median
    over steps and layers 1..L-2 of the median and of the maximum over the 256
    workgroups; the layer, LM head and whole-step durations. Per GEMV stage:
    from the first workgroup's start of the stage (the hand-off before it) to
    the last workgroup's partial sums in LDS, which takes in the stage's input
    staging and its weight stream, median over steps and layers; its bytes
    and rate."""
    import numpy as np
    import torch
    import synth
    from w4a16_gemv_paged_amd.engine import DeviceModel, KVCache, Stepper, Prefill
    own = dm is None
    if own:
        head = synth.head_params(shape, seed=0)
        dm = DeviceModel(shape, lambda l: synth.layer_params(shape, l, seed=0), head, max_batch=8, max_pos=32768)
    P, L = 512, shape.layers
    pt, total = synth.decode_page_tables(1, 52, seed=3)
    kv = KVCache(dm, total, poison=False)
    st = Stepper(dm, kv, pt, hist_len=P + steps + 16)
    buf = torch.full((256 * (L + 1) * 16,), -1, dtype=torch.int64, device="cuda")
    samples = []
    with torch.cuda.stream(stream):
        pf = Prefill(dm, kv, P)
        pf.run(synth.prompt_ids(P, shape.vocab, seed=2), st.page_table[0], 0, next_token=st.tokens[0:1],
               pos_out=st.pos[0:1], stream=stream)
        pf.check(stream)
        dm.set_step_trace(buf)
        st.capture(stream)
        for i in range(steps + 4):
            st.replay(stream)
            torch.cuda.synchronize()
            if i >= 4:
                samples.append(buf.cpu().numpy().reshape(256, L + 1, 16).copy())
        st.check(stream)
        dm.set_step_trace(None)
    st.close()
    kv.close()
    if own:
        dm.close()
    ev_med = [[] for _ in range(16)]
    span = {name: [] for name, _, _, _ in GEMV_STAGES}
    ev_max = [[] for _ in range(16)]
    layer_us, lm_us, step_us = [], [], []
    for t in samples:
        t = t.astype(np.float64) / 100.0                      # 100 MHz counter -> us
        for l in range(1, L - 1):
            start = t[:, l - 1, 15]
            for e in range(16):
                d = t[:, l, e] - start
                ev_med[e].append(float(np.median(d)))
                ev_max[e].append(float(np.max(d)))
            layer_us.append(float(np.median(t[:, l, 15] - t[:, l - 1, 15])))
            for name, e0, e1, _ in GEMV_STAGES:
                t0 = t[:, l - 1, 14] if e0 is None else t[:, l, e0]
                span[name].append(float(np.max(t[:, l, e1]) - np.min(t0)))
        lm_us.append(float(np.median(t[:, L, 2] - t[:, L - 1, 15])))
        step_us.append(float(np.max(t[:, L, 2]) - np.min(t[:, L, 0])))
    med = lambda v: round(float(np.median(v)), 2)
    H, I, nh, nkv, d = shape.hidden, shape.intermediate, shape.n_heads, shape.n_kv_heads, shape.head_dim
    kn = {"qkv": (H, (nh + 2 * nkv) * d), "o": (nh * d, H), "gate_up": (H, 2 * I), "down": (I, H)}
    stages = []
    for name, _, _, key in GEMV_STAGES:
        k, n = kn[key]
        nb, us = gemv_bytes(k, n, 1), med(span[name])
        stages.append({"stage": name, "K": k, "N": n, "bytes": nb, "us": us, "GBs": round(nb / us / 1e3, 1),
                       "frac": round(nb / us / 8e6, 4)})
    tb, tt = sum(x["bytes"] for x in stages), sum(x["us"] for x in stages)
    return {"mode": "stagetrace",
            "gemv_stages": stages,
            "gemv_stages_aggregate": {"GBs": round(tb / tt / 1e3, 1), "frac": round(tb / tt / 8e6, 4)}, "steps": len(samples), "context": [P + 4, P + 4 + len(samples)],
            "events": [{"event": STAGE_EVENTS[e], "us_since_layer_start_median_wg": med(ev_med[e]),
                        "us_since_layer_start_slowest_wg": med(ev_max[e])} for e in range(16)],
            "layer_us": med(layer_us), "lm_head_and_greedy_us": med(lm_us), "step_us": med(step_us),
            "first_layer_start_us": med([float(np.median(t[:, 0, 0] - t[:, L, 0])) / 100.0 for t in samples])}


def host_info() -> dict:
    """BLAS the oracle's NumPy links, host RAM and this process's peak resident set."""
    import resource
    import numpy as np
    info = {"blas": None, "ram_total_gb": None,
            "peak_rss_gb": round(resource.getrusage(resource.RUSAGE_SELF).ru_maxrss / 2**20, 2)}
    try:
        cfg = np.show_config(mode="dicts")
        blas = cfg.get("Build Dependencies", {}).get("blas", {})
        info["blas"] = f"{blas.get('name')} {blas.get('version')}"
    except Exception:
        pass
    try:
        import psutil
        info["ram_total_gb"] = round(psutil.virtual_memory().total / 2**30, 1)
    except Exception:
        pass
    return info


def cpu_rows(shape, budget_s: float = 4.0) -> dict:
    """The oracle's building blocks timed on the host cores (median of up to 5
    runs within ``budget_s`` each): the W4A16 GEMV (dequantise + float64
    product) at the four projection shapes for B = 1 and 4, the decode
    attention of one layer at 511, 4097 and 32767 cached tokens, and one
    decode step of the tiny config (all layers and the LM head)."""
    import numpy as np
    import synth
    import oracle
    from oracle.model import OracleModel, ContiguousKV, decode_step

    def med(fn):
        ts = []
        t_end = time.perf_counter() + budget_s
        while len(ts) < 5 and (len(ts) < 1 or time.perf_counter() < t_end):
            t = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t)
        return sorted(ts)[len(ts) // 2], len(ts)

    rows = {"gemv": [], "attention": [], "tiny": None}
    for (k, n) in GEMV_ROTATION:
        q, s16 = oracle.quantize_w4(synth.gemv_weight(k, n, seed=0))
        for b in (1, 4):
            x = synth.activations(b, k, seed=1)
            t, m = med(lambda: oracle.gemv_w4a16(q, s16, x))
            rows["gemv"].append({"K": k, "N": n, "B": b, "s": round(t, 4), "runs": m})
        del q, s16
    d, nh, nkv = shape.head_dim, shape.n_heads, shape.n_kv_heads
    rng = np.random.default_rng(5)
    for L in (511, 4097, 32767):
        qv = rng.standard_normal((nh, d)).astype(np.float16)
        kk = rng.standard_normal((L, nkv, d)).astype(np.float16)
        vv = rng.standard_normal((L, nkv, d)).astype(np.float16)
        t, m = med(lambda: oracle.attend(qv, kk, vv))
        rows["attention"].append({"len": L, "s": round(t, 4), "runs": m})
    tiny = synth.TINY
    layers = [synth.layer_params(tiny, i, seed=0) for i in range(tiny.layers)]
    om = OracleModel.build(tiny, layers, synth.head_params(tiny, seed=0))
    cache = ContiguousKV(tiny.layers, tiny.n_kv_heads, tiny.head_dim)
    pos = [0]

    def tiny_step():
        decode_step(om, [cache], [17], [pos[0]])
        pos[0] += 1

    t, m = med(tiny_step)
    rows["tiny"] = {"config": tiny.name, "s_per_token": round(t, 4), "runs": m,
                    "context": "0..%d (a fresh contiguous cache)" % (m - 1)}
    rows["cores"] = len(os.sched_getaffinity(0))
    rows.update(host_info())
    return rows


def cpu_baseline(shape, head, sample_layers: int = 1, head_frac: int = 8, budget_s: float = 10.0, ctx: int = 512):
    """The oracle's decode step timed on the host cores on a bounded sample:
    ``sample_layers`` of the layers and 1/``head_frac`` of the LM-head rows, at
    context ``ctx`` with a synthetic (random) contiguous cache, stepped for about
    ``budget_s`` seconds (at least 3 steps); the per-token time is scaled to the
    whole model (layers x L + head slice x head_frac)."""
    import numpy as np
    import synth
    import oracle
    from oracle.model import Dims, OracleLayer, OracleHead, ContiguousKV, layer_decode, head_logits, OracleModel
    cores = len(os.sched_getaffinity(0))
    rows = shape.vocab // head_frac
    dims = Dims(shape.hidden, shape.intermediate, shape.n_heads, shape.n_kv_heads, shape.head_dim, rows,
                shape.rms_eps, shape.rope_theta)
    t0 = time.time()
    layers = [OracleLayer(synth.layer_params(shape, i, seed=0)) for i in range(sample_layers)]
    for L in layers:
        for nm in ("qkv", "o", "gu", "d"):
            L.w(nm)
    oh = OracleHead({"embed": head["embed"], "lm_head": head["lm_head"][:rows], "g_final": head["g_final"]})
    oh.w_lm()
    model = OracleModel(dims, layers, oh)
    rng = np.random.default_rng(9)
    cache = ContiguousKV(sample_layers, shape.n_kv_heads, shape.head_dim)
    for li in range(sample_layers):
        cache.k[li] = rng.standard_normal((ctx, shape.n_kv_heads, shape.head_dim)).astype(np.float16)
        cache.v[li] = rng.standard_normal((ctx, shape.n_kv_heads, shape.head_dim)).astype(np.float16)
    setup = time.time() - t0
    t_layers, t_head = [], []
    tok = 17
    t_all = time.perf_counter()
    s = 0
    while s < 3 or (time.perf_counter() - t_all < budget_s and s < 4096):
        pos = ctx + s
        s += 1
        h = oh.embed[tok]
        t1 = time.perf_counter()
        for li, L in enumerate(layers):
            h = layer_decode(L, dims, h, pos, lambda k, v, li=li: cache.append(li, pos, k, v),
                             lambda n, li=li: cache.get(li, n))
        t2 = time.perf_counter()
        z = head_logits(model, h)
        tok = oracle.argmax_lowest(z)
        t3 = time.perf_counter()
        t_layers.append((t2 - t1) / sample_layers)
        t_head.append(t3 - t2)
    timed = time.perf_counter() - t_all
    per_layer = sorted(t_layers)[len(t_layers) // 2]
    per_head = sorted(t_head)[len(t_head) // 2]
    per_token = per_layer * shape.layers + per_head * head_frac
    return {"value": round(1.0 / per_token, 4), "unit": "tok/s", "cores": cores, "kind": "oracle",
            "sample": (f"oracle decode step (NumPy float64 on dequantised weights) over {sample_layers} of "
                       f"{shape.layers} layers and 1/{head_frac} of the LM-head rows, context {ctx} with a "
                       f"synthetic contiguous cache, median of {s} steps; per-token time = layer time x "
                       f"{shape.layers} + head-slice time x {head_frac}"),
            "s_per_token": round(per_token, 3), "timed_s": round(timed, 2), "setup_s": round(setup, 1)}


def limits(shape, stream, launches: int = 256, replays: int = 8) -> dict:
    """Fixed costs and cache reuse, measured with the library's own kernels.
    (1) The per-launch floor: ``launches`` KV appends of one token (one
    64-thread workgroup writing 4 KiB) captured in one HIP graph and replayed
    ``replays`` times; the graph time per launch against the kernel's own
    duration (from a kernel trace of this mode) is the cost of a kernel
    boundary. (2) Reuse across consecutive launches: the QKV GEMV (8.5 MB, less
    than the eight 4 MB L2s together) and the gate/up GEMV (70 MB, less than
    the 256 MB last-level cache) back to back on one copy of the weights,
    against a rotation over distinct copies (>= 512 MB, nothing reused)."""
    import numpy as np
    import torch
    import synth
    import w4a16_gemv_paged_amd as nq
    sid = stream.cuda_stream
    cfg = nq.NQConfig.from_shape(shape, 1, 4096)
    npages = 8
    nbytes = nq.nq_kv_pool_bytes(cfg, npages)
    pool = torch.zeros(nbytes // 2, dtype=torch.int16, device="cuda")
    kv = nq.nq_kv_alloc(cfg, pool, nbytes, npages)
    pt = torch.arange(npages, dtype=torch.int32, device="cuda").view(1, npages)
    pos = torch.tensor([5], dtype=torch.int32, device="cuda")
    k = torch.randn(1, shape.n_kv_heads, shape.head_dim, device="cuda").half()
    v = torch.randn(1, shape.n_kv_heads, shape.head_dim, device="cuda").half()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    append = lambda: nq.nq_kv_append(kv, 0, 1, pt, npages, pos, k, v, err, stream=sid)
    with torch.cuda.stream(stream):
        append()
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(launches):
                append()
        g.replay()
        stream.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(replays):
            g.replay()
        e1.record(stream)
        stream.synchronize()
    nq.nq_check_device_error(err)
    floor_us = e0.elapsed_time(e1) * 1e3 / (launches * replays)
    del g
    nq.nq_kv_free(kv)
    log(f"kernel floor: {floor_us:.2f} us per graph-launched kernel")
    reuse = []
    for (kk, n), copies in (((3584, 4608), 64), ((3584, 37888), 8)):
        packed = nq.nq_pack_weights(synth.gemv_weight(kk, n, seed=0))
        bufs = [torch.from_numpy(packed).cuda() for _ in range(copies)]
        x = torch.from_numpy(synth.activations(1, kk, seed=1).view(np.int16)).cuda()
        y = torch.empty(1, n, dtype=torch.float16, device="cuda")
        gemv = lambda j: nq.nq_gemv_w4a16(bufs[j % copies], n, kk, 0, 0, 1, x, None, 1e-6, None, y, 0, sid)
        with torch.cuda.stream(stream):
            for j in range(copies):
                gemv(j)
            _, rot = time_launches(gemv, copies, stream, reps=max(1, 256 // copies))
            _, same = time_launches(lambda j: gemv(0), copies, stream, reps=max(1, 256 // copies))
        nb = gemv_bytes(kk, n, 1)
        reuse.append({"K": kk, "N": n, "bytes": nb, "distinct_copies_us": round(rot * 1e6, 2),
                      "same_copy_us": round(same * 1e6, 2), "distinct_GBs": round(nb / rot / 1e9, 1),
                      "same_GBs": round(nb / same / 1e9, 1)})
        log(f"GEMV {kk}x{n}: distinct copies {rot * 1e6:.2f} us, same copy {same * 1e6:.2f} us")
        del bufs
        torch.cuda.empty_cache()
    return {"mode": "limits", "graph_launches": launches, "replays": replays,
            "kv_append_graph_us_per_launch": round(floor_us, 3), "gemv_reuse": reuse}


def b1_phase(dm, shape, stream, W: int, K: int, ttft_reps: int = 6) -> dict:
    """The headline: a 512-token random prompt through the chunked prefill (time
    to first token, median of ``ttft_reps`` - 1 repeats on the same pages), then
    the step captured as one HIP graph, W untimed and K timed replays (host clock
    and HIP events on the replay stream), then 16 eager steps."""
    import numpy as np
    import torch
    import synth
    from w4a16_gemv_paged_amd.engine import KVCache, Stepper, Prefill
    P = 512
    prompt = synth.prompt_ids(P, shape.vocab, seed=2)
    need = P + W + K + 64
    max_pages = (need + 15) // 16
    pt, total = synth.decode_page_tables(1, max_pages, seed=3)
    kv1 = KVCache(dm, total, poison=False)
    st = Stepper(dm, kv1, pt, hist_len=need + 1)
    with torch.cuda.stream(stream):
        # the prefill leaves the first generated token and its position in the
        # step's device buffers; the repeats rewrite the same pages
        pf = Prefill(dm, kv1, P)
        row = st.page_table[0]
        ttft = []
        for r in range(ttft_reps):
            ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ea.record(stream)
            pf.run(prompt, row, 0, next_token=st.tokens[0:1], pos_out=st.pos[0:1], stream=stream)
            eb.record(stream)
            torch.cuda.synchronize()
            if r > 0:
                ttft.append(ea.elapsed_time(eb))
        pf.check(stream)
        ttft_ms = float(np.median(ttft))
        del pf
        n_kernels = st.capture(stream)
        log(f"prefill of {P} tokens (TTFT): {ttft_ms:.2f} ms; captured the step: {n_kernels} kernels")
        for _ in range(W):
            st.replay(stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t1 = time.perf_counter()
        e0.record(stream)
        for _ in range(K):
            st.replay(stream)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t1
        st.check(stream)
        # eager launches of the same step (the pages' eager vs graph comparison)
        ne = 16
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for _ in range(ne):
            st.step(stream)
        torch.cuda.synchronize()
        ms_eager = (time.perf_counter() - t2) * 1e3 / ne
        st.check(stream)
    gen = st.hist.cpu().numpy()[0][P + 1:P + 1 + W + K]
    st.close()
    kv1.close()
    # the step at position p reads the K/V rows of p + 1 tokens; the timed
    # replays run at positions P + W .. P + W + K - 1
    lens = [P + W + i + 1 for i in range(K)]
    alg = step_weight_bytes(shape) + shape.layers * attn_bytes(shape, lens) / K
    return {"P": P, "prompt": prompt, "pt": pt, "total": total, "need": need, "ttft_ms": ttft_ms,
            "n_kernels": n_kernels, "ctx0": P + W, "ms": wall * 1e3 / K, "ms_events": e0.elapsed_time(e1) / K,
            "ms_eager": ms_eager, "gen": gen, "alg_bytes_per_step": int(round(alg))}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=248)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--mode", choices=["full", "steproof", "limits", "roofline", "copy", "stepkern", "stagetrace"], default="full")
    ap.add_argument("--skip-b8", action="store_true")
    ap.add_argument("--skip-sweep", action="store_true")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--b8-steps", type=int, default=128)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build measures one GPU only (the decode step runs on a single MI355X; there is "
              "no multi-GPU mode). Run it with --gpus 1.", file=sys.stderr, flush=True)
        return 2

    import numpy as np
    import torch
    import synth
    import w4a16_gemv_paged_amd as nq
    from w4a16_gemv_paged_amd.engine import DeviceModel, KVCache, Stepper, Prefill

    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    shape = synth.QWEN7B

    if args.mode == "copy":
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            for _ in range(3):
                dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy", "bytes_read_per_copy": n, "bytes_written_per_copy": n}), flush=True)
        return 0

    if args.mode == "roofline":
        packed = nq.nq_pack_weights(np.concatenate([synth.gemv_weight(3584, 18944, seed=0, copy=1),
                                                    synth.gemv_weight(3584, 18944, seed=0, copy=2)]),
                                    nq.NQ_MAT_GATE_UP)
        gain = torch.from_numpy((1 + 0.02 * np.random.default_rng(3).standard_normal(3584))
                                .astype(np.float16).view(np.int16)).cuda()
        layers = [(torch.from_numpy(packed).cuda(), gain) for _ in range(shape.layers)]
        with torch.cuda.stream(stream):
            r = gate_up_roofline(layers, shape.hidden, shape.intermediate, stream, reps=4)
        print(json.dumps({"mode": "roofline", "roofline": r}), flush=True)
        return 0

    if args.mode == "limits":
        print(json.dumps(limits(shape, stream)), flush=True)
        return 0

    if args.mode == "stagetrace":
        print(json.dumps(stage_trace(shape, stream)), flush=True)
        return 0

    if args.mode == "stepkern":
        head = synth.head_params(shape, seed=0)
        dm = DeviceModel(shape, lambda l: synth.layer_params(shape, l, seed=0), head, max_batch=8, max_pos=32768)
        pt, total = synth.decode_page_tables(1, 40, seed=3)
        kv = KVCache(dm, total, poison=False)
        synth.fill_device_normal(kv.pool.view(torch.float16), seed=7)
        for mode in ("kernels", "auto"):
            dm.set_step_mode(mode)
            st = Stepper(dm, kv, pt)
            st.set_pos([520])
            st.set_tokens([17])
            with torch.cuda.stream(stream):
                for _ in range(4):
                    st.step(stream)
                torch.cuda.synchronize()
                st.check(stream)
            st.close()
        kv.close()
        with torch.cuda.stream(stream):
            att = attention_sweep(dm, shape, stream, reps=1)
        print(json.dumps({"mode": "stepkern", "steps_per_mode": 4, "context": 520, "attention": att}), flush=True)
        return 0

    if args.mode == "steproof":
        head = synth.head_params(shape, seed=0)
        dm = DeviceModel(shape, lambda l: synth.layer_params(shape, l, seed=0), head, max_batch=8, max_pos=32768)
        r1 = b1_phase(dm, shape, stream, args.warmup, args.steps, ttft_reps=1)
        dm.close()
        print(json.dumps({"mode": "steproof", "kernel": STEP_KERNEL, "kernel_sha": step_sha(),
                          "warmup": args.warmup, "steps": args.steps, "context_during_timing":
                          [r1["ctx0"], r1["ctx0"] + args.steps], "ms_per_token_events": round(r1["ms_events"], 4),
                          "alg_bytes_per_step": r1["alg_bytes_per_step"]}), flush=True)
        return 0

    # ------------------------------------------------------------------ model
    t0 = time.time()
    log("drawing and packing the 7B-shaped weights")
    head = synth.head_params(shape, seed=0)
    dm = DeviceModel(shape, lambda l: synth.layer_params(shape, l, seed=0), head, max_batch=8, max_pos=32768)
    torch.cuda.synchronize()
    log(f"model ready in {time.time() - t0:.1f} s ({dm.weight_bytes() / 1e9:.2f} GB on device)")

    # ------------------------------------------------------------------ B = 1
    W, K = args.warmup, args.steps
    r1 = b1_phase(dm, shape, stream, W, K)
    P, prompt, pt, total, need = r1["P"], r1["prompt"], r1["pt"], r1["total"], r1["need"]
    ms_b1, ms_b1_events, ms_eager, ttft_ms, n_kernels, ctx0, gen = (
        r1["ms"], r1["ms_events"], r1["ms_eager"], r1["ttft_ms"], r1["n_kernels"], r1["ctx0"], r1["gen"])
    log(f"B=1: {ms_b1:.3f} ms/token ({1e3 / ms_b1:.1f} tok/s), eager {ms_eager:.3f} ms/token; "
        f"first tokens {gen[:8].tolist()}")
    # the same prompt, page table and timed contexts with one kernel per stage
    dm.set_step_mode("kernels")
    kv1 = KVCache(dm, total, poison=False)
    st = Stepper(dm, kv1, pt, hist_len=need + 1)
    with torch.cuda.stream(stream):
        pf = Prefill(dm, kv1, P)
        pf.run(prompt, st.page_table[0], 0, next_token=st.tokens[0:1], pos_out=st.pos[0:1], stream=stream)
        pf.check(stream)
        del pf
        n_kernels_k = st.capture(stream)
        for _ in range(W):
            st.replay(stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(K):
            st.replay(stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_b1_k = e0.elapsed_time(e1) / K
        st.check(stream)
    gen_k = st.hist.cpu().numpy()[0][P + 1:P + 1 + W + K]
    dm.set_step_mode("auto")
    b1_kernels = {"ms_per_token": round(ms_b1_k, 4), "tok_s": round(1e3 / ms_b1_k, 1), "kernels_per_step": n_kernels_k,
                  "context_during_timing": [ctx0, ctx0 + K],
                  "tokens_equal_to_persistent": int(np.sum(gen_k == gen)), "tokens_compared": int(len(gen))}
    log(f"B=1 with one kernel per stage ({n_kernels_k} kernels): {ms_b1_k:.3f} ms/token; "
        f"{b1_kernels['tokens_equal_to_persistent']}/{len(gen)} tokens as the persistent step's")
    st.close()
    kv1.close()
    del st, kv1
    # the persistent step's own stage stamps: per-stage GEMV rates in the product path
    stg = stage_trace(shape, stream, steps=16, dm=dm)
    log(f"persistent step stages: layer {stg['layer_us']} us; GEMV stages " +
        ", ".join(f"{x['stage']} {x['us']} us ({x['frac'] * 100:.0f}%)" for x in stg["gemv_stages"]) +
        f"; aggregate {stg['gemv_stages_aggregate']['frac'] * 100:.1f}% of 8 TB/s")

    # ------------------------------------------------------------------ roofline of the dominant kernel
    # At batch 1 the timed graph holds one kernel, the persistent step, so its
    # average launch duration is the replay time measured by the HIP events on
    # the replay stream, and its algorithmic bytes are the step's weights plus
    # every layer's K/V rows at the timed contexts.
    alg = r1["alg_bytes_per_step"]
    roof_step = {"kernel": STEP_KERNEL, "bound": "hbm",
                 "achieved": round(alg / (ms_b1_events * 1e-3) / 1e9, 1), "peak": 8000.0, "unit": "GB/s",
                 "frac": round(alg / (ms_b1_events * 1e-3) / PEAK_HBM, 4),
                 "traffic": read_traffic(STEP_TRAFFIC_FILE, step_sha),
                 "algorithmic_bytes_per_launch": alg, "mean_launch_us": round(ms_b1_events * 1e3, 2),
                 "launches_timed": K}
    log(f"persistent step kernel: {roof_step['achieved']} GB/s ({roof_step['frac'] * 100:.1f}% of 8 TB/s)")
    with torch.cuda.stream(stream):
        roof = gate_up_roofline([(L["gate_up"], L["g2"]) for L in dm.layers], shape.hidden, shape.intermediate,
                                stream, reps=10)
    log(f"gate/up GEMV: {roof['back_to_back_us']} us/launch, {roof['achieved']} GB/s ({roof['frac'] * 100:.1f}%)")

    # ------------------------------------------------------------------ long contexts, attention
    ctx_sweep = att_sweep = None
    if not args.skip_sweep:
        ctx_sweep = context_sweep(dm, shape, stream)
        with torch.cuda.stream(stream):
            att_sweep = attention_sweep(dm, shape, stream)

    # ------------------------------------------------------------------ B = 8
    b8 = None
    if not args.skip_b8:
        lens = synth.ragged_lengths(8, 128, 16384, seed=4)
        max_pages8 = 2048
        pt8, total8 = synth.decode_page_tables(8, max_pages8, seed=3)
        kv8 = KVCache(dm, total8, poison=False)
        synth.fill_device_normal(kv8.pool.view(torch.float16), seed=7)
        st8 = Stepper(dm, kv8, pt8)
        with torch.cuda.stream(stream):
            st8.set_pos(lens)
            st8.set_tokens(synth.prompt_ids(8, shape.vocab, seed=8))
            st8.capture(stream)
            for _ in range(4):
                st8.replay(stream)
            torch.cuda.synchronize()
            ctx_start = (lens + 4).tolist()
            t3 = time.perf_counter()
            for _ in range(args.b8_steps):
                st8.replay(stream)
            torch.cuda.synchronize()
            ms8 = (time.perf_counter() - t3) * 1e3 / args.b8_steps
            st8.check(stream)
        mean_ctx = float(np.mean(lens)) + 4 + args.b8_steps / 2
        kv_bytes = 2 * shape.layers * shape.n_kv_heads * shape.head_dim * 2 * mean_ctx * 8
        w_bytes = step_weight_bytes(shape)
        b8 = {"ms_per_step": round(ms8, 4), "tok_s": round(8e3 / ms8, 1), "steps": args.b8_steps,
              "context_at_start": ctx_start, "mean_context": round(mean_ctx, 1),
              "bytes_per_step": int(w_bytes + kv_bytes),
              "hbm_frac": round((w_bytes + kv_bytes) / (ms8 * 1e-3) / PEAK_HBM, 4)}
        log(f"B=8: {ms8:.3f} ms/step ({8e3 / ms8:.1f} tok/s)")
        st8.close()
        kv8.close()
        del st8, kv8
        torch.cuda.empty_cache()

    # ------------------------------------------------------------------ GEMV sweep
    sweep, agg = (None, None)
    if not args.skip_sweep:
        with torch.cuda.stream(stream):
            sweep, agg = gemv_sweep(stream)
    dm.close()
    del dm
    torch.cuda.empty_cache()

    # ------------------------------------------------------------------ CPU oracle
    cpu = None
    if not args.skip_cpu:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(shape, head)
        log(f"oracle: {cpu['s_per_token']} s/token on {cpu['cores']} cores")
        cpu["rows"] = cpu_rows(shape)
        log(f"oracle rows: {len(cpu['rows']['gemv'])} GEMV, {len(cpu['rows']['attention'])} attention, tiny "
            f"{cpu['rows']['tiny']['s_per_token']} s/token; BLAS {cpu['rows']['blas']}")

    wb = step_weight_bytes(shape)
    res = {
        "metric": METRIC, "value": round(1e3 / ms_b1, 2), "unit": "tok/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_b1, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": "Qwen2.5-Coder-7B-shaped greedy decode, batch 1, 512-token random prompt, "
                               "step replayed as one HIP graph", "batch": 1, "prompt_tokens": P,
                   "context_during_timing": [ctx0, ctx0 + K], "weights": "int4 symmetric g128, fp16 scales",
                   "activations": "fp16, fp32 accumulation", "kernels_per_step": n_kernels},
        "roofline": {k: roof_step[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")},
        "traffic_source": ("profiles/decode_step_7b_b1_persistent_pmc.md: rocprofv3 FETCH_SIZE / WRITE_SIZE runs "
                           "of bench.py --mode steproof on the same step source hash (not measured in this run; "
                           "null when the hash differs)"),
        "cpu_baseline": cpu,
        "ms_per_token_b1_events": round(ms_b1_events, 4),
        "ms_per_token_b1_eager": round(ms_eager, 4),
        "b1_kernel_per_stage": b1_kernels,
        "b1_persistent_stages": {k: stg[k] for k in ("gemv_stages", "gemv_stages_aggregate", "layer_us",
                                                     "lm_head_and_greedy_us", "step_us", "context")},
        "b1_context_sweep": ctx_sweep,
        "attention_sweep": att_sweep,
        "step_weight_bytes": wb,
        "step_roofline_ms": round(wb / PEAK_HBM * 1e3, 4),
        "step_roofline_frac": round(wb / PEAK_HBM * 1e3 / ms_b1, 4),
        "dominant_kernel": roof_step,
        "gemv_gate_up_roofline": roof,
        "ttft": ttft_block(shape, P, ttft_ms, ms_b1),
        "b8": b8,
        "gemv_sweep": sweep, "gemv_aggregate": agg,
        "context": {"pages_h100_ms_per_token_graph": 16.7, "pages_h100_ms_per_token_eager": 119,
                    "pages_h100_tok_s": 60},
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
