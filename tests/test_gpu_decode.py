"""End-to-end GPU decode parity against the oracle (tiny Qwen2-style config).

Run: 16-token prompt, 32 greedy tokens, KV in 16-token pages ending on a
partial page (47 cached positions = 2 full pages + 15). Every test runs in both
step modes: "auto" (batch 1 as the persistent whole-step kernel) and
"kernels" (one kernel per stage)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.model import OracleModel, layer_causal, head_logits
from w4a16_gemv_paged_amd.engine import DeviceModel, KVCache, Stepper, run_greedy, write_container
from gpu_util import F16, rel_inf, say

pytestmark = pytest.mark.gpu

SHAPE = synth.TINY
PROMPT_LEN, N_GEN = 16, 32
TOL_LAYER, TOL_LOGITS, MARGIN = 2e-3, 5e-3, 1e-2


@pytest.fixture(scope="module", params=["auto", "kernels"])
def tiny(request):
    layers = [synth.layer_params(SHAPE, i, seed=0) for i in range(SHAPE.layers)]
    head = synth.head_params(SHAPE, seed=0)
    om = OracleModel.build(SHAPE, layers, head)
    say("build tiny device model, step mode", request.param)
    dm = DeviceModel(SHAPE, lambda i: layers[i], head, max_batch=8, max_pos=4096)
    dm.set_step_mode(request.param)
    dm.mode = request.param
    yield om, dm
    dm.close()


def _expected_kernels(dm, batch, max_pages):
    n = dm.step_kernels(batch, max_pages)
    if dm.mode == "auto" and batch == 1:
        assert n == 1           # the persistent step is what runs (MI355X, 256 CUs)
    else:
        assert n > 1
    return n


def _run(dm, prompts, n_gen, graph=False, pages=None, seed=3, layers=True):
    B = len(prompts)
    need = max(len(p) for p in prompts) + n_gen
    max_pages = pages or (need + 15) // 16
    pt, total = synth.decode_page_tables(B, max_pages, seed=seed, spare_pages=3)
    kv = KVCache(dm, total, poison=True)
    st = Stepper(dm, kv, pt, hist_len=need + 1, want_logits=True, want_layers=layers)
    stream = torch.cuda.Stream() if graph else torch.cuda.current_stream()   # capture needs a non-null stream
    with torch.cuda.stream(stream):
        out = run_greedy(st, prompts, n_gen, use_graph=graph, stream=stream, record_logits=True,
                         record_layers=layers)
    torch.cuda.synchronize()
    out["pool"] = kv.pool.cpu().numpy()
    out["page_table"] = pt
    out["hist"] = st.hist.cpu().numpy()
    out["kernels"] = None
    out["max_pages"] = max_pages
    if graph:
        from w4a16_gemv_paged_amd import nq_graph_kernel_count
        out["kernels"] = nq_graph_kernel_count(st.graph)
    st.close()
    kv.close()
    return out


@pytest.fixture(scope="module")
def tiny_run(tiny):
    om, dm = tiny
    prompt = synth.prompt_ids(PROMPT_LEN, SHAPE.vocab, seed=2)
    say("tiny eager run")
    gpu = _run(dm, [prompt], N_GEN)
    orc = oracle.generate(om, prompt, N_GEN, forced=gpu["tokens"][0])
    return prompt, gpu, orc


def test_tokens_match_where_margin_is_clear(tiny_run):
    prompt, gpu, orc = tiny_run
    ok = orc["margins"] > MARGIN
    assert ok.sum() >= N_GEN // 2          # the gate must not be vacuous
    np.testing.assert_array_equal(gpu["tokens"][0][ok], orc["tokens"][ok])


def test_logits_within_tolerance(tiny_run):
    prompt, gpu, orc = tiny_run
    gl = gpu["logits"][PROMPT_LEN - 1:, 0]
    assert gl.shape == orc["logits"].shape
    errs = [rel_inf(gl[i], orc["logits"][i]) for i in range(N_GEN)]
    assert max(errs) < TOL_LOGITS, max(errs)


def test_each_layer_teacher_forced(tiny_run, tiny):
    """Layer l recomputed by the oracle from the GPU's own layer l-1 output at
    every position (the oracle's own KV for those inputs)."""
    om, dm = tiny
    prompt, gpu, orc = tiny_run
    fed = list(prompt) + list(gpu["tokens"][0][:-1])
    lo = gpu["layer_out"][:, :, 0]                     # [T, L, H]
    x = om.head.embed[np.array(fed)]
    for li in range(SHAPE.layers):
        ref = layer_causal(om.layers[li], om.dims, x)
        errs = [rel_inf(lo[t, li], ref[t]) for t in range(len(fed))]
        assert max(errs) < TOL_LAYER, (li, max(errs))
        x = lo[:, li]
    z = head_logits(om, lo[:, -1])
    errs = [rel_inf(gpu["logits"][t, 0], z[t]) for t in range(PROMPT_LEN - 1, len(fed))]
    assert max(errs) < TOL_LOGITS


def test_free_running_layers_within_tolerance(tiny_run):
    prompt, gpu, orc = tiny_run
    lo = gpu["layer_out"][:, :, 0]
    olo = orc["layer_out"]                              # [T, L, H]
    errs = [rel_inf(lo[t, li], olo[t, li]) for t in range(lo.shape[0]) for li in range(SHAPE.layers)]
    assert max(errs) < 5e-3, max(errs)


def test_kv_pool_contents_and_untouched_slots(tiny_run, tiny):
    """K (after RoPE) and V in the pool match the oracle's projections of the
    GPU's layer inputs; slots past the last position keep their NaN poison."""
    om, dm = tiny
    prompt, gpu, orc = tiny_run
    fed = list(prompt) + list(gpu["tokens"][0][:-1])
    T = len(fed)
    cfg = dm.cfg
    pool = gpu["pool"].view(F16).reshape(cfg.layers, 2, -1, cfg.n_kv_heads, 16 * cfg.head_dim)
    kvm = oracle.PagedKVEmu(cfg.layers, pool.shape[2], cfg.n_kv_heads, cfg.head_dim, gpu["page_table"], pool=pool)
    lo = gpu["layer_out"][:, :, 0]
    x = om.head.embed[np.array(fed)]
    d, nh, nkv = cfg.head_dim, cfg.n_heads, cfg.n_kv_heads
    for li in range(cfg.layers):
        L = om.layers[li]
        xn = oracle.rmsnorm(x, L.g1, 1e-6)
        qkv = (xn.astype(np.float64) @ L.w("qkv").T + L.b_qkv.astype(np.float64)).astype(F16)
        k = oracle.rope(qkv[:, nh * d:(nh + nkv) * d].reshape(T, nkv, d), np.arange(T), 1e6)
        v = qkv[:, (nh + nkv) * d:].reshape(T, nkv, d)
        kg, vg = kvm.get(li, 0, T)
        assert rel_inf(kg, k) < TOL_LAYER and rel_inf(vg, v) < TOL_LAYER
        x = lo[:, li]
    last_page = gpu["page_table"][0, (T - 1) // 16]
    s0 = (T - 1) % 16 + 1
    kpage = pool[:, 0, last_page].reshape(cfg.layers, cfg.n_kv_heads, 16, d).astype(np.float32)
    vpage = pool[:, 1, last_page].reshape(cfg.layers, cfg.n_kv_heads, d, 16).astype(np.float32)
    assert np.all(np.isnan(kpage[:, :, s0:])) and np.all(np.isnan(vpage[..., s0:]))


def test_token_history_written(tiny_run):
    prompt, gpu, orc = tiny_run
    hist = gpu["hist"][0]
    np.testing.assert_array_equal(hist[PROMPT_LEN:PROMPT_LEN + N_GEN], gpu["tokens"][0])


def test_graph_replay_equals_eager_bitwise(tiny, tiny_run):
    om, dm = tiny
    prompt, eager, _ = tiny_run
    say("tiny graph run")
    g = _run(dm, [prompt], N_GEN, graph=True)
    np.testing.assert_array_equal(g["tokens"], eager["tokens"])
    np.testing.assert_array_equal(g["logits"].view(np.uint32), eager["logits"].view(np.uint32))
    np.testing.assert_array_equal(g["layer_out"].view(np.uint16), eager["layer_out"].view(np.uint16))
    assert g["kernels"] == _expected_kernels(dm, 1, g["max_pages"])


def test_batched_ragged_equals_single_sequences(tiny):
    """B = 4 with ragged prompts gives, per sequence, what B = 1 gives."""
    om, dm = tiny
    prompts = [synth.prompt_ids(n, SHAPE.vocab, seed=20 + n) for n in (5, 16, 9, 23)]
    say("tiny batched run")
    bat = _run(dm, prompts, 8, layers=False)
    for b, p in enumerate(prompts):
        say("tiny single run", b)
        one = _run(dm, [p], 8, layers=False)
        np.testing.assert_array_equal(bat["tokens"][b], one["tokens"][0])


def test_batch8_logits_against_oracle(tiny):
    om, dm = tiny
    prompts = [synth.prompt_ids(n, SHAPE.vocab, seed=40 + n) for n in (3, 7, 12, 16, 4, 9, 2, 14)]
    say("tiny batch-8 run")
    gpu = _run(dm, prompts, 4, layers=False)
    for b, p in enumerate(prompts):
        orc = oracle.generate(om, p, 4, forced=gpu["tokens"][b])
        steps = range(len(p) - 1, len(p) + 3)
        for i, s in enumerate(steps):
            assert rel_inf(gpu["logits"][s, b], orc["logits"][i]) < TOL_LOGITS
        ok = orc["margins"] > MARGIN
        np.testing.assert_array_equal(gpu["tokens"][b][ok], orc["tokens"][ok])


def test_split_attention_long_context(tiny):
    """Batch 1 over 64-page tables, 200-token prompt (13-14 pages in use). One
    kernel per stage: the pages split over 16 workgroups per KV head (4 pages
    each, one per wave; four splits hold pages, the rest are empty) whose
    partials the combine kernel merges. Persistent step: four splits of 4 pages
    per KV head, on XCD 0 for the first KV head and XCD 4 for the second, whose
    32 workgroups merge the head's outputs after a barrier of that XCD alone.
    Logits and tokens against the oracle; graph replay equals eager bitwise."""
    om, dm = tiny
    prompt = synth.prompt_ids(200, SHAPE.vocab, seed=60)
    say("tiny long-context eager run")
    gpu = _run(dm, [prompt], 8, pages=64, layers=False)
    orc = oracle.generate(om, prompt, 8, forced=gpu["tokens"][0])
    gl = gpu["logits"][len(prompt) - 1:, 0]
    errs = [rel_inf(gl[i], orc["logits"][i]) for i in range(8)]
    assert max(errs) < TOL_LOGITS, max(errs)
    ok = orc["margins"] > MARGIN
    np.testing.assert_array_equal(gpu["tokens"][0][ok], orc["tokens"][ok])
    say("tiny long-context graph run")
    g = _run(dm, [prompt], 8, pages=64, graph=True, layers=False)
    np.testing.assert_array_equal(g["logits"].view(np.uint32), gpu["logits"].view(np.uint32))
    assert g["kernels"] == _expected_kernels(dm, 1, 64)


def test_split_attention_many_splits(tiny):
    """Batch 1 at a 2500-token context (157 pages): the persistent step splits
    each KV head's pages 40 ways (4 pages per workgroup, one per attention
    wave), more than one XCD's 32 workgroups, so after a hand-off across all
    XCDs every workgroup merges two outputs over the 40 splits (the tiny
    model's 512 outputs over 256 workgroups), ten per lane in three batches of
    loads. Logits and tokens against the oracle."""
    om, dm = tiny
    prompt = synth.prompt_ids(2500, SHAPE.vocab, seed=61)
    say("tiny 2500-token context run")
    gpu = _run(dm, [prompt], 4, layers=False)
    orc = oracle.generate(om, prompt, 4, forced=gpu["tokens"][0])
    gl = gpu["logits"][len(prompt) - 1:, 0]
    errs = [rel_inf(gl[i], orc["logits"][i]) for i in range(4)]
    assert max(errs) < TOL_LOGITS, max(errs)
    ok = orc["margins"] > MARGIN
    np.testing.assert_array_equal(gpu["tokens"][0][ok], orc["tokens"][ok])


def test_split_attention_local_to_global_merge(tiny):
    """Batch 1 from a 2040-token prompt through 16 generated tokens (contexts
    2041-2056): the persistent step splits each KV head's pages into at most
    32 splits of 4 pages, all on one XCD and merged after a barrier of that XCD
    alone, while the context is at most 2048 tokens (128 pages); from 2049
    tokens on 33 splits no longer fit one XCD's 32 workgroups, and every
    workgroup merges its share after a hand-off across all XCDs. Every step's
    logits against the oracle, and the tokens where the margin is clear."""
    om, dm = tiny
    prompt = synth.prompt_ids(2040, SHAPE.vocab, seed=62)
    say("tiny 2040-token context run")
    gpu = _run(dm, [prompt], 16, layers=False)
    orc = oracle.generate(om, prompt, 16, forced=gpu["tokens"][0])
    gl = gpu["logits"][len(prompt) - 1:, 0]
    errs = [rel_inf(gl[i], orc["logits"][i]) for i in range(16)]
    assert max(errs) < TOL_LOGITS, max(errs)
    ok = orc["margins"] > MARGIN
    np.testing.assert_array_equal(gpu["tokens"][0][ok], orc["tokens"][ok])


def test_split_attention_batch8(tiny):
    """Batch 8 over 64-page tables: ragged prompts of 90-300 tokens span one to
    three splits of the pages."""
    om, dm = tiny
    lens = (90, 300, 130, 210, 160, 250, 100, 180)
    prompts = [synth.prompt_ids(n, SHAPE.vocab, seed=70 + i) for i, n in enumerate(lens)]
    say("tiny long-context batch-8 run")
    gpu = _run(dm, prompts, 3, pages=64, layers=False)
    for b, p in enumerate(prompts):
        orc = oracle.generate(om, p, 3, forced=gpu["tokens"][b])
        for i, s in enumerate(range(len(p) - 1, len(p) + 2)):
            assert rel_inf(gpu["logits"][s, b], orc["logits"][i]) < TOL_LOGITS, (b, i)
        ok = orc["margins"] > MARGIN
        np.testing.assert_array_equal(gpu["tokens"][b][ok], orc["tokens"][ok])
    say("tiny long-context batch-8 graph run")
    g = _run(dm, prompts, 3, pages=64, graph=True, layers=False)
    assert g["kernels"] == _expected_kernels(dm, 8, 64) == 6 * SHAPE.layers + 2
    np.testing.assert_array_equal(g["logits"].view(np.uint32), gpu["logits"].view(np.uint32))


def test_stage_trace_changes_nothing(tiny):
    """The persistent step's stage stamps (nq_model_set_step_trace) leave every
    logit bitwise unchanged; after the run the buffer holds the last step's
    stamps, in order within each workgroup (kernel start, 16 events per layer,
    LM head partials, end). With one kernel per stage nothing is written."""
    om, dm = tiny
    prompt = synth.prompt_ids(20, SHAPE.vocab, seed=12)
    say("trace off / on runs")
    a = _run(dm, [prompt], 6, layers=False)
    L = SHAPE.layers
    buf = torch.full((256 * (L + 1) * 16,), -1, dtype=torch.int64, device="cuda")
    dm.set_step_trace(buf)
    try:
        b = _run(dm, [prompt], 6, layers=False)
    finally:
        dm.set_step_trace(None)
    np.testing.assert_array_equal(a["logits"].view(np.uint32), b["logits"].view(np.uint32))
    t = buf.cpu().numpy().reshape(256, L + 1, 16)
    if dm.mode == "auto":
        seq = np.concatenate([t[:, L, :1], t[:, :L, :].reshape(256, -1), t[:, L, 1:3]], axis=1)
        assert np.all(seq > 0)
        assert np.all(np.diff(seq, axis=1) >= 0)
        assert np.all(t[:, L, 3:] == -1)
    else:
        assert np.all(t == -1)


def test_model_from_container_decodes_identically(tiny, tmp_path):
    """The same weights through the packed-weight container (written once,
    memory-mapped and uploaded without repacking) decode bit for bit alike."""
    om, dm = tiny
    path = str(tmp_path / "tiny.nqpack")
    write_container(path, SHAPE, lambda l: synth.layer_params(SHAPE, l, seed=0), synth.head_params(SHAPE, seed=0))
    say("tiny model from container")
    dm2 = DeviceModel.load(path, max_batch=8, max_pos=4096)
    dm2.set_step_mode(dm.mode)
    prompt = synth.prompt_ids(PROMPT_LEN, SHAPE.vocab, seed=2)
    a = _run(dm, [prompt], 8, layers=False)
    b = _run(dm2, [prompt], 8, layers=False)
    dm2.close()
    np.testing.assert_array_equal(a["tokens"], b["tokens"])
    np.testing.assert_array_equal(a["logits"].view(np.uint32), b["logits"].view(np.uint32))
