"""The greedy choice on the GPU: exact ties decided by the lowest index across
the partial results of different workgroups, and a NaN logit reported as an
error while every kernel of the step still runs to its end.

Ties are made exact by construction. Every LM-head row is 0.5 w, except the
rows TIE_POS (= w) and TIE_NEG (= -w), for one random row w. Halving a row
halves its fp16 group scales exactly and leaves its INT4 codes unchanged, so
the logit of a 0.5 w row is exactly half that of a w row, and identical rows
give bitwise identical logits. The largest logit is therefore attained by all
of TIE_POS (when the logit of w is positive) or all of TIE_NEG (negative), and
those rows lie in the tiles of different LM-head workgroups (and, for the first
two, in one workgroup). The rule (lowest index on ties, "How to build your own
LLM runtime from scratch", intro: greedy sampling) then fixes the token.

Two vocabularies reach the two LM-head kernels: 4096 rows (per-tile GEMV, 32
rows per workgroup) and 65536 rows (streaming GEMV, 256 rows per workgroup)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from w4a16_gemv_paged_amd import NQError
from w4a16_gemv_paged_amd.engine import DeviceModel, KVCache, Stepper, run_greedy
from gpu_util import say

pytestmark = pytest.mark.gpu

SMALL = synth.TINY                                                         # vocab 4096
BIG = synth.ModelShape("tiny-1L-v65536", 1, 512, 1408, 8, 2, 64, 65536)   # streaming LM head
TIES = {SMALL.vocab: ((40, 45, 3000), (70, 75, 4000)),
        BIG.vocab: ((300, 305, 60000), (700, 705, 50000))}


def _tie_head(shape):
    head = synth.head_params(shape, seed=0)
    w = synth.gemv_weight(shape.hidden, 1, seed=90)[0]
    lm = np.tile(np.float32(0.5) * w, (shape.vocab, 1))
    pos, neg = TIES[shape.vocab]
    lm[list(pos)] = w
    lm[list(neg)] = -w
    head["lm_head"] = lm
    return head


def _model(shape, head):
    say("build model", shape.name)
    return DeviceModel(shape, lambda l: synth.layer_params(shape, l, seed=0), head, max_batch=8, max_pos=1024)


def _decode(dm, prompts, n_gen, graph):
    pt, total = synth.decode_page_tables(len(prompts), 4, seed=3, spare_pages=2)
    kv = KVCache(dm, total, poison=True)
    st = Stepper(dm, kv, pt, want_logits=True)
    stream = torch.cuda.Stream() if graph else torch.cuda.current_stream()
    with torch.cuda.stream(stream):
        out = run_greedy(st, prompts, n_gen, use_graph=graph, stream=stream, record_logits=True)
    torch.cuda.synchronize()
    st.close()
    kv.close()
    return out


@pytest.mark.parametrize("shape", [SMALL, BIG], ids=["per-tile-head", "streaming-head"])
@pytest.mark.parametrize("batch", [1, 8])
def test_ties_go_to_the_lowest_index(shape, batch):
    dm = _model(shape, _tie_head(shape))
    pos, neg = TIES[shape.vocab]
    prompts = [synth.prompt_ids(5 + b, shape.vocab, seed=80 + b) for b in range(batch)]
    say("tie run", shape.name, "batch", batch)
    out = _decode(dm, prompts, 6, graph=batch == 8)
    dm.close()
    seen = set()
    for b, p in enumerate(prompts):
        for i, s in enumerate(range(len(p) - 1, len(p) + 5)):
            z = out["logits"][s, b]
            zp, zn = z[list(pos)], z[list(neg)]
            assert np.all(zp.view(np.uint32) == zp[0].view(np.uint32)), (b, i)   # the ties are exact
            assert np.all(zn.view(np.uint32) == zn[0].view(np.uint32)), (b, i)
            want = pos[0] if zp[0] > zn[0] else neg[0]
            assert oracle.argmax_lowest(z) == want, (b, i)                     # the construction holds
            assert out["tokens"][b][i] == want, (b, i, out["tokens"][b][i], want)
            seen.add(want)
    if batch == 8:
        assert seen == {pos[0], neg[0]}       # both tie groups were decided somewhere in the batch


def _scale_offset(shape, row, group):
    """Byte offset of the fp16 scale of (row, group) in the packed LM head:
    the codes of all (tile, group) blocks come first, then the scales of block
    (t, g) as 16 consecutive rows (identity row order for the LM head)."""
    G = shape.hidden // 128
    T = (shape.vocab + 15) // 16
    codes = T * G * 1024
    t, r = divmod(row, 16)
    return codes + ((t * G + group) * 16 + r) * 2


@pytest.mark.parametrize("shape", [SMALL, BIG], ids=["per-tile-head", "streaming-head"])
@pytest.mark.parametrize("batch", [1, 2])
def test_nan_logit_is_reported_and_the_step_completes(shape, batch):
    """At batch 1 the step is the persistent kernel, at batch 2 the kernel per stage."""
    dm = _model(shape, synth.head_params(shape, seed=0))
    off = _scale_offset(shape, 123, 0)
    saved = dm.lm[off:off + 2].clone()
    dm.lm[off:off + 2] = torch.tensor([0x00, 0x7E], dtype=torch.uint8, device="cuda")   # fp16 NaN
    prompts = [synth.prompt_ids(3, shape.vocab, seed=85 + b) for b in range(batch)]
    pt, total = synth.decode_page_tables(batch, 4, seed=3, spare_pages=2)
    kv = KVCache(dm, total, poison=True)
    st = Stepper(dm, kv, pt, want_logits=True)
    st.set_pos(np.zeros(batch, np.int32))
    st.set_tokens([p[0] for p in prompts])
    say("NaN logit step", shape.name)
    st.step()
    torch.cuda.synchronize()
    assert int(st.err.cpu()[0]) & 8
    assert np.all(np.isnan(st.logits.cpu().numpy()[:, 123]))
    with pytest.raises(NQError) as e:
        st.check()
    assert e.value.status == 6                    # NQ_ERR_DEVICE_FAULT
    assert int(st.err.cpu()[0]) == 0              # the check resets the flag
    # the same buffers step again normally once the scale is restored
    dm.lm[off:off + 2] = saved
    st.set_tokens([p[1] for p in prompts])
    say("step after NaN", shape.name)
    st.step()
    st.check()
    z = st.logits.cpu().numpy()
    assert np.all(np.isfinite(z))
    np.testing.assert_array_equal(st.tokens.cpu().numpy(), [oracle.argmax_lowest(z[b]) for b in range(batch)])
    st.close()
    kv.close()
    dm.close()
