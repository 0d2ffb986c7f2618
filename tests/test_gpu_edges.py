"""Edge cases of the path against the oracle (needs an MI355X): one-token and
chunk-boundary prompts, a cache filled to its last position on both decode
paths, prompts that continue a sequence at an unaligned position, and the
degenerate attention spans (a window of one row, sinks covering the window).
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import SMALL, SMALL_F16, SMALL_Q8
from test_gpu_parity import check_step

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import llama_family_decode_amd as llm

    CHUNK = llm.llm_op_prefill_chunk()
else:
    CHUNK = 2048


def prefill_both(cfg, ts, toks):
    g, r = llm.Model(cfg, ts), oracle.Model(cfg, ts)
    nxt = g.prefill(toks)
    return g, r, nxt, g.logits(), r.prefill(toks)


@pytest.mark.parametrize("n", [1, CHUNK, CHUNK + 1])
def test_prompt_lengths_at_chunk_edges(monkeypatch, n):
    # one token; exactly one full chunk; one chunk plus a one-row chunk
    monkeypatch.setenv("LLM_STEP", "graph")
    cfg = SMALL_Q8.with_(n_ctx=CHUNK + 8)
    ts = synth.make_tensor_set(cfg)
    g, r, nxt, got, want = prefill_both(cfg, ts, synth.prompt(cfg, n))
    check_step(cfg, got, want, nxt, f"prompt of {n}")
    assert g.kv_len() == r.kv_len() == n
    g.close()
    r.close()


@pytest.mark.parametrize("kind", ["persistent", "graph"])
def test_cache_filled_to_its_last_position(monkeypatch, kind):
    monkeypatch.setenv("LLM_STEP", kind)
    cfg = SMALL_F16.with_(n_ctx=40)
    ts = synth.make_tensor_set(cfg)
    g, r, nxt, got, want = prefill_both(cfg, ts, synth.prompt(cfg, 33))
    check_step(cfg, got, want, nxt, "prompt")
    for pos in range(33, cfg.n_ctx):  # through position n_ctx - 1
        tok = oracle.argmax(want)
        want = r.forward(tok, pos)
        nxt = g.decode(tok, pos)
        check_step(cfg, g.logits(), want, nxt, f"pos {pos}")
    assert g.kv_len() == cfg.n_ctx
    with pytest.raises(llm.LlmError):
        g.decode(0, cfg.n_ctx)  # no row left
    with pytest.raises(llm.LlmError) as e:
        g.prefill([1])
    assert e.value.code == -8
    with pytest.raises(llm.LlmError):
        g.generate(1, 2)
    assert g.kv_len() == cfg.n_ctx  # failed calls change nothing
    g.close()
    r.close()


def test_prompts_continue_at_unaligned_positions(monkeypatch):
    # decode 3 tokens, then prefill 7, decode 1, prefill 5: every prefill
    # starts at a position that is not a multiple of anything the kernels tile by
    monkeypatch.setenv("LLM_STEP", "persistent")
    cfg = SMALL
    ts = synth.make_tensor_set(cfg)
    toks = synth.prompt(cfg, 16)
    g, r = llm.Model(cfg, ts), oracle.Model(cfg, ts)
    for p in range(3):
        nxt = g.decode(int(toks[p]), p)
        want = r.forward(int(toks[p]), p)
    nxt = g.prefill(toks[3:10])
    check_step(cfg, g.logits(), r.prefill(toks[3:10]), nxt, "prefill at 3")
    nxt = g.decode(int(toks[10]), 10)
    check_step(cfg, g.logits(), r.forward(int(toks[10]), 10), nxt, "decode at 10")
    nxt = g.prefill(toks[11:16])
    check_step(cfg, g.logits(), r.prefill(toks[11:16]), nxt, "prefill at 11")
    assert g.kv_len() == r.kv_len() == 16
    g.close()
    r.close()


@pytest.mark.parametrize("window,sinks", [(1, 0), (1, 3), (2, 40)])
def test_degenerate_spans(monkeypatch, window, sinks):
    # a window of one row (each query sees only itself), one row plus sinks,
    # and sinks that cover every row the window leaves out (the full span)
    monkeypatch.setenv("LLM_STEP", "persistent")
    cfg = SMALL_Q8.with_(attn_window=window, attn_sinks=sinks)
    ts = synth.make_tensor_set(cfg)
    g, r, nxt, got, want = prefill_both(cfg, ts, synth.prompt(cfg, 12))
    check_step(cfg, got, want, nxt, "prompt")
    pos = 12
    for _ in range(3):
        tok = oracle.argmax(want)
        want = r.forward(tok, pos)
        nxt = g.decode(tok, pos)
        check_step(cfg, g.logits(), want, nxt, f"pos {pos}")
        pos += 1
    if sinks >= 40:  # the whole span: identical to plain attention on the same path
        plain = llm.Model(cfg.with_(attn_window=0, attn_sinks=0), ts)
        plain.prefill(synth.prompt(cfg, 12))
        assert np.array_equal(plain.logits().view(np.uint32), got.view(np.uint32))
        plain.close()
    g.close()
    r.close()
