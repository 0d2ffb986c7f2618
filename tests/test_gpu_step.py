"""Parity of the persistent decode-step kernel with the CPU oracle (needs an MI355X).

The same checks as test_gpu_parity.py (logit tolerance, bit-exact argmax,
greedy agreement where the oracle's top-2 gap exceeds the tolerance, KV cache),
on contexts loaded with LLM_STEP=persistent, where one cooperative launch runs
each token's forward pass with the grid split into eight block groups. The
shapes cover every code path of that kernel: grouped-query heads with G = 1, 2,
4 and 8 (G = 8 runs as two passes of four query heads), KV-head counts below,
equal to and above the group count, short rows read by part of a wave, NEOX
RoPE with bias, partial RoPE, all three weight types, splits long enough to need
two attention chunks, llama.cpp's rounding points (numerics 1: rounded product
inputs and two attention passes), and the 1B shape of the decode benchmark.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import (SMALL, SMALL_F16, SMALL_F16_RND, SMALL_FREQS, SMALL_MHA, SMALL_RND, SMALL_NEOX_BIAS,
                     SMALL_PARTIAL_ROPE, SMALL_Q8, SMALL_Q8_RND, SMALL_SINKS, SMALL_SPAN_ALL, SMALL_TEMP, SMALL_WINDOW,
                     SMALL_YARN, SMALL_SPAN_RND)
from test_gpu_parity import check_llamacpp_q8_agreement, check_step, run_decode, tol

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import llama_family_decode_amd as llm


@pytest.fixture(autouse=True)
def persistent(monkeypatch):
    monkeypatch.setenv("LLM_STEP", "persistent")
    monkeypatch.delenv("LLM_STEP_TRACE", raising=False)


def load(cfg, ts=None, kind=1):
    m = llm.Model(cfg, synth.make_tensor_set(cfg) if ts is None else ts)
    assert llm.llm_op_step_kind(m.ctx) == kind, f"{cfg.name}: unexpected decode path"
    return m


G8 = SMALL.with_(name="small-g8", dim=256, n_heads=8, n_kv_heads=1, head_dim=32, seed=21)
KV16 = SMALL.with_(name="small-kv16", dim=512, n_heads=16, n_kv_heads=16, head_dim=32, ffn=320, seed=22)
SHORT_ROWS_Q8 = SMALL_Q8.with_(name="small-q8-g1", n_heads=2, n_kv_heads=2, head_dim=64, seed=23)
STEP_SMALLS = [SMALL, SMALL_F16, SMALL_Q8, SMALL_NEOX_BIAS, SMALL_PARTIAL_ROPE, G8, KV16, SHORT_ROWS_Q8, SMALL_FREQS,
               SMALL_WINDOW, SMALL_SINKS, SMALL_TEMP, SMALL_SPAN_ALL, SMALL_YARN, SMALL_RND, SMALL_F16_RND, SMALL_Q8_RND,
               G8.with_(name="small-g8-q8_0-llamacpp", mat_dtype="q8_0", tied=True, numerics=1, seed=26),
               KV16.with_(name="small-kv16-f16-llamacpp", mat_dtype="f16", embd_dtype="f16", tied=True, numerics=1,
                          seed=27),
               SHORT_ROWS_Q8.with_(name="small-q8-g1-llamacpp", numerics=1, seed=28), SMALL_SPAN_RND]


@pytest.mark.parametrize("cfg", STEP_SMALLS, ids=lambda c: c.name)
def test_step_decode_small(cfg):
    load(cfg).close()
    run_decode(cfg, n_prompt=5, n_steps=12)


@pytest.mark.parametrize("cfg", [SMALL_Q8, SMALL_F16], ids=lambda c: c.name)
def test_step_after_prefill(cfg):
    run_decode(cfg.with_(n_ctx=700), n_prompt=600, n_steps=6, prefill_gpu=True, prefill_ref=True)


def test_step_two_attention_chunks():
    # 8300 cached positions over 32 splits: 260 per split, more than the 128
    # positions one pass of a block covers at head_dim 64; four query heads
    # per KV head, as in the 1B shape.
    cfg = SMALL.with_(name="small-long", dim=256, n_heads=4, n_kv_heads=1, head_dim=64, n_ctx=8400, seed=24)
    run_decode(cfg, n_prompt=8300, n_steps=3, prefill_gpu=True, prefill_ref=True)


def test_step_config2_workload():
    cfg = synth.C2
    run_decode(cfg, n_prompt=cfg.prompt_len, n_steps=64, prefill_gpu=True, prefill_ref=True)


def test_step_1b_q8_shape():
    # the benchmark shape runs the kernel compiled for it (kind 2)
    cfg = synth.C4.with_(n_ctx=160)
    load(cfg, kind=2).close()
    run_decode(cfg, n_prompt=20, n_steps=4)


def test_step_1b_q8_rope_freqs_shape():
    # the benchmark kernel (kind 2) with Llama 3's frequency factors in the table
    cfg = synth.C4.with_(n_ctx=160, rope_freq_factors=True)
    load(cfg, kind=2).close()
    run_decode(cfg, n_prompt=20, n_steps=4)


def test_step_1b_q8_window_sinks_temperature():
    # the benchmark kernel (kind 2) with a window plus sinks and the attention
    # temperature: the span's 73 rows split five ways
    cfg = synth.C4.with_(n_ctx=200, attn_window=70, attn_sinks=3, attn_temp_scale=0.1, attn_temp_len=64)
    load(cfg, kind=2).close()
    run_decode(cfg, n_prompt=150, n_steps=4, prefill_gpu=True, prefill_ref=True)


def test_step_1b_q8_yarn_shape():
    # the benchmark kernel (kind 2) reading a YaRN table (factor 16)
    cfg = synth.C4.with_(n_ctx=160, yarn_factor=16.0, yarn_orig_ctx=16384)
    load(cfg, kind=2).close()
    run_decode(cfg, n_prompt=20, n_steps=4)


def test_step_1b_f16_llamacpp_numerics():
    # llama.cpp's rounding points in the F16 benchmark kernel (kind 2): binary16
    # product inputs, q, and the two attention passes over 150 positions
    cfg = synth.C3.with_(n_ctx=200, numerics=1)
    load(cfg, kind=2).close()
    run_decode(cfg, n_prompt=150, n_steps=4, prefill_gpu=True, prefill_ref=True)


def test_step_1b_q8_llamacpp_numerics_agreement_level():
    # the Q8_0 benchmark kernel (kind 2) with llama.cpp's rounding points, at
    # the agreement level of Q8_0 activations (the launch-graph test explains it)
    cfg = synth.C4.with_(n_ctx=160, numerics=1)
    load(cfg, kind=2).close()
    check_llamacpp_q8_agreement(cfg)


def test_step_llamacpp_numerics_generate_equals_decode_loop():
    # an extra barrier per layer in this mode: the counters must stay in step
    # over many launches, through llm_generate's device-side feedback as well
    cfg = SMALL_Q8_RND
    ts = synth.make_tensor_set(cfg)
    toks = synth.prompt(cfg, 6)
    a, b = load(cfg, ts), load(cfg, ts)
    n1, n2 = a.prefill(toks), b.prefill(toks)
    assert n1 == n2
    gen = a.generate(n1, 40)
    seq, t, pos = [], n2, len(toks)
    for _ in range(40):
        t = b.decode(t, pos)
        seq.append(t)
        pos += 1
    assert gen.tolist() == seq
    a.close()
    b.close()


def test_step_1b_f16_shape():
    cfg = synth.C3.with_(n_ctx=160)
    load(cfg, kind=2).close()
    run_decode(cfg, n_prompt=12, n_steps=3)


def test_step_falls_back_when_heads_do_not_align():
    # G * head_dim = 48 is not a multiple of 32: the launch graph runs the steps
    load(SMALL_MHA, kind=0).close()


def test_step_generate_equals_decode_loop():
    cfg = SMALL_Q8
    ts = synth.make_tensor_set(cfg)
    toks = synth.prompt(cfg, 6)
    a, b = load(cfg, ts), load(cfg, ts)
    n1, n2 = a.prefill(toks), b.prefill(toks)
    assert n1 == n2
    gen = a.generate(n1, 24)
    seq, t, pos = [], n2, len(toks)
    for _ in range(24):
        t = b.decode(t, pos)
        seq.append(t)
        pos += 1
    assert gen.tolist() == seq
    assert a.kv_len() == b.kv_len() == len(toks) + 24
    a.close()
    b.close()


def test_step_bit_exact_repeat_and_close_to_graph(monkeypatch):
    cfg = SMALL_F16
    ts = synth.make_tensor_set(cfg)
    toks = synth.prompt(cfg, 7)
    outs = []
    for _ in range(2):
        m = load(cfg, ts)
        m.prefill(toks)
        m.decode(5, len(toks))
        outs.append(m.logits())
        m.close()
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    monkeypatch.setenv("LLM_STEP", "graph")
    g = load(cfg, ts, kind=0)
    g.prefill(toks)
    g.decode(5, len(toks))
    assert float(np.max(np.abs(g.logits() - outs[0]))) <= tol(cfg)
    g.close()


def test_step_trace(monkeypatch):
    monkeypatch.setenv("LLM_STEP_TRACE", "1")
    cfg = SMALL
    m = load(cfg)
    m.prefill(synth.prompt(cfg, 4))
    m.decode(1, 4)
    tr = llm.llm_op_step_trace(m.ctx, cfg.n_layers).astype(np.int64)
    assert tr.shape == (5 * cfg.n_layers + 2,)
    assert np.all(np.diff(tr) >= 0)
    m.close()
