"""Full-size checks in the launch configuration bench.py times (needs an MI355X).

The oracle cannot run the whole 1B model through a 2048-position prompt in a
test's time, so at these sizes the checks are outputs the oracle computes one
at a time, plus properties that hold at any size:
  - layer-0 K and V rows at sampled positions depend only on that position's
    token, so the oracle computes them directly (RMSNorm, the K/V products,
    bias, RoPE, binary16 rounding; "The Forward Pass in Java", Examples 4, 5,
    6 and 10): rows the decode path wrote agree within 2 binary16 ulps, rows
    the matrix-core prefill wrote within the logit tolerance of the head rms;
  - the greedy token is the first index of the strict maximum of the GPU's own
    logits, bit for bit ("The Forward Pass in Java", Example 9);
  - the KV length is the prompt plus the decoded steps;
  - the decode path bench.py times (the shape-compiled persistent kernel) and
    the launch-graph path (separate kernels) agree within the logit tolerance
    on every teacher-forced step, and a second run repeats bit for bit;
  - the 512-token matrix-core prefill agrees with the same tokens decoded one
    at a time, within the logit tolerance;
  - with a sliding window plus sink rows, the step reads exactly the rows of
    its span: overwriting any other cache row changes no logit bit.
"""
import numpy as np
import pytest

import oracle
import synth
from test_gpu_parity import f16_ulp_diff, first_max, tol

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import llama_family_decode_amd as llm


def _tensors_by_name(ts):
    return {t.name: t for t in ts}


def _row(t, dim, row):
    """Row `row` of a [rows][dim] tensor, dequantized to fp32 by the oracle."""
    if t.dtype == 8:  # Q8_0: 34 bytes per block of 32
        nb = dim // 32 * 34
        raw = t.data[row * nb:(row + 1) * nb]
    else:
        es = 4 if t.dtype == 0 else 2
        raw = t.data[row * dim * es:(row + 1) * dim * es]
    return oracle.dequantize(t.dtype, raw, dim)


def layer0_kv_oracle(cfg, T, token, pos):
    """Binary16 bits of layer 0's K and V rows for `token` at `pos`."""
    x = _row(T["token_embd.weight"], cfg.dim, int(token))
    h = oracle.rmsnorm(x, oracle.dequantize(0, T["blk.0.attn_norm.weight"].data, cfg.dim), cfg.eps)
    kvd = cfg.kv_dim
    out = []
    for name, bias_name in (("blk.0.attn_k.weight", "blk.0.attn_k.bias"), ("blk.0.attn_v.weight", "blk.0.attn_v.bias")):
        t = T[name]
        w = oracle.dequantize(t.dtype, t.data, kvd * cfg.dim)
        # the rounding mode rounds the product's input for the weight type
        hx = oracle.round_input(h, t.dtype) if cfg.numerics else h
        v = oracle.matvec(w, hx, kvd, cfg.dim)
        if bias_name in T:
            v = v + oracle.dequantize(0, T[bias_name].data, kvd)
        if name.endswith("attn_k.weight"):
            v = oracle.rope(v, cfg.n_kv_heads, cfg.head_dim, cfg.n_rot, pos, cfg.rope_base, cfg.rope_neox)
        out.append(np.array([oracle.f32_to_f16(float(e)) for e in v], np.uint16))
    return out


def check_layer0_kv(cfg, T, model, tokens_at, max_ulps):
    """Layer-0 K/V rows against the oracle's. Rows written by the decode path
    see fp32 activations on both sides and may differ only by binary16
    rounding flips (max_ulps = 2). Rows written by the matrix-core prefill
    (max_ulps None) are held to the logit tolerance relative to the head's rms,
    plus 2 ulps, as the parity suite holds every layer."""
    worst = 0.0
    for pos, tok in tokens_at:
        kg, vg = model.kv_read(0, pos)
        ko, vo = layer0_kv_oracle(cfg, T, tok, pos)
        for g, o in ((kg, ko), (vg, vo)):
            if max_ulps is not None:
                worst = max(worst, float(f16_ulp_diff(g, o, cfg.head_dim).max()))
            else:
                a = g.view(np.float16).astype(np.float64).reshape(-1, cfg.head_dim)
                b = o.view(np.float16).astype(np.float64).reshape(-1, cfg.head_dim)
                rms = np.sqrt(np.mean(b * b, axis=1, keepdims=True)) + 1e-30
                ulp = np.spacing(np.maximum(np.abs(a), np.abs(b)).astype(np.float16)).astype(np.float64)
                worst = max(worst, float(((np.abs(a - b) - 2 * ulp) / rms).max()))
    if max_ulps is not None:
        assert worst <= max_ulps, f"layer-0 KV differs from the oracle by {worst} binary16 ulps"
    else:
        assert worst <= tol(cfg), f"layer-0 KV differs from the oracle by {worst:.3e} of the head rms"
    return worst


@pytest.mark.parametrize("cfg,ctx", [(synth.C4, 2048), (synth.C3, 2048), (synth.C4_LONG, 8192),
                                     (synth.C3.with_(name="llama-1b-f16-llamacpp", numerics=1), 2048)],
                         ids=["q8_0-ctx2048", "f16-ctx2048", "q8_0-ctx8192", "f16-llamacpp-ctx2048"])
def test_decode_at_full_context_in_the_benchmarked_kernel(monkeypatch, cfg, ctx):
    # the three decode workloads: 1B Q8_0 with the tied F32 embedding at 2048
    # (the headline) and at 8192 positions, 1B F16 at 2048; and the F16 one
    # with llama.cpp's rounding points (the benchmark kernel's rounding
    # variant: binary16 product inputs, two attention passes over 2048 rows)
    ts = synth.make_tensor_set(cfg)
    T = _tensors_by_name(ts)
    toks = synth.prompt(cfg, ctx)
    n_steps = 6

    def run(kind_env):
        monkeypatch.setenv("LLM_STEP", kind_env)
        m = llm.Model(cfg, ts)
        nxt = m.prefill(toks)
        feed, logits, nexts = [], [], []
        t, pos = nxt, len(toks)
        for _ in range(n_steps):
            feed.append((pos, int(t)))
            n2 = m.decode(int(t), pos)
            logits.append(m.logits())
            nexts.append(n2)
            t, pos = n2, pos + 1
        return m, feed, logits, nexts

    step, feed, lg_step, nx_step = run("persistent")
    assert llm.llm_op_step_kind(step.ctx) == 2, "the benchmark shape must run the shape-compiled step kernel"
    assert step.kv_len() == len(toks) + n_steps
    for lg, nx in zip(lg_step, nx_step):
        assert np.all(np.isfinite(lg))
        assert nx == first_max(lg)
    w0 = check_layer0_kv(cfg, T, step, feed, 2.0)
    wp = check_layer0_kv(cfg, T, step, [(0, toks[0]), (ctx // 2, toks[ctx // 2]), (ctx - 1, toks[ctx - 1])], None)

    # the independent launch-graph path, teacher-forced with the same tokens
    monkeypatch.setenv("LLM_STEP", "graph")
    g = llm.Model(cfg, ts)
    assert llm.llm_op_step_kind(g.ctx) == 0
    g.prefill(toks)
    worst = 0.0
    for (pos, tok), lg in zip(feed, lg_step):
        g.decode(tok, pos)
        worst = max(worst, float(np.max(np.abs(g.logits().astype(np.float64) - lg))))
    assert worst <= tol(cfg), f"persistent vs graph: max |dlogit| {worst:.3e}"
    g.close()

    # a second persistent run repeats bit for bit
    step.close()
    again, _, lg2, nx2 = run("persistent")
    assert nx2 == nx_step
    for a, b in zip(lg_step, lg2):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    again.close()
    print(f"[{cfg.name} ctx {ctx}] layer-0 KV: decode rows {w0} ulps, prefill rows {wp:.2e} rms; persistent vs "
          f"graph {worst:.3e}", flush=True)


def test_q8_llamacpp_integer_products_layer0_against_the_oracle(monkeypatch):
    # llama.cpp's rounding points on the 1B Q8_0 model in the benchmarked
    # kernel: its products are integer dot products of the weight codes with
    # the input's Q8_0 codes ("What a Llama model computes, and why", section
    # 8). Layer 0's K and V rows of the decode steps depend only on each
    # step's token, and the oracle computes them as the product of the
    # dequantized weights with the rounded input: the two agree within
    # binary16 rounding flips. Two runs repeat bit for bit.
    cfg = synth.C4.with_(name="llama-1b-q8_0-llamacpp", numerics=1)
    ts = synth.make_tensor_set(cfg)
    T = _tensors_by_name(ts)
    toks = synth.prompt(cfg, 2048)
    monkeypatch.setenv("LLM_STEP", "persistent")
    runs = []
    for _ in range(2):
        m = llm.Model(cfg, ts)
        assert llm.llm_op_step_kind(m.ctx) == 2
        t, pos = int(m.prefill(toks)), len(toks)
        feed, logits, nexts = [], [], []
        for _ in range(6):
            feed.append((pos, t))
            t = m.decode(t, pos)
            logits.append(m.logits())
            nexts.append(t)
            pos += 1
        for lg, nx in zip(logits, nexts):
            assert np.all(np.isfinite(lg)) and nx == first_max(lg)
        w0 = check_layer0_kv(cfg, T, m, feed, 2.0)
        runs.append((nexts, logits))
        m.close()
    assert runs[0][0] == runs[1][0]
    for a, b in zip(runs[0][1], runs[1][1]):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    print(f"[{cfg.name}] layer-0 K/V of the integer products within {w0} binary16 ulps", flush=True)


def test_c5_prefill_512_against_decode_and_oracle(monkeypatch):
    cfg = synth.C5  # Qwen2-style 1B, F16, NEOX RoPE, QKV bias
    ts = synth.make_tensor_set(cfg)
    T = _tensors_by_name(ts)
    toks = synth.prompt(cfg, 512)
    monkeypatch.setenv("LLM_STEP", "persistent")
    pre = llm.Model(cfg, ts)
    nxt = pre.prefill(toks)
    lp = pre.logits()
    assert pre.kv_len() == 512
    assert np.all(np.isfinite(lp)) and nxt == first_max(lp)
    w0 = check_layer0_kv(cfg, T, pre, [(p, toks[p]) for p in (0, 1, 127, 128, 255, 256, 383, 511)], None)
    dec = llm.Model(cfg, ts)
    for p, t in enumerate(toks):
        dec.decode(int(t), p)
    ld = dec.logits()
    err = float(np.max(np.abs(lp.astype(np.float64) - ld)))
    assert err <= tol(cfg), f"prefill vs token-by-token decode: max |dlogit| {err:.3e}"
    pre.close()
    dec.close()
    print(f"[C5 prefill 512] layer-0 KV {w0:.2e} rms, prefill vs decode {err:.3e}", flush=True)


def test_c4_window_and_sinks_read_exactly_their_rows_at_ctx_4096(monkeypatch):
    # a 1024-row window plus 4 sink rows at position 4096 in the benchmarked
    # kernel ("The Engine", sink:s,w). Layer 0's cache is rewritten so that
    # every row has the current position's K (equal scores, so any row that
    # is read gets weight 1/(rows read)) and its own random V. Then a new V in
    # a row of the span (the window's first row, a sink row) changes the
    # logits, and a new V anywhere else (the row just below the window, the
    # first row above the sinks, every row in between, also in the last
    # layer) leaves them bit for bit the same. The launch graph agrees within
    # the logit tolerance.
    cfg = synth.C4.with_(attn_window=1024, attn_sinks=4)
    ts = synth.make_tensor_set(cfg)
    toks = synth.prompt(cfg, 4096)
    monkeypatch.setenv("LLM_STEP", "persistent")
    m = llm.Model(cfg, ts)
    assert llm.llm_op_step_kind(m.ctx) == 2
    tok = int(m.prefill(toks))
    pos = len(toks)
    lo = pos - 1024 + 1  # first window row
    kvd = cfg.kv_dim
    rng = np.random.default_rng(7)

    def garbage(n):
        return rng.normal(0, 1, n * kvd).astype(np.float16).view(np.uint16).reshape(n, kvd)

    def step():
        m.rewind(pos)
        m.decode(tok, pos)
        return m.logits()

    step()  # writes row pos
    k_pos, _ = m.kv_read(0, pos)
    llm.llm_op_kv_write(m.ctx, 0, 0, np.tile(k_pos, (pos, 1)), garbage(pos), kvd)
    base = step()
    assert np.all(np.isfinite(base))

    def same_after(layer, row, n=1):
        k = np.tile(k_pos, (n, 1)) if layer == 0 else garbage(n)
        llm.llm_op_kv_write(m.ctx, layer, row, k, garbage(n), kvd)
        return np.array_equal(step().view(np.uint32), base.view(np.uint32))

    assert same_after(0, lo - 1), "the row below the window was read"
    assert same_after(0, 4), "the first row above the sinks was read"
    assert same_after(0, 5, lo - 6), "rows between the sinks and the window were read"
    assert same_after(cfg.n_layers - 1, 4, lo - 5), "last layer: rows outside the span were read"
    assert not same_after(0, lo), "the window's first row was not read"
    base = step()
    assert not same_after(0, 2), "a sink row was not read"
    base = step()
    assert not same_after(0, pos - 1), "the row before the current one was not read"
    m.close()

    monkeypatch.setenv("LLM_STEP", "graph")
    g = llm.Model(cfg, ts)
    g.prefill(toks)
    g.decode(tok, pos)
    lg = g.logits()
    g.close()
    monkeypatch.setenv("LLM_STEP", "persistent")
    p2 = llm.Model(cfg, ts)
    p2.prefill(toks)
    p2.decode(tok, pos)
    err = float(np.max(np.abs(lg.astype(np.float64) - p2.logits())))
    p2.close()
    assert err <= tol(cfg), f"persistent vs graph with a window: {err:.3e}"
    print(f"[C4 window 1024 + 4 sinks at 4096] persistent vs graph {err:.3e}", flush=True)
