"""The integer matrix-core prefill of llama.cpp's rounding points (needs an MI355X).

With numerics = 1 and Q8_0 layer matrices the prompt pass rounds each
product's input rows to Q8_0 blocks and multiplies the codes as integers
("What a Llama model computes, and why", sections 5 and 8): each 32-deep block's
int32 sum of code products, times the weight and input block scales, joins the
fp32 sum. That equals the oracle's float product of the rounded input with the
dequantized weights up to fp32 rounding, so:

  - at the 1B shape, layer 0's K and V rows of prompt positions (the first
    product of the pass, before any attention) are within 2 binary16 ulps of the
    oracle's;
  - on a medium model whose prompt spans three 128-row tiles with a ragged tail
    and whose products split K (an odd number of steady K steps among them),
    layer 0's K and V of all 300 prompt positions are within 2 binary16 ulps of
    the oracle's. Past layer 0 the GPU is held to the oracle's own spread: the
    oracle's two other builds (every dot product summed in the other order;
    every sum accumulated in double) are two more valid evaluations, and with
    Q8_0 inputs a last-bit difference before a product can move one of its
    8-bit codes by a whole step, so they differ from the oracle by a median
    1.5e-2 and up to about 5e-2 in a logit on this prompt ("What a Llama model
    computes, and why", section 8: implementations that differ only in
    summation order drift apart). The GPU's per-row max |dlogit| must have a
    median and a 90th percentile within 1.5 times the builds' (the larger of
    the two), and every row must lie within max(tolerance, 1.5 times the
    largest row distance of either build); each layer's K/V at sampled
    positions likewise within max(tolerance, 1.5 times the builds' largest
    distance in that layer). A wrong block scale, tile or K step moves whole
    rows by far more than that.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import SMALL_F16_RND, SMALL_Q8, SMALL_Q8_RND
from test_gpu_fullsize import _row, _tensors_by_name, check_layer0_kv
from test_gpu_fullsize_oracle import _kv_dist
from test_gpu_parity import tol

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import llama_family_decode_amd as llm

MEDIUM_Q8_RND = SMALL_Q8_RND.with_(name="medium-q8_0-llamacpp", dim=512, n_heads=8, n_kv_heads=2, head_dim=64,
                                   ffn=1408, n_ctx=400, seed=41)


def test_prefill_int8_selects_the_integer_products():
    for cfg, want in ((SMALL_Q8_RND, 1), (SMALL_Q8, 0), (SMALL_F16_RND, 0)):
        m = llm.Model(cfg, synth.make_tensor_set(cfg))
        assert llm.llm_op_prefill_int8(m.ctx) == want, cfg.name
        m.close()


def test_int8_prefill_layer0_rows_1b():
    cfg = synth.C4.with_(name="llama-1b-q8_0-llamacpp", numerics=1)
    ts = synth.make_tensor_set(cfg)
    T = _tensors_by_name(ts)
    toks = synth.prompt(cfg, 2048)
    m = llm.Model(cfg, ts)
    assert llm.llm_op_prefill_int8(m.ctx) == 1
    m.prefill(toks)
    rows = [0, 1, 127, 128, 777, 1500, 2047]
    w0 = check_layer0_kv(cfg, T, m, [(p, int(toks[p])) for p in rows], 2.0)
    m.close()
    print(f"[{cfg.name}] layer-0 K/V of prompt rows within {w0} binary16 ulps", flush=True)


def _oracle_rows(cfg, ts, toks, positions, variant="", rows=None):
    m = oracle.Model(cfg, ts, variant=variant)
    lg = m.prefill_rows(toks, list(range(len(toks))) if rows is None else rows).astype(np.float64)
    kv = {(l, p): m.kv_read(l, p) for l in range(cfg.n_layers) for p in positions}
    m.close()
    return lg, kv


def test_int8_prefill_medium_against_the_oracle():
    cfg = MEDIUM_Q8_RND
    ts = synth.make_tensor_set(cfg)
    n = 300
    toks = synth.prompt(cfg, n)
    m = llm.Model(cfg, ts)
    assert llm.llm_op_prefill_int8(m.ctx) == 1
    got = m.prefill_rows(toks).astype(np.float64)
    assert np.all(np.isfinite(got))
    w0 = check_layer0_kv(cfg, _tensors_by_name(ts), m, [(p, int(toks[p])) for p in range(n)], 2.0)
    positions = (0, 1, 127, 128, 255, 256, 299)
    want, wkv = _oracle_rows(cfg, ts, toks, positions)
    stats = []
    kv_spread = {k: 0.0 for k in wkv}
    for v in ("desc", "f64"):
        lg, kv = _oracle_rows(cfg, ts, toks, positions, v)
        e = np.abs(lg - want).max(axis=1)
        stats.append((np.median(e), np.percentile(e, 90), e.max()))
        for k in kv:
            kv_spread[k] = max([kv_spread[k]] + [_kv_dist(a, b, cfg.head_dim) for a, b in zip(kv[k], wkv[k])])
    stats = np.array(stats)
    t = tol(cfg)
    err = np.abs(got - want).max(axis=1)
    med, p90 = 1.5 * float(np.max(stats[:, 0])), 1.5 * float(np.max(stats[:, 1]))
    bar = max(t, 1.5 * float(np.max(stats[:, 2])))
    assert np.median(err) <= med, f"median row |dlogit| {np.median(err):.3e} > {med:.3e}"
    assert np.percentile(err, 90) <= p90, f"90th percentile row |dlogit| {np.percentile(err, 90):.3e} > {p90:.3e}"
    bad = np.flatnonzero(err > bar)
    assert bad.size == 0, f"rows {bad[:8].tolist()}: max |dlogit| {err[bad[:8]].tolist()} > {bar:.3e}"
    ratio = 0.0
    for (l, p), (ko, vo) in wkv.items():
        kb = max(t, 1.5 * max(v for (l2, _), v in kv_spread.items() if l2 == l))
        for a_bits, b_bits in zip(m.kv_read(l, p), (ko, vo)):
            d = _kv_dist(a_bits, b_bits, cfg.head_dim, slack_ulps=2)
            assert d <= kb, f"K/V of layer {l} at position {p} differ from the oracle by {d:.3e} > {kb:.3e}"
            ratio = max(ratio, d / kb)
    m.close()
    print(f"[{cfg.name}] layer-0 K/V within {w0:.0f} ulps; row |dlogit| median {np.median(err):.3e} "
          f"(oracle builds {stats[:, 0].max():.3e}), max {err.max():.3e} (builds {stats[:, 2].max():.3e}); "
          f"K/V {ratio:.2f} of the bar", flush=True)


def test_int8_prefill_across_chunks():
    # A prompt of one whole prefill chunk plus a ragged 52 rows: the second
    # chunk's products reuse the codes buffers and attend the first chunk's
    # cache. Layer-0 K/V on both sides of the boundary within 2 binary16 ulps of
    # the oracle's; the logits of rows on both sides, and every layer's K/V
    # there, within max(tolerance, 1.5 times the largest distance of the
    # oracle's two other builds) as above.
    cfg = MEDIUM_Q8_RND.with_(name="medium-q8_0-llamacpp-2chunks", n_ctx=2200)
    chunk = llm.llm_op_prefill_chunk()
    n = chunk + 52
    ts = synth.make_tensor_set(cfg)
    toks = synth.prompt(cfg, n)
    rows = [0, 1000, chunk - 1, chunk, n - 1]
    positions = (0, chunk - 2, chunk - 1, chunk, chunk + 1, n - 1)
    m = llm.Model(cfg, ts)
    assert llm.llm_op_prefill_int8(m.ctx) == 1
    got = m.prefill_rows(toks, rows).astype(np.float64)
    assert np.all(np.isfinite(got))
    w0 = check_layer0_kv(cfg, _tensors_by_name(ts), m, [(p, int(toks[p])) for p in positions], 2.0)
    want, wkv = _oracle_rows(cfg, ts, toks, positions, rows=rows)
    spread, kv_spread = 0.0, {k: 0.0 for k in wkv}
    for v in ("desc", "f64"):
        lg, kv = _oracle_rows(cfg, ts, toks, positions, v, rows=rows)
        spread = max(spread, float(np.abs(lg - want).max()))
        for k in kv:
            kv_spread[k] = max([kv_spread[k]] + [_kv_dist(a, b, cfg.head_dim) for a, b in zip(kv[k], wkv[k])])
    t = tol(cfg)
    bar = max(t, 1.5 * spread)
    err = np.abs(got - want).max(axis=1)
    assert np.all(err <= bar), f"rows {rows}: max |dlogit| {err.tolist()} > {bar:.3e}"
    ratio = 0.0
    for (l, p), (ko, vo) in wkv.items():
        kb = max(t, 1.5 * max(v for (l2, _), v in kv_spread.items() if l2 == l))
        for a_bits, b_bits in zip(m.kv_read(l, p), (ko, vo)):
            d = _kv_dist(a_bits, b_bits, cfg.head_dim, slack_ulps=2)
            assert d <= kb, f"K/V of layer {l} at position {p} differ from the oracle by {d:.3e} > {kb:.3e}"
            ratio = max(ratio, d / kb)
    m.close()
    print(f"[{cfg.name}] layer-0 K/V within {w0:.0f} ulps; max |dlogit| {err.max():.3e} (bar {bar:.3e}); "
          f"K/V {ratio:.2f} of the bar", flush=True)


def _scaled(ts, gain_scale, kv_scale):
    """The tensor set with layer 0's norm gain times gain_scale and the binary16
    block scales of its K and V matrices times kv_scale (powers of two)."""
    out = []
    for t in ts:
        if t.name == "blk.0.attn_norm.weight":
            t = synth.Tensor(t.name, t.dtype, t.ne, (t.data.view(np.float32) * np.float32(gain_scale)).view(np.uint8))
        elif t.name in ("blk.0.attn_k.weight", "blk.0.attn_v.weight"):
            assert t.dtype == synth.Q8_0
            b = t.data.copy().reshape(-1, 34)
            d = b[:, :2].copy().view(np.float16).astype(np.float32) * np.float32(kv_scale)
            b[:, :2] = d.astype(np.float16).view(np.uint8).reshape(-1, 2)
            t = synth.Tensor(t.name, t.dtype, t.ne, b.reshape(-1))
        out.append(t)
    return out


@pytest.mark.parametrize("gain_scale,kv_scale,which", [(2.0 ** -16, 2.0 ** 12, "input"), (2.0 ** 6, 2.0 ** -8, "weight")],
                         ids=["subnormal-input-scales", "subnormal-weight-scales"])
def test_int8_prefill_subnormal_block_scales(gain_scale, kv_scale, which):
    # Q8_0 block scales below binary16's normal range on one side of layer 0's
    # K and V products (all input scales, from a norm gain shrunk by 2^-16; or
    # all K/V weight scales, shrunk by 2^-8), the other side scaled up so the
    # rows stay normal. The product of the two scales must stay exact ("What a
    # Llama model computes, and why", section 5: a Q8_0 value is its code times
    # the block's binary16 scale, subnormals included): layer-0 K/V of all
    # prompt rows within 2 binary16 ulps of the oracle's. A scale flushed to
    # zero would zero whole rows.
    cfg = MEDIUM_Q8_RND.with_(name=f"medium-q8_0-llamacpp-{which}-subnormal")
    ts = _scaled(synth.make_tensor_set(cfg), gain_scale, kv_scale)
    T = _tensors_by_name(ts)
    n = 300
    toks = synth.prompt(cfg, n)
    # the premise: the chosen side's block scales are binary16 subnormals
    tiny = 2.0 ** -14
    if which == "input":
        g = oracle.dequantize(0, T["blk.0.attn_norm.weight"].data, cfg.dim)
        for tok in toks[:8]:
            h = oracle.rmsnorm(_row(T["token_embd.weight"], cfg.dim, int(tok)), g, cfg.eps)
            assert np.abs(h).max() / 127 < tiny
    else:
        for name in ("blk.0.attn_k.weight", "blk.0.attn_v.weight"):
            d = T[name].data.reshape(-1, 34)[:, :2].copy().view(np.float16).astype(np.float64)
            assert np.abs(d).max() < tiny
    m = llm.Model(cfg, ts)
    assert llm.llm_op_prefill_int8(m.ctx) == 1
    m.prefill(toks)
    w0 = check_layer0_kv(cfg, T, m, [(p, int(toks[p])) for p in range(n)], 2.0)
    k, v = m.kv_read(0, n - 1)
    assert np.count_nonzero(k.view(np.float16)) > k.size // 2 and np.count_nonzero(v.view(np.float16)) > v.size // 2
    m.close()
    print(f"[{cfg.name}] layer-0 K/V of {n} prompt rows within {w0:.0f} binary16 ulps", flush=True)
