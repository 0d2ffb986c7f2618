"""Pins of how the oracle composes its pinned operations into a layer.

Two parts of the forward pass are not fixed by any single-operation pin:

* where the optional q/k/v biases enter ("The Forward Pass in Java",
  Project 18's forward: added to the three products' outputs, before RoPE);
* which values llama.cpp's rounding points round ("What a Llama model computes,
  and why", section 8: a quantized product's input to 8-bit blocks, an F16
  product's input to binary16, an F32 product's input not at all, q after the
  temperature to binary16, the normalised probabilities to binary16).

The bias pin uses a model whose q and k products are zero, so q and k are the
biases rotated by RoPE, a closed form. The rounding pin rebuilds the forward
pass stage by stage from operations pinned elsewhere (RMSNorm, the
matrix-vector product, RoPE, plain attention with rounded probabilities, silu,
dequantisation) with the input rounding written here from the pages' Q8_0
quantizer and IEEE binary16, and requires the model's logits bit for bit.
"""
import math

import numpy as np

import oracle
import synth
from helpers import f32_tensor

F32, F16, Q8_0 = 0, 1, 8


def _f16(x):
    return np.asarray(x, np.float32).astype(np.float16).astype(np.float32)


def _rot(vec, n_heads, hd, pos, base):
    """RoPE (normal pairs 2i, 2i+1) in float64 with exact angles pos * base^(-2i/hd)."""
    v = np.array(vec, np.float64).reshape(n_heads, hd)
    out = v.copy()
    for i in range(hd // 2):
        a = pos * base ** (-2.0 * i / hd)
        c, s = math.cos(a), math.sin(a)
        out[:, 2 * i] = v[:, 2 * i] * c - v[:, 2 * i + 1] * s
        out[:, 2 * i + 1] = v[:, 2 * i] * s + v[:, 2 * i + 1] * c
    return out.reshape(-1)


def _rms(x, eps):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x) + eps)


def _ulp16(x):
    """Spacing of binary16 values at |x| (subnormal spacing below 2^-14)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -14)))
    return 2.0 ** (e - 10)


# ------------------------------------------------------------- bias placement
def _bias_model():
    d, H, KVH, hd, V = 64, 4, 2, 16, 64
    cfg = synth.ModelConfig("bias-pin", dim=d, n_layers=1, n_heads=H, n_kv_heads=KVH, head_dim=hd, ffn=32,
                            vocab=V, n_ctx=16, eps=1e-5, rope_base=100.0, qkv_bias=True, seed=61)
    kvd = KVH * hd
    arr = {
        "token_embd.weight": synth.normal(61, "embd", V * d, std=1.0),
        "blk.0.attn_norm.weight": np.ones(d, np.float32),
        "blk.0.attn_q.weight": np.zeros(d * d, np.float32),
        "blk.0.attn_k.weight": np.zeros(kvd * d, np.float32),
        "blk.0.attn_v.weight": synth.normal(61, "wv", kvd * d, std=0.3),
        "blk.0.attn_q.bias": synth.normal(61, "bq", d, std=1.0),
        "blk.0.attn_k.bias": synth.normal(61, "bk", kvd, std=1.0),
        "blk.0.attn_v.bias": synth.normal(61, "bv", kvd, std=1.0),
        "blk.0.attn_output.weight": np.eye(d, dtype=np.float32).reshape(-1),
        "blk.0.ffn_norm.weight": np.ones(d, np.float32),
        "blk.0.ffn_gate.weight": np.zeros(32 * d, np.float32),
        "blk.0.ffn_up.weight": synth.normal(61, "up", 32 * d, std=0.3),
        "blk.0.ffn_down.weight": synth.normal(61, "down", d * 32, std=0.3),
        "output_norm.weight": np.ones(d, np.float32),
        "output.weight": np.eye(d, dtype=np.float32).reshape(-1),
    }
    ts = [f32_tensor(name, arr[name], ne) for (name, _, ne, _) in synth.tensor_specs(cfg)]
    return cfg, arr, ts


def test_bias_enters_after_the_product_and_before_rope():
    cfg, arr, ts = _bias_model()
    d, H, KVH, hd = cfg.dim, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    kvd, G = KVH * hd, H // KVH
    E = arr["token_embd.weight"].reshape(cfg.vocab, d)
    Wv = arr["blk.0.attn_v.weight"].reshape(kvd, d).astype(np.float64)
    bq, bk, bv = (arr["blk.0.attn_%s.bias" % n].astype(np.float64) for n in "qkv")
    toks = [5, 40, 17, 63, 2, 29]
    m = oracle.Model(cfg, ts)
    K, Vr = [], []
    for p, tok in enumerate(toks):
        logits = m.forward(tok, p)
        kb, vb = m.kv_read(0, p)
        k_got = np.array([oracle.f16_to_f32(b) for b in kb], np.float64)
        v_got = np.array([oracle.f16_to_f32(b) for b in vb], np.float64)
        # W_k = 0: the stored key is the rotated bias; the value is W_v h + b_v
        k_want = _rot(bk, KVH, hd, p, cfg.rope_base)
        v_want = Wv @ _rms(E[tok], cfg.eps) + bv
        assert np.all(np.abs(k_got - k_want) <= _ulp16(k_want) + 1e-6 * np.abs(k_want)), p
        assert np.all(np.abs(v_got - v_want) <= _ulp16(v_want) + 1e-5), p
        K.append(k_got.reshape(KVH, hd))
        Vr.append(v_got.reshape(KVH, hd))
        # W_q = 0: q is the rotated bias; W_o = I, the FFN adds zero (gate 0),
        # output = I with unit gains: logits = rmsnorm(E[tok] + attention)
        q = _rot(bq, H, hd, p, cfg.rope_base).reshape(H, hd)
        heads = np.zeros((H, hd))
        for h in range(H):
            g = h // G
            sc = np.array([q[h] @ K[t][g] for t in range(p + 1)]) / math.sqrt(hd)
            a = np.exp(sc - sc.max())
            a /= a.sum()
            heads[h] = sum(a[t] * Vr[t][g] for t in range(p + 1))
        want = _rms(E[tok].astype(np.float64) + heads.reshape(-1), cfg.eps)
        np.testing.assert_allclose(logits, want, rtol=2e-5, atol=2e-5, err_msg=f"position {p}")
    m.close()


# ------------------------------------------------- rounding-mode composition
def _q8_round(x):
    """A product input rounded as a Q8_0 block sequence: per 32 values the scale
    d = max|x| / 127 (float), codes = x * (1/d) rounded half away from zero,
    values = binary16(d) * code (float)."""
    x = np.asarray(x, np.float32).reshape(-1, 32)
    out = np.empty_like(x)
    for b in range(x.shape[0]):
        d = np.float32(np.max(np.abs(x[b]))) / np.float32(127)
        inv = np.float32(1) / d if d > 0 else np.float32(0)
        t = (x[b] * inv).astype(np.float64)
        code = np.sign(t) * np.floor(np.abs(t) + 0.5)
        out[b] = np.float32(np.float16(d)) * code.astype(np.float32)
    return out.reshape(-1)


def _round_for(x, dt):
    if dt == Q8_0:
        return _q8_round(x)
    if dt == F16:
        return _f16(x)
    return np.asarray(x, np.float32)  # F32 weights see the input as it is


# per-layer types of q, k, v, o, gate, up, down: every product kind meets every type
_LAYER_TYPES = [
    dict(attn_q=Q8_0, attn_k=F16, attn_v=F32, attn_output=Q8_0, ffn_gate=F16, ffn_up=Q8_0, ffn_down=F32),
    dict(attn_q=F32, attn_k=Q8_0, attn_v=F16, attn_output=F16, ffn_gate=Q8_0, ffn_up=F32, ffn_down=Q8_0),
    dict(attn_q=F16, attn_k=F32, attn_v=Q8_0, attn_output=F32, ffn_gate=F32, ffn_up=F16, ffn_down=F16),
]


def _mixed_model():
    cfg = synth.ModelConfig("rounding-pin", dim=128, n_layers=3, n_heads=4, n_kv_heads=2, head_dim=32, ffn=224,
                            vocab=300, n_ctx=16, eps=1e-5, rope_base=10000.0, gain_std=0.1, out_dtype="f16",
                            attn_temp_scale=0.7, attn_temp_len=2, numerics=1, weight_std=0.1, q8_scale_std=0.004,
                            seed=62)
    ts = []
    for name, dt, ne, kind in synth.tensor_specs(cfg):
        if kind == "matrix" and name.startswith("blk."):
            layer, what = int(name.split(".")[1]), name.split(".")[2]
            dt = _LAYER_TYPES[layer][what]
        ts.append(synth.gen_tensor(cfg.seed, name, dt, ne, kind, cfg))
    return cfg, ts


def test_rounding_mode_rounds_each_product_input_for_its_weight_type():
    cfg, ts = _mixed_model()
    by = {t.name: t for t in ts}
    d, H, KVH, hd, f = cfg.dim, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn
    kvd = KVH * hd

    def mat(name):
        t = by[name]
        return oracle.dequantize(t.dtype, t.data, t.n), t.dtype, t.ne[1], t.ne[0]

    def prod(name, x):
        w, dt, rows, cols = mat(name)
        return oracle.matvec(w, _round_for(x, dt), rows, cols)

    gain = lambda n: by[n].data.view(np.float32)
    E = oracle.dequantize(by["token_embd.weight"].dtype, by["token_embd.weight"].data, d * cfg.vocab).reshape(
        cfg.vocab, d)
    m = oracle.Model(cfg, ts)
    kc = [np.zeros((cfg.n_ctx, kvd), np.uint16) for _ in range(cfg.n_layers)]
    vc = [np.zeros((cfg.n_ctx, kvd), np.uint16) for _ in range(cfg.n_layers)]
    toks = synth.prompt(cfg, 5)
    for p, tok in enumerate(toks):
        x = E[tok].copy()
        for l in range(cfg.n_layers):
            pre = f"blk.{l}."
            h = oracle.rmsnorm(x, gain(pre + "attn_norm.weight"), cfg.eps)
            q = oracle.rope(prod(pre + "attn_q.weight", h), H, hd, hd, p, cfg.rope_base, False)
            k = oracle.rope(prod(pre + "attn_k.weight", h), KVH, hd, hd, p, cfg.rope_base, False)
            v = prod(pre + "attn_v.weight", h)
            kc[l][p] = k.astype(np.float16).view(np.uint16)
            vc[l][p] = v.astype(np.float16).view(np.uint16)
            # the temperature first, then binary16 (the attention below rounds
            # only the probabilities when the query is already on the grid)
            qs = _f16(np.float32(oracle.attn_temp(p, cfg.attn_temp_scale, cfg.attn_temp_len)) * q)
            att = oracle.attention(qs, kc[l], vc[l], H, KVH, hd, p, round16=True)
            x = x + prod(pre + "attn_output.weight", att)
            h = oracle.rmsnorm(x, gain(pre + "ffn_norm.weight"), cfg.eps)
            g = prod(pre + "ffn_gate.weight", h)
            u = prod(pre + "ffn_up.weight", h)
            sw = np.array([oracle.silu(z) for z in g], np.float32) * u
            x = x + prod(pre + "ffn_down.weight", sw)
        want = prod("output.weight", oracle.rmsnorm(x, gain("output_norm.weight"), cfg.eps))
        got = m.forward(int(tok), p)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"position {p}"
        for l in range(cfg.n_layers):
            kb, vb = m.kv_read(l, p)
            assert np.array_equal(kb, kc[l][p]) and np.array_equal(vb, vc[l][p])
    # the temperature changes the query from position 2 on, and the rounding moves the logits
    assert oracle.attn_temp(4, cfg.attn_temp_scale, cfg.attn_temp_len) > 1.0
    plain = oracle.Model(cfg.with_(numerics=0), ts)
    base = np.stack([plain.forward(int(t), p) for p, t in enumerate(toks)])
    assert float(np.max(np.abs(base[-1] - got))) > 1e-4
    m.close()
    plain.close()


def test_q8_round_helper_agrees_with_the_quantizer_pins():
    # the helper above against the page-pinned quantizer (tests/test_oracle_pins.py)
    x = synth.normal(63, "x", 32 * 40, std=2.0)
    x[5] = np.float32(0.0)
    x[64:96] = 0.0  # an all-zero block
    np.testing.assert_array_equal(_q8_round(x), oracle.round_input(x, Q8_0))
