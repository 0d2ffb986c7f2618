"""Pins of the CPU oracle against what the pages fix (no GPU needed).

Each test checks the oracle against something other than itself: values the
pages print for a worked example (tests/golden/*.json, each with its
citation), closed forms, invariants the pages state, exhaustive comparison with
a library's IEEE conversion, or brute force on tiny inputs.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from conftest import golden
from helpers import (SMALL, SMALL_F16, SMALL_MHA, SMALL_NEOX_BIAS, SMALL_PARTIAL_ROPE, SMALL_Q8, SMALL_SPAN_ALL, drop,
                     f32_tensor, replace_tensors, selftest_config, selftest_tensors)


def f32(x):
    return np.float32(x)


def near(actual, printed, digits):
    """`printed` is a value the pages print with `digits` decimals."""
    return abs(float(actual) - float(printed)) <= 0.5 * 10.0 ** (-digits) + 1e-12


# ------------------------------------------------------------------ RMSNorm
def test_rmsnorm_printed_values_bit_exact():
    g = golden("rmsnorm.json")
    for case in g["cases"]:
        y = oracle.rmsnorm(np.array(case["x"], np.float32), np.array(case["w"], np.float32), case["eps"])
        expect = np.array([np.float32(s) for s in case["y"]], np.float32)
        assert np.array_equal(y.view(np.uint32), expect.view(np.uint32)), (case, y)


def test_rmsnorm_eps_dominates_small_input():
    c = golden("rmsnorm.json")["constant_1e-4"]
    x = np.full(c["n"], c["value"], np.float32)
    y = oracle.rmsnorm(x, np.ones_like(x), c["eps"])
    rms = math.sqrt(float(np.sum(y.astype(np.float64) ** 2)) / y.size)
    assert near(rms, c["rms_after"], c["digits"])


@pytest.mark.parametrize("c", [0.3, -2.5, 7.0, 1e-3])
def test_rmsnorm_constant_input_closed_form(c):
    # x = c everywhere: y = g * c / sqrt(c^2 + eps) (exact in real arithmetic).
    n, eps = 64, 1e-5
    g = synth.normal(3, "gain", n, std=0.3, mean=1.0)
    y = oracle.rmsnorm(np.full(n, c, np.float32), g, eps)
    ref = g.astype(np.float64) * c / math.sqrt(float(np.float32(c)) ** 2 + float(np.float32(eps)))
    np.testing.assert_allclose(y, ref, rtol=3e-7, atol=0)


def test_rmsnorm_constant_input_eps0_returns_gain():
    # With eps = 0 and |c| a power of two the output is exactly g * sign(c).
    g = synth.normal(4, "gain", 32, std=0.3, mean=1.0)
    for c in (0.25, -4.0):
        y = oracle.rmsnorm(np.full(32, c, np.float32), g, 0.0)
        assert np.array_equal(y, (g * np.float32(np.sign(c))).astype(np.float32))


# ------------------------------------------------------------------ matvec
def test_matvec_gguf_order():
    g = golden("matvec.json")
    out = oracle.matvec(np.array(g["w"], np.float32), np.array(g["x"], np.float32), g["dims"][1], g["dims"][0])
    assert out.tolist() == g["out"]
    assert out.tolist() != g["out_if_read_as_columns"]


def test_matvec_error_bound_vs_float64():
    # Sequential summation: |fl(dot) - dot| <= gamma_n * sum |w_i x_i|, gamma_n = n u / (1 - n u).
    rows, cols = 37, 301
    w = synth.normal(5, "w", rows * cols)
    x = synth.normal(5, "x", cols)
    out = oracle.matvec(w, x, rows, cols).astype(np.float64)
    W = w.reshape(rows, cols).astype(np.float64)
    exact = W @ x.astype(np.float64)
    u = 2.0 ** -24
    gamma = cols * u / (1 - cols * u)
    bound = gamma * (np.abs(W) @ np.abs(x.astype(np.float64))) + 1e-30
    assert np.all(np.abs(out - exact) <= bound)


def test_matmul_rows_equal_matvec_bit_exact():
    rows, cols, n = 29, 77, 5
    w = synth.normal(6, "w", rows * cols)
    x = synth.normal(6, "x", n * cols)
    y = oracle.matmul(w, x, n, rows, cols)
    for t in range(n):
        assert np.array_equal(y[t], oracle.matvec(w, x[t * cols:(t + 1) * cols], rows, cols))


# ------------------------------------------------------------------ RoPE
def test_rope_printed_values():
    g = golden("rope.json")
    x = np.array(g["x"], np.float32)
    normal = oracle.rope(x, 1, g["head_dim"], g["n_rot"], g["pos"], g["base"], False)
    neox = oracle.rope(x, 1, g["head_dim"], g["n_rot"], g["pos"], g["base"], True)
    for a, b in zip(normal, g["normal"]):
        assert near(a, b, g["digits"])
    for a, b in zip(neox, g["neox"]):
        assert near(a, b, g["digits"])


def test_rope_layouts_are_one_rotation_bit_exact():
    g = golden("rope.json")
    x = np.array(g["x"], np.float32)
    perm = np.array(g["interleave"])
    neox = oracle.rope(x, 1, 8, 8, 1, g["base"], True)
    normal_of_perm = oracle.rope(x[perm], 1, 8, 8, 1, g["base"], False)
    assert np.array_equal(normal_of_perm.view(np.uint32), neox[perm].view(np.uint32))
    # the same at a larger size and position, on random values
    v = synth.normal(7, "rope", 64)
    perm64 = np.stack([np.arange(32), np.arange(32) + 32], 1).reshape(-1)
    a = oracle.rope(v, 1, 64, 64, 1234, 500000.0, True)
    b = oracle.rope(v[perm64], 1, 64, 64, 1234, 500000.0, False)
    assert np.array_equal(b.view(np.uint32), a[perm64].view(np.uint32))


def test_rope_position_zero_is_identity_and_angles():
    g = golden("rope.json")
    x = np.array(g["x"], np.float32)
    for neox in (False, True):
        assert np.array_equal(oracle.rope(x, 1, 8, 8, 0, g["base"], neox), x)
    c, s = oracle.rope_cos_sin(1, 8, g["base"])
    theta = np.arctan2(s.astype(np.float64), c.astype(np.float64))
    np.testing.assert_allclose(theta, g["angles"], rtol=1e-6)


def test_rope_float_recurrence_closed_form():
    # theta_i = pos * s^i with s = (float)base^(-2/n) and every product rounded to float.
    pos, n, base = 4097, 64, 500000.0
    c, s = oracle.rope_cos_sin(pos, n, base)
    scale = np.float32(base ** (-2.0 / n))
    th = np.float32(pos)
    for i in range(n // 2):
        assert c[i] == np.float32(math.cos(float(th))) and s[i] == np.float32(math.sin(float(th)))
        th = np.float32(th * scale)


def test_rope_preserves_pair_norms_and_partial_dims():
    v = synth.normal(8, "rope-norm", 4 * 64)
    for neox in (False, True):
        r = oracle.rope(v, 4, 64, 32, 777, 10000.0, neox)
        for h in range(4):
            a, b = v[h * 64:(h + 1) * 64].astype(np.float64), r[h * 64:(h + 1) * 64].astype(np.float64)
            for i in range(16):
                ia, ib = (i, i + 16) if neox else (2 * i, 2 * i + 1)
                n0 = math.hypot(a[ia], a[ib])
                assert abs(math.hypot(b[ia], b[ib]) - n0) <= 4e-7 * max(n0, 1e-30) + 1e-12
            assert np.array_equal(r[h * 64 + 32:(h + 1) * 64], v[h * 64 + 32:(h + 1) * 64])


@pytest.mark.parametrize("neox", [False, True])
def test_rope_dot_depends_on_position_difference(neox):
    q = synth.normal(9, "q", 64)
    k = synth.normal(9, "k", 64)
    ref = None
    for shift in (0, 1, 17, 300):
        qa = oracle.rope(q, 1, 64, 64, 40 + shift, 10000.0, neox).astype(np.float64)
        kb = oracle.rope(k, 1, 64, 64, 13 + shift, 10000.0, neox).astype(np.float64)
        d = float(qa @ kb)
        ref = d if ref is None else ref
        assert abs(d - ref) <= 2e-5 * (np.linalg.norm(q) * np.linalg.norm(k))


# ------------------------------------------------------------ RoPE frequency factors
# "What a Llama model computes, and why", sections 2.4 and 6: theta_i = p *
# base^(-2i/n) / f_i, one divisor per pair from rope_freqs.weight; factor 1
# keeps a pair's angle, the slow pairs are slowed by the scaling factor.
def _ramp(n):
    i = np.arange(n, dtype=np.float64)
    return (1.0 + 31.0 * np.clip((i - n / 4) / (n / 2), 0.0, 1.0)).astype(np.float32)


def test_rope_factor_one_keeps_the_angle_bit_exact():
    for pos in (0, 1, 77, 4097):
        c0, s0 = oracle.rope_cos_sin(pos, 64, 500000.0)
        c1, s1 = oracle.rope_cos_sin(pos, 64, 500000.0, np.ones(32, np.float32))
        assert np.array_equal(c0.view(np.uint32), c1.view(np.uint32))
        assert np.array_equal(s0.view(np.uint32), s1.view(np.uint32))


def test_rope_factor_angles_closed_form():
    # small positions keep every angle below pi, so atan2 recovers it; the
    # reference is the formula in double, independent of the float recurrence
    f = _ramp(32)
    for pos in (1, 2, 3):
        c, s = oracle.rope_cos_sin(pos, 64, 500000.0, f)
        got = np.arctan2(s.astype(np.float64), c.astype(np.float64))
        want = pos * 500000.0 ** (-2.0 * np.arange(32) / 64) / f.astype(np.float64)
        np.testing.assert_allclose(got, want, rtol=2e-6, atol=1e-9)


def test_rope_factor_slows_a_pair_by_its_divisor():
    # a pair with divisor 32 turns at position 32 p as the undivided pair does at p
    f = np.full(32, 32.0, np.float32)
    for p in (1, 5, 40):
        c32, s32 = oracle.rope_cos_sin(32 * p, 64, 10000.0, f)
        c1, s1 = oracle.rope_cos_sin(p, 64, 10000.0)
        np.testing.assert_allclose(c32, c1, atol=2e-5)
        np.testing.assert_allclose(s32, s1, atol=2e-5)


@pytest.mark.parametrize("neox", [False, True])
def test_rope_factor_dot_depends_on_position_difference(neox):
    q = synth.normal(19, "q", 64)
    k = synth.normal(19, "k", 64)
    f = _ramp(32)
    ref = None
    for shift in (0, 1, 17, 300):
        qa = oracle.rope(q, 1, 64, 64, 40 + shift, 500000.0, neox, f).astype(np.float64)
        kb = oracle.rope(k, 1, 64, 64, 13 + shift, 500000.0, neox, f).astype(np.float64)
        d = float(qa @ kb)
        ref = d if ref is None else ref
        assert abs(d - ref) <= 2e-5 * (np.linalg.norm(q) * np.linalg.norm(k))


def test_model_with_unit_factors_equals_model_without():
    cfg = SMALL.with_(name="small-unit-freqs")
    ts = synth.make_tensor_set(cfg)
    ones = synth.Tensor("rope_freqs.weight", synth.F32, (cfg.n_rot // 2,),
                        np.ones(cfg.n_rot // 2, np.float32).view(np.uint8))
    a, b = oracle.Model(cfg, ts), oracle.Model(cfg, ts + [ones])
    toks = synth.prompt(cfg, 5)
    for p, t in enumerate(toks):
        la, lb = a.forward(int(t), p), b.forward(int(t), p)
        assert np.array_equal(la.view(np.uint32), lb.view(np.uint32))
    a.close()
    b.close()


def test_model_reads_the_factors():
    cfg = SMALL.with_(name="small-freqs", rope_freq_factors=True)
    ts = synth.make_tensor_set(cfg)
    plain = [t for t in ts if t.name != "rope_freqs.weight"]
    a, b = oracle.Model(cfg, ts), oracle.Model(cfg, plain)
    toks = synth.prompt(cfg, 6)
    diff = 0.0
    for p, t in enumerate(toks):
        diff = max(diff, float(np.max(np.abs(a.forward(int(t), p) - b.forward(int(t), p)))))
    assert diff > 1e-4  # pairs past the first quarter turn slower, so the logits move
    a.close()
    b.close()


# ------------------------------------------------------------ YaRN
# "What a Llama model computes, and why", section 6 names YaRN (Ministral 3:
# factor 16); the ramp and the rescale follow the YaRN paper (Peng et al.,
# 2023). The 64-dim, base 1e6, original-context 16384 case below has
# r_i = 16384 * 1e6^(-i/32) / (2 pi) turns per pair: above 32 up to pair 10,
# below 1 from pair 19, r_11 = 22.59 in between.
YARN16 = (16.0, 16384, 32.0, 1.0)
M16 = 1 + 0.1 * math.log(16)  # 1.2772588722...


def _ulps32(a, b):
    a = np.asarray(a, np.float32).astype(np.float64)
    b = np.asarray(b, np.float32).astype(np.float64)
    return np.abs(a - b) / np.spacing(np.maximum(np.abs(a), np.abs(b)).astype(np.float32)).astype(np.float64)


def test_yarn_ramp_closed_form():
    g = [oracle.yarn_ramp(YARN16, i, 64, 1e6) for i in range(32)]
    assert g[:11] == [1.0] * 11 and g[19:] == [0.0] * 13
    assert abs(g[11] - (22.59 - 1) / 31) < 1e-3
    assert all(x > y for x, y in zip(g[11:19], g[12:20]))


def test_yarn_factor_one_is_plain_rope_bit_exact():
    for pos in (0, 1, 777, 16000):
        c0, s0 = oracle.rope_cos_sin(pos, 64, 1e6)
        c1, s1 = oracle.rope_cos_sin(pos, 64, 1e6, yarn=(1.0, 16384, 32.0, 1.0))
        assert np.array_equal(c0.view(np.uint32), c1.view(np.uint32))
        assert np.array_equal(s0.view(np.uint32), s1.view(np.uint32))


def test_yarn_fast_pairs_keep_their_angle_and_slow_pairs_are_interpolated():
    # fast pairs: m times the plain cos/sin at the same position; slow pairs at
    # position 16 q: m times the plain cos/sin at position q (the float angle
    # recurrence scales exactly by the power of two 16)
    for q in (1, 5, 300, 1000):
        p = 16 * q
        cy, sy = oracle.rope_cos_sin(p, 64, 1e6, yarn=YARN16)
        cp, sp = oracle.rope_cos_sin(p, 64, 1e6)
        cq, sq = oracle.rope_cos_sin(q, 64, 1e6)
        assert _ulps32(cy[:11], np.float32(M16 * cp[:11].astype(np.float64))).max() <= 1
        assert _ulps32(sy[:11], np.float32(M16 * sp[:11].astype(np.float64))).max() <= 1
        assert _ulps32(cy[19:], np.float32(M16 * cq[19:].astype(np.float64))).max() <= 1
        assert _ulps32(sy[19:], np.float32(M16 * sq[19:].astype(np.float64))).max() <= 1
        # every pair keeps norm m
        np.testing.assert_allclose(np.hypot(cy.astype(np.float64), sy), M16, rtol=1e-6)


@pytest.mark.parametrize("neox", [False, True])
def test_yarn_dot_depends_on_position_difference(neox):
    q = synth.normal(40, "q", 2 * 64)
    k = synth.normal(40, "k", 2 * 64)
    dots = []
    for p in (0, 37, 900):
        qr = oracle.rope(q, 2, 64, 64, p + 5, 1e6, neox, yarn=YARN16)
        kr = oracle.rope(k, 2, 64, 64, p, 1e6, neox, yarn=YARN16)
        dots.append(float(np.dot(qr.astype(np.float64), kr)))
    np.testing.assert_allclose(dots, dots[0], rtol=2e-4)
    plain = float(np.dot(oracle.rope(q, 2, 64, 64, 5, 1e6, neox).astype(np.float64),
                         oracle.rope(k, 2, 64, 64, 0, 1e6, neox)))
    assert abs(dots[0]) > 0 and abs(dots[0] - plain) > 1e-3  # the logits are rescaled (m^2) and slow pairs turn slower


def test_model_yarn_factor_one_equals_plain_and_model_reads_yarn():
    ts = synth.make_tensor_set(SMALL)
    toks = synth.prompt(SMALL, 6)
    ref = oracle.Model(SMALL, ts)
    want = [ref.forward(int(t), p) for p, t in enumerate(toks)]
    one = oracle.Model(SMALL.with_(yarn_factor=1.0, yarn_orig_ctx=8), ts)
    got = [one.forward(int(t), p) for p, t in enumerate(toks)]
    assert all(np.array_equal(a.view(np.uint32), b.view(np.uint32)) for a, b in zip(got, want))
    y = oracle.Model(SMALL.with_(yarn_factor=4.0, yarn_orig_ctx=8), ts)
    diff = max(float(np.max(np.abs(y.forward(int(t), p) - w))) for (p, t), w in zip(enumerate(toks), want))
    assert diff > 1e-4
    for m in (ref, one, y):
        m.close()
    for kw in (dict(yarn_factor=0.5, yarn_orig_ctx=8), dict(yarn_factor=4.0), dict(yarn_factor=4.0, yarn_orig_ctx=8,
                                                                                 yarn_beta_fast=1.0)):
        with pytest.raises(Exception):
            oracle.Model(SMALL.with_(**kw), ts)


# ------------------------------------------------------------ llama.cpp's rounding points
# "What a Llama model computes, and why", section 8: a quantized product's input
# is rounded to Q8_0 before the integer dot, an F16 product's input to binary16,
# q to binary16 before q.k, and the probabilities to binary16 before they
# weight V (numerics = 1).
def _q8_fields(raw):
    blocks = raw.reshape(-1, 34)
    d = np.array([oracle.f16_to_f32(int(b[0]) | (int(b[1]) << 8)) for b in blocks], np.float64)
    return d, blocks[:, 2:].view(np.int8).astype(np.int64)


def test_rounded_q8_input_is_its_quantized_blocks():
    x = synth.normal(41, "x", 256) * np.float32(3)
    x[40] = np.float32(-7.5)  # a block whose largest magnitude is negative
    y = oracle.round_input(x, 8)
    d, q = _q8_fields(oracle.quantize_q8_0(x))
    np.testing.assert_array_equal(y, (d[:, None] * q).astype(np.float32).reshape(-1))
    assert np.all(np.abs(q) <= 127) and np.all(np.abs(q).max(1) == 127)
    # within half a step of the block's scale (plus the scale's binary16 rounding)
    amax = np.abs(x.reshape(-1, 32)).max(1).astype(np.float64)
    bound = d / 2 + 127 * np.abs(d - amax / 127) + 1e-9
    assert np.all(np.abs(y.reshape(-1, 32) - x.reshape(-1, 32)) <= bound[:, None])


def test_rounded_f16_input_is_the_library_conversion_and_f32_is_untouched():
    x = synth.normal(42, "x", 512) * np.float32(50)
    np.testing.assert_array_equal(oracle.round_input(x, 1), x.astype(np.float16).astype(np.float32))
    np.testing.assert_array_equal(oracle.round_input(x, 0), x)


def test_q8_product_of_rounded_input_is_the_integer_dot():
    # the product of the dequantized weights with the rounded input equals the
    # integer formulation sum_b d_w d_x sum_j q_w q_x within fp32 summation error
    rows, cols = 7, 96
    w = synth.normal(43, "w", rows * cols) * np.float32(0.5)
    x = synth.normal(43, "x", cols) * np.float32(2)
    wraw = oracle.quantize_q8_0(w)
    wd = oracle.dequantize(8, wraw, rows * cols)
    got = oracle.matvec(wd, oracle.round_input(x, 8), rows, cols)
    dw, qw = _q8_fields(wraw)
    dx, qx = _q8_fields(oracle.quantize_q8_0(x))
    nb = cols // 32
    for r in range(rows):
        exact = sum(dw[r * nb + b] * dx[b] * int(np.dot(qw[r * nb + b], qx[b])) for b in range(nb))
        scale = sum(abs(dw[r * nb + b] * dx[b]) * int(np.abs(qw[r * nb + b]) @ np.abs(qx[b])) for b in range(nb))
        assert abs(got[r] - exact) <= 1e-6 * scale


def test_rounded_attention_brute_force():
    q, kb, vb, H, KVH, hd, P = _span_inputs(44)
    for pos in (0, 6, P - 1):
        out, w = oracle.attention(q, kb, vb, H, KVH, hd, pos, want_weights=True, round16=True)
        K = _f16_vals(kb[:pos + 1].reshape(-1)).reshape(pos + 1, KVH, hd).astype(np.float64)
        V = _f16_vals(vb[:pos + 1].reshape(-1)).reshape(pos + 1, KVH, hd).astype(np.float64)
        Q = q.astype(np.float16).astype(np.float64).reshape(H, hd)
        for h in range(H):
            g = h // (H // KVH)
            sc = K[:, g] @ Q[h] / math.sqrt(hd)
            a = np.exp(sc - sc.max())
            a = (a / a.sum()).astype(np.float16).astype(np.float64)
            np.testing.assert_allclose(w[h], a, rtol=1e-3, atol=1e-7)  # probabilities on the binary16 grid
            assert np.array_equal(w[h].astype(np.float16).astype(np.float32), w[h])
            np.testing.assert_allclose(out[h * hd:(h + 1) * hd], w[h].astype(np.float64) @ V[:, g], rtol=1e-5,
                                       atol=1e-6)
        plain = oracle.attention(q, kb, vb, H, KVH, hd, pos)
        if pos > 0:
            assert not np.array_equal(plain, out)


@pytest.mark.parametrize("cfg", [SMALL, SMALL_F16, SMALL_Q8], ids=lambda c: c.name)
def test_llamacpp_numerics_prefill_rows_equal_token_by_token_bit_exact(cfg):
    cfg = cfg.with_(numerics=1)
    ts = synth.make_tensor_set(cfg)
    toks = synth.prompt(cfg, 9)
    a, b = oracle.Model(cfg, ts), oracle.Model(cfg, ts)
    want = np.stack([a.forward(int(t), p) for p, t in enumerate(toks)])
    got = b.prefill_rows(toks, [8, 0, 4])
    for r, g in zip([8, 0, 4], got):
        assert np.array_equal(g.view(np.uint32), want[r].view(np.uint32))
    plain = oracle.Model(cfg.with_(numerics=0), ts)
    base = np.stack([plain.forward(int(t), p) for p, t in enumerate(toks)])
    diff = float(np.max(np.abs(base - want)))
    assert 0 < diff < 0.5, diff  # the rounding moves the logits, a little
    for m in (a, b, plain):
        m.close()


# ------------------------------------------------------------ silu / SwiGLU
def test_silu_printed_values():
    g = golden("swiglu.json")["silu"]
    for z, y in zip(g["z"], g["y"]):
        assert near(oracle.silu(z), y, g["digits"])


def test_swiglu_worked_block():
    b = golden("swiglu.json")["block"]
    x = np.array(b["x"], np.float32)
    gate = oracle.matvec(np.array(b["gate_w"], np.float32), x, b["ffn"], b["dim"])
    up = oracle.matvec(np.array(b["up_w"], np.float32), x, b["ffn"], b["dim"])
    h = np.array([f32(oracle.silu(g)) * u for g, u in zip(gate, up)], np.float32)
    down = oracle.matvec(np.array(b["down_w"], np.float32), h, b["dim"], b["ffn"])
    for got, want in ((gate, b["gate"]), (up, b["up"]), (h, b["h"]), (down, b["down"])):
        for a, w in zip(got, want):
            assert near(a, w, b["digits"])
    for gv, w in zip(gate, b["silu_gate"]):
        assert near(oracle.silu(gv), w, b["digits"])


# ------------------------------------------------------------ logits / argmax
def test_greedy_choice_and_tie_rule():
    g = golden("greedy.json")
    logits = oracle.matvec(np.array(g["output_w"], np.float32), np.array(g["h"], np.float32), g["vocab"], g["dim"])
    for a, b in zip(logits, g["logits"]):
        assert near(a, b, 3)
    p = np.exp(logits.astype(np.float64) - logits.max())
    p /= p.sum()
    for a, b in zip(p, g["probabilities"]):
        assert near(a, b, 3)
    assert oracle.argmax(logits) == g["token"]
    assert oracle.argmax(np.array(g["tie"]["logits"], np.float32)) == g["tie"]["token"]


def test_argmax_first_strict_maximum_brute_force():
    for seed in range(20):
        v = np.round(synth.normal(seed, "am", 97) * 2).astype(np.float32)  # many ties
        m = v.max()
        assert oracle.argmax(v) == int(np.flatnonzero(v == m)[0])


# ------------------------------------------------------------ attention
def _f16_bits(x):
    return np.array([oracle.f32_to_f16(v) for v in np.asarray(x, np.float32).reshape(-1)], np.uint16)


def _f16_vals(bits):
    return np.array([oracle.f16_to_f32(b) for b in bits], np.float32)


def test_attention_position_zero_returns_v0_with_gqa_mapping():
    g = golden("attention.json")
    H, KVH, hd = g["heads"], g["kv_heads"], g["head_dim"]
    kvd = KVH * hd
    q = synth.normal(10, "q", H * hd)
    k = _f16_bits(synth.normal(10, "k", kvd))
    v = _f16_bits(np.array([0 + 1 + i / 10 for i in range(kvd)], np.float32))
    out, w = oracle.attention(q, k[None], v[None], H, KVH, hd, 0, want_weights=True)
    assert w[:, 0].tolist() == g["pos0"]["weights"]
    vv = _f16_vals(v)
    for h in range(H):
        kv = g["head_to_kv"][h]
        assert np.array_equal(out[h * hd:(h + 1) * hd], vv[kv * hd:(kv + 1) * hd])  # exactly V[0] of its kv head
    for a, b in zip(out[0:2], g["pos0"]["head0_output"]):
        assert near(a, b, 3)
    for a, b in zip(out[4:6], g["pos0"]["head2_output"]):
        assert near(a, b, 3)


def test_attention_weights_sum_to_one_and_brute_force():
    H, KVH, hd, P = 8, 2, 32, 50
    kvd = KVH * hd
    q = synth.normal(11, "q", H * hd) * 3
    kb = _f16_bits(synth.normal(11, "k", P * kvd)).reshape(P, kvd)
    vb = _f16_bits(synth.normal(11, "v", P * kvd)).reshape(P, kvd)
    out, w = oracle.attention(q, kb, vb, H, KVH, hd, P - 1, want_weights=True)
    np.testing.assert_allclose(w.astype(np.float64).sum(1), 1.0, atol=2e-6)
    K = _f16_vals(kb.reshape(-1)).reshape(P, KVH, hd).astype(np.float64)
    V = _f16_vals(vb.reshape(-1)).reshape(P, KVH, hd).astype(np.float64)
    Q = q.reshape(H, hd).astype(np.float64)
    for h in range(H):
        g = h // (H // KVH)
        s = K[:, g, :] @ Q[h] / math.sqrt(hd)
        a = np.exp(s - s.max())
        a /= a.sum()
        np.testing.assert_allclose(w[h], a, rtol=2e-5, atol=1e-7)
        np.testing.assert_allclose(out[h * hd:(h + 1) * hd], a @ V[:, g, :], rtol=2e-5, atol=2e-6)


def test_attention_reads_only_positions_up_to_pos():
    H, KVH, hd, P = 4, 2, 16, 12
    kvd = KVH * hd
    q = synth.normal(12, "q", H * hd)
    kb = _f16_bits(synth.normal(12, "k", P * kvd)).reshape(P, kvd)
    vb = _f16_bits(synth.normal(12, "v", P * kvd)).reshape(P, kvd)
    a = oracle.attention(q, kb, vb, H, KVH, hd, 5)
    kb2, vb2 = kb.copy(), vb.copy()
    kb2[6:] = 0x7c00  # +inf in later rows must not matter
    vb2[6:] = 0x7c00
    assert np.array_equal(a, oracle.attention(q, kb2, vb2, H, KVH, hd, 5))


# ------------------------------------------------------------ attention spans and temperature
# "The Engine" names sliding:N (the last N positions) and sink:s,w (the first s
# positions plus the last w); "What a Llama model computes, and why", section
# 6, gives Mistral 3's query scale 1 + 0.1 ln(floor(p / 16384) + 1).
def _span_inputs(seed, H=4, KVH=2, hd=16, P=16):
    kvd = KVH * hd
    q = synth.normal(seed, "q", H * hd) * 2
    kb = _f16_bits(synth.normal(seed, "k", P * kvd)).reshape(P, kvd)
    vb = _f16_bits(synth.normal(seed, "v", P * kvd)).reshape(P, kvd)
    return q, kb, vb, H, KVH, hd, P


def test_window_covering_the_span_is_full_attention_bit_exact():
    q, kb, vb, H, KVH, hd, P = _span_inputs(30)
    for pos in (0, 5, P - 1):
        full = oracle.attention(q, kb, vb, H, KVH, hd, pos)
        for w, s in ((pos + 1, 0), (P + 7, 0), (2, pos + 1), (1, pos)):
            got = oracle.attention(q, kb, vb, H, KVH, hd, pos, window=w, sinks=s)
            assert np.array_equal(got.view(np.uint32), full.view(np.uint32)), (pos, w, s)


def test_window_of_one_returns_the_current_value_row():
    q, kb, vb, H, KVH, hd, P = _span_inputs(31)
    for pos in (0, 7, P - 1):
        out = oracle.attention(q, kb, vb, H, KVH, hd, pos, window=1, temp_scale=0.3, temp_len=2)
        vv = _f16_vals(vb[pos])
        for h in range(H):
            g = h // (H // KVH)
            assert np.array_equal(out[h * hd:(h + 1) * hd], vv[g * hd:(g + 1) * hd])


@pytest.mark.parametrize("window,sinks", [(3, 0), (3, 2), (4, 1), (2, 5), (6, 3)])
def test_span_equals_full_attention_over_the_kept_rows(window, sinks):
    # the masked attention at pos is the plain attention over a cache that
    # holds only the kept rows, in order: the first `sinks` rows and the last
    # `window` rows up to pos
    q, kb, vb, H, KVH, hd, P = _span_inputs(32)
    for pos in range(P):
        keep = sorted(set(range(min(sinks, pos + 1))) | set(range(max(0, pos - window + 1), pos + 1)))
        got, w = oracle.attention(q, kb, vb, H, KVH, hd, pos, want_weights=True, window=window, sinks=sinks)
        want = oracle.attention(q, kb[keep], vb[keep], H, KVH, hd, len(keep) - 1)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), pos
        off = [t for t in range(pos + 1) if t not in keep]
        assert not np.any(w[:, off])
        np.testing.assert_allclose(w.astype(np.float64).sum(1), 1.0, atol=2e-6)
        assert [oracle.attends(t, pos, window, sinks) for t in range(P)] == [t in keep for t in range(P)]


def test_temperature_closed_form():
    for p in (0, 1, 16383):
        assert oracle.attn_temp(p, 0.1, 16384) == 1.0
    assert oracle.attn_temp(16384, 0.1, 16384) == np.float32(1 + 0.1 * math.log(2))
    assert oracle.attn_temp(32767, 0.1, 16384) == np.float32(1 + 0.1 * math.log(2))
    assert oracle.attn_temp(32768, 0.1, 16384) == np.float32(1 + 0.1 * math.log(3))
    assert oracle.attn_temp(10 ** 6, 0.0, 16384) == 1.0


def test_temperature_scales_the_query():
    q, kb, vb, H, KVH, hd, P = _span_inputs(33)
    pos = P - 1  # floor(15 / 5) + 1 = 4
    tau = np.float32(1 + 0.25 * math.log(4))
    got = oracle.attention(q, kb, vb, H, KVH, hd, pos, temp_scale=0.25, temp_len=5)
    want = oracle.attention((q * tau).astype(np.float32), kb, vb, H, KVH, hd, pos)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    below = oracle.attention(q, kb, vb, H, KVH, hd, 4, temp_scale=0.25, temp_len=5)
    assert np.array_equal(below, oracle.attention(q, kb, vb, H, KVH, hd, 4))


def test_model_span_and_temperature_switch_on_where_the_pages_say():
    # a window of W changes nothing before position W and changes the logits
    # from there on; a temperature changes nothing before its original
    # context; neither changes anything when it covers the whole cache
    base = SMALL_Q8.with_(n_ctx=24)
    ts = synth.make_tensor_set(base)
    toks = synth.prompt(base, 14)
    ref = oracle.Model(base, ts)
    want = [ref.forward(int(t), p) for p, t in enumerate(toks)]
    for cfg, first_change in ((base.with_(attn_window=6), 6), (base.with_(attn_window=6, attn_sinks=2), 8),
                              (base.with_(attn_temp_scale=0.1, attn_temp_len=9), 9),
                              (base.with_(attn_window=24, attn_sinks=3, attn_temp_scale=0.1, attn_temp_len=24), None)):
        m = oracle.Model(cfg, ts)
        got = [m.forward(int(t), p) for p, t in enumerate(toks)]
        for p in range(len(toks)):
            same = np.array_equal(got[p].view(np.uint32), want[p].view(np.uint32))
            assert same == (first_change is None or p < first_change), (cfg, p)
        m.close()
    ref.close()


def test_bad_span_configs_are_rejected():
    ts = synth.make_tensor_set(SMALL)
    for kw in (dict(attn_window=-1), dict(attn_sinks=2), dict(attn_sinks=-1, attn_window=3),
               dict(attn_temp_scale=-0.1), dict(attn_temp_scale=float("inf")), dict(attn_temp_scale=0.1, attn_temp_len=0)):
        with pytest.raises(Exception):
            oracle.Model(SMALL.with_(**kw), ts)


# ------------------------------------------------------------ binary16
def test_f16_printed_values():
    g = golden("f16_values.json")
    xs = [np.float32(np.float32(0.1) * np.float32(i) - np.float32(0.35)) for i in range(12)]
    for x, want in zip(xs, g["f16"]):
        assert near(oracle.f16_to_f32(oracle.f32_to_f16(x)), want, g["digits"])
    assert oracle.f32_to_f16(xs[1]) == int(g["element1_bits"], 16)


def test_f16_matches_ieee_library_conversion():
    # numpy's float16 casts implement IEEE 754 binary16 with round-to-nearest-even.
    allbits = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    ref = allbits.view(np.float16).astype(np.float32)
    got = np.array([oracle.f16_to_f32(int(b)) for b in allbits], np.float32)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite].view(np.uint32), ref[finite].view(np.uint32))
    assert np.all(np.isnan(got[np.isnan(ref)]))
    # encoding: random floats over the whole binary16 range, exact halfway cases and subnormals
    x = np.concatenate([
        synth.normal(13, "f16", 20000) * 100,
        synth.normal(13, "f16s", 20000) * 1e-5,
        synth.uniform(13, "f16u", 20000, -70000, 70000),
        (ref[finite & (np.abs(ref) < 60000)].astype(np.float64)[:-1] +
         np.diff(ref[finite & (np.abs(ref) < 60000)].astype(np.float64)) / 2).astype(np.float32),
    ]).astype(np.float32)
    with np.errstate(over="ignore"):  # values past 65504 become infinity on both sides
        want = x.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16(v) for v in x], np.uint16)
    assert np.array_equal(got, want)


# ------------------------------------------------------------ dequantisation / Q8_0
def _java_cos_row():
    return np.array([np.float32(math.cos(i * 0.7)) * np.float32(0.08) for i in range(64)], np.float32)


def _max_err(a, b):
    return float(np.max(np.abs((a - b).astype(np.float32))))


def test_dequantize_printed_values():
    g = golden("dequantize.json")
    w = _java_cos_row()
    f16 = np.array([oracle.f32_to_f16(v) for v in w], np.uint16)
    q8 = oracle.quantize_q8_0(w)
    cases = {"f32": (0, w.view(np.uint8)), "f16": (1, f16.view(np.uint8)), "q8_0": (8, q8)}
    for key, (dt, raw) in cases.items():
        x = oracle.dequantize(dt, raw, 64)
        assert raw.nbytes == g[key]["bytes"]
        for a, b in zip(x[1:4], g[key]["x123"]):
            assert near(a, b, g["digits"])
        assert near(_max_err(x, w), g[key]["max_error"], g["digits"])
    for n, a, b in g["gib"]:
        assert near(n * 4 / 1024 ** 3, a, 2) and near(n * 34 / 32 / 1024 ** 3, b, 2)


def test_q8_0_blocks_printed_values():
    g = golden("q8_blocks.json")
    x = np.array([np.float32(math.sin(i * 0.3)) * (np.float32(0.1) if i < 32 else np.float32(1.0)) for i in range(128)],
                 np.float32)
    q = oracle.quantize_q8_0(x)
    assert q.nbytes == g["bytes"]
    for b in g["blocks"]:
        at = b["at"]
        d = oracle.f16_to_f32(int(q[at]) | (int(q[at + 1]) << 8))
        assert near(d, b["d"], g["digits"])
        assert q[at + 2:at + 6].view(np.int8).tolist() == b["qs0123"]
    y = oracle.dequantize(8, q, 128)
    for r, row in enumerate(g["rows"]):
        assert near(y[r * 64 + 5], row["element5"], g["digits"])
        assert near(x[r * 64 + 5], row["original5"], g["digits"])
        assert near(_max_err(y[r * 64:(r + 1) * 64], x[r * 64:(r + 1) * 64]), row["max_error"], g["digits"])
    # element 70 sits in block 2 at byte 76 (block 70/32 at 34*(70/32), quant 70%32 after the 2-byte scale)
    assert 70 // 32 == g["element70"]["block"] and 34 * (70 // 32) + 2 + 70 % 32 == g["element70"]["byte"]


def test_gguf_writer_round_trip_errors():
    g = golden("gguf_writer.json")
    w = np.array([np.float32(math.sin(i * 0.37)) * np.float32(0.5) for i in range(64)], np.float32)
    f16 = np.array([oracle.f32_to_f16(v) for v in w], np.uint16)
    q8 = oracle.quantize_q8_0(w)
    for key, dt, raw in (("f32", 0, w.view(np.uint8)), ("f16", 1, f16.view(np.uint8)), ("q8_0", 8, q8)):
        assert raw.nbytes == g[key]["bytes"]
        assert near(_max_err(oracle.dequantize(dt, raw, 64), w), g[key]["max_error"], g["digits"])


def test_q8_0_error_bound():
    # |x - fp16(d) q| <= d/2 + 127 |fp16(d) - d| (+ rounding of x * id), d = amax/127.
    x = synth.normal(14, "q8", 32 * 400) * np.repeat(np.abs(synth.normal(14, "q8s", 400)) + 1e-3, 32)
    q = oracle.quantize_q8_0(x)
    y = oracle.dequantize(8, q, x.size)
    for b in range(400):
        xb = x[32 * b:32 * (b + 1)].astype(np.float64)
        d = float(np.float32(np.float32(np.max(np.abs(x[32 * b:32 * (b + 1)]))) / np.float32(127)))
        dh = oracle.f16_to_f32(int(q[34 * b]) | (int(q[34 * b + 1]) << 8))
        err = np.abs(y[32 * b:32 * (b + 1)].astype(np.float64) - xb)
        assert np.all(err <= d / 2 + 127 * abs(dh - d) + 1e-6 * d)
        assert np.all(np.abs(xb / d - q[34 * b + 2:34 * b + 34].view(np.int8)) <= 0.5 + 1e-5)


def test_q8_0_decode_subnormal_scales_exactly():
    raw = synth.q8_0_blocks(15, "q8sub", 64, scale_std=5e-5)  # many fp16-subnormal scales
    y = oracle.dequantize(8, raw, 64 * 32)
    for b in range(64):
        bits = int(raw[34 * b]) | (int(raw[34 * b + 1]) << 8)
        d = float(np.frombuffer(np.array([bits], np.uint16).tobytes(), np.float16)[0])
        qs = raw[34 * b + 2:34 * b + 34].view(np.int8).astype(np.float64)
        assert np.array_equal(y[32 * b:32 * (b + 1)].astype(np.float64), d * qs)
    assert sum((int(raw[34 * b + 1]) & 0x7c) == 0 for b in range(64)) > 10


# ------------------------------------------------------------ sizes
def test_weight_counts():
    g = golden("sizes.json")
    for key in ("tiny", "qwen_7b"):
        m = g[key]
        hd = m["dim"] // m["heads"]
        kvd = m["kv_heads"] * hd
        assert (hd, kvd, m["heads"] // m["kv_heads"]) == (m["head_dim"], m["kv_dim"], m["group"])
        per = oracle.weights_per_layer(m["dim"], kvd, m["ffn"])
        assert per == m["per_layer"]
        assert m["layers"] * per + 2 * m["vocab"] * m["dim"] + m["dim"] == m["total"]
    # the synthetic tensor set of a tiny-shaped model holds exactly that many weights
    tiny = synth.C2.with_(vocab=g["tiny"]["vocab"], rope_base=5e5, eps=1e-5)
    assert synth.weight_count(tiny) == g["tiny"]["total"]
    b = g["llama_3_2_1b"]
    per = oracle.weights_per_layer(b["dim"], b["kv_heads"] * b["head_dim"], b["ffn"])
    assert round(per / 1e6, 1) == b["weights_per_layer_M"]
    layer_macs = b["layers"] * (per - 2 * b["dim"])
    logit_macs = b["vocab"] * b["dim"]
    assert round(layer_macs / 1e6) == b["layer_macs_M"] and round(logit_macs / 1e6) == b["logit_macs_M"]
    assert round((layer_macs + logit_macs) / 1e9, 3) == b["total_macs_G"]
    assert b["heads"] * b["head_dim"] * 2 * b["layers"] == b["attention_macs_per_position"]
    assert 2 * b["layers"] * b["kv_heads"] * b["head_dim"] * 2 == b["kv_bytes_per_position"]
    assert 2 * b["layers"] * b["heads"] * b["head_dim"] * 2 == b["kv_bytes_without_gqa"]
    t = g["tiny_kv_per_token"]
    vals = 2 * 4 * 2 * 32
    assert (vals, 4 * vals, 2 * vals) == (t["values"], t["f32_bytes"], t["f16_bytes"])


# ------------------------------------------------------------ whole model
def _greedy_selftest(neox):
    g = golden("selftest.json")
    cfg = selftest_config(neox)
    ts = selftest_tensors(cfg)
    cached, uncached = oracle.Model(cfg, ts), oracle.Model(cfg, ts)
    seq = list(g["prompt"])
    calls_c = calls_u = 0
    logits = None
    for p, t in enumerate(seq):
        logits = cached.forward(t, p)
        calls_c += 1
    same = True
    for _ in range(g["steps"]):
        ref = None
        for p, t in enumerate(seq):
            ref = uncached.forward(t, p)
            calls_u += 1
        same &= np.array_equal(logits.view(np.uint32), ref.view(np.uint32))
        seq.append(oracle.argmax(logits))
        logits = cached.forward(seq[-1], len(seq) - 1)
        calls_c += 1
    return seq, same, calls_c, calls_u


def test_cached_decode_equals_recomputation_bit_exact():
    g = golden("selftest.json")
    seqs = []
    for neox in (False, True):
        seq, same, cc, cu = _greedy_selftest(neox)
        assert same is True
        assert (cc, cu) == (g["forward_calls"]["cached"], g["forward_calls"]["uncached"])
        seqs.append(seq)
    assert seqs[0] != seqs[1]  # the RoPE layout alone changes the generated tokens


@pytest.mark.parametrize("cfg", [SMALL, SMALL_F16, SMALL_Q8, SMALL_NEOX_BIAS, SMALL_PARTIAL_ROPE],
                         ids=lambda c: c.name)
def test_prefill_equals_token_by_token_bit_exact(cfg):
    ts = synth.make_tensor_set(cfg)
    toks = synth.prompt(cfg, 11)
    a, b = oracle.Model(cfg, ts), oracle.Model(cfg, ts)
    la = None
    for p, t in enumerate(toks):
        la = a.forward(t, p)
    lb = b.prefill(toks[:4])
    lb = b.prefill(toks[4:5])
    lb = b.prefill(toks[5:])
    assert np.array_equal(la.view(np.uint32), lb.view(np.uint32))
    assert a.kv_len() == b.kv_len() == len(toks)
    for l in range(cfg.n_layers):
        for p in range(len(toks)):
            ka, va = a.kv_read(l, p)
            kb, vb = b.kv_read(l, p)
            assert np.array_equal(ka, kb) and np.array_equal(va, vb)
    # decode after prefill reads the cache the prefill wrote
    assert np.array_equal(a.forward(3, len(toks)), b.forward(3, len(toks)))


@pytest.mark.parametrize("cfg", [SMALL, SMALL_Q8, SMALL_SPAN_ALL], ids=lambda c: c.name)
def test_prefill_rows_equal_token_by_token_logits_bit_exact(cfg):
    # every prompt row has its own next-token logits ("What a Llama model
    # computes, and why", section 4); the batch pass gives each row the logits
    # a token-by-token pass gives it, bit for bit, in any row order
    ts = synth.make_tensor_set(cfg)
    toks = synth.prompt(cfg, 9)
    a, b = oracle.Model(cfg, ts), oracle.Model(cfg, ts)
    want = np.stack([a.forward(int(t), p) for p, t in enumerate(toks)])
    rows = [8, 0, 3, 3, 5]
    got = b.prefill_rows(toks, rows)
    for r, g in zip(rows, got):
        assert np.array_equal(g.view(np.uint32), want[r].view(np.uint32))
    assert b.kv_len() == len(toks)
    c = oracle.Model(cfg, ts)
    assert np.array_equal(c.prefill(toks).view(np.uint32), want[-1].view(np.uint32))
    with pytest.raises(ValueError):
        c.prefill_rows(toks, [len(toks)])
    a.close()
    b.close()
    c.close()


def test_reset_and_rewind():
    cfg = SMALL
    ts = synth.make_tensor_set(cfg)
    m = oracle.Model(cfg, ts)
    toks = synth.prompt(cfg, 6)
    first = m.prefill(toks)
    m.reset()
    assert m.kv_len() == 0
    assert np.array_equal(m.prefill(toks), first)
    m.forward(5, 2)  # rewind: rewrite position 2
    assert m.kv_len() == 3
    with pytest.raises(ValueError):
        m.forward(5, 4)  # beyond len


def _np_rmsnorm(x, g, eps):
    x = x.astype(np.float64)
    return x / np.sqrt(np.mean(x * x) + eps) * g


def test_reduction_without_blocks_is_norm_and_projection():
    # W_o = 0 and W_down = 0: every layer adds zero, so logits = W_out rmsnorm(E[token]).
    for cfg in (SMALL, SMALL_F16):
        ts = synth.make_tensor_set(cfg)
        zero = {}
        for l in range(cfg.n_layers):
            zero[f"blk.{l}.attn_output.weight"] = np.zeros(cfg.q_dim * cfg.dim, np.float32)
            zero[f"blk.{l}.ffn_down.weight"] = np.zeros(cfg.ffn * cfg.dim, np.float32)
        ts2 = replace_tensors(ts, **{k.replace(".", "__"): v for k, v in zero.items()})
        m = oracle.Model(cfg, ts2)
        by = {t.name: t for t in ts2}
        E = oracle.dequantize(by["token_embd.weight"].dtype, by["token_embd.weight"].data, cfg.dim * cfg.vocab)
        E = E.reshape(cfg.vocab, cfg.dim)
        W = E if cfg.tied else oracle.dequantize(by["output.weight"].dtype, by["output.weight"].data,
                                                 cfg.dim * cfg.vocab).reshape(cfg.vocab, cfg.dim)
        g = by["output_norm.weight"].data.view(np.float32)
        for pos, tok in enumerate([0, 999, 17]):
            logits = m.forward(tok, pos)
            ref = W.astype(np.float64) @ _np_rmsnorm(E[tok], g, cfg.eps)
            np.testing.assert_allclose(logits, ref, rtol=1e-5, atol=1e-5)


def test_reduction_first_position_attention_returns_v():
    # One layer, H = KVH, W_v = W_o = identity, W_down = 0, no gains: at position 0
    # attention returns f16(v) exactly, so x1 = x + f16(rmsnorm(x)).
    d = 64
    cfg = synth.ModelConfig("ident", dim=d, n_layers=1, n_heads=4, n_kv_heads=4, head_dim=16, ffn=32, vocab=50,
                            n_ctx=8, eps=1e-5, rope_base=10000.0, seed=21)
    ts = synth.make_tensor_set(cfg)
    eye = np.eye(d, dtype=np.float32).reshape(-1)
    ts = replace_tensors(ts, **{"blk.0.attn_v.weight": eye, "blk.0.attn_output.weight": eye,
                                "blk.0.ffn_down.weight": np.zeros(32 * d, np.float32)})
    m = oracle.Model(cfg, ts)
    by = {t.name: t for t in ts}
    E = by["token_embd.weight"].data.view(np.float32).reshape(cfg.vocab, d)
    Wout = by["output.weight"].data.view(np.float32).reshape(cfg.vocab, d)
    tok = 7
    h = oracle.rmsnorm(E[tok], np.ones(d, np.float32), cfg.eps)
    vh = np.array([oracle.f16_to_f32(oracle.f32_to_f16(v)) for v in h], np.float32)
    x1 = E[tok].astype(np.float64) + vh
    ref = Wout.astype(np.float64) @ _np_rmsnorm(x1, 1.0, cfg.eps)
    np.testing.assert_allclose(m.forward(tok, 0), ref, rtol=2e-5, atol=2e-5)


def test_reduction_ffn_only():
    # W_o = 0: the layer is x + W_down (silu(W_gate h) * (W_up h)), h = rmsnorm(x) g_ffn.
    cfg = SMALL.with_(n_layers=1, seed=22)
    ts = synth.make_tensor_set(cfg)
    ts = replace_tensors(ts, **{"blk.0.attn_output.weight": np.zeros(cfg.q_dim * cfg.dim, np.float32)})
    by = {t.name: t for t in ts}
    m = oracle.Model(cfg, ts)
    f = lambda n: by[n].data.view(np.float32).astype(np.float64)
    E = f("token_embd.weight").reshape(cfg.vocab, cfg.dim)
    G = f("blk.0.ffn_gate.weight").reshape(cfg.ffn, cfg.dim)
    U = f("blk.0.ffn_up.weight").reshape(cfg.ffn, cfg.dim)
    D = f("blk.0.ffn_down.weight").reshape(cfg.dim, cfg.ffn)
    tok = 123
    h = _np_rmsnorm(E[tok], f("blk.0.ffn_norm.weight"), cfg.eps)
    gz = G @ h
    x1 = E[tok] + D @ ((gz / (1 + np.exp(-gz))) * (U @ h))
    ref = f("output.weight").reshape(cfg.vocab, cfg.dim) @ _np_rmsnorm(x1, f("output_norm.weight"), cfg.eps)
    np.testing.assert_allclose(m.forward(tok, 0), ref, rtol=1e-4, atol=1e-4)


def test_missing_and_malformed_tensors_are_rejected():
    ts = synth.make_tensor_set(SMALL)
    with pytest.raises(ValueError):
        oracle.Model(SMALL, drop(ts, "blk.1.ffn_up.weight"))
    bad = [f32_tensor(t.name, np.zeros(3, np.float32), (3,)) if t.name == "blk.0.attn_norm.weight" else t for t in ts]
    with pytest.raises(ValueError):
        oracle.Model(SMALL, bad)
    # GQA and MHA shapes both load
    oracle.Model(SMALL_MHA, synth.make_tensor_set(SMALL_MHA))
