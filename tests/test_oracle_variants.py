"""Pins of the oracle's two other builds (test infrastructure).

liboracle_desc.so and liboracle_f64.so evaluate the same definition as
liboracle.so in another valid way; the full-size tests use how far they move a
workload's logits as the measure of its sensitivity to the rounding of its sums
("What a Llama model computes, and why", section 8: implementations that differ
only in summation order drift apart). These pins fix what each build sums:

* the default build adds fp32 products in fp32, index ascending;
* "desc" adds the same fp32 products index descending;
* "f64" accumulates in double and rounds the sum to float once, in the
  products and in the attention scores alike.

Each case is chosen so that the three orders give three different values, each
the closed form of its own order.
"""
import ctypes
import math

import numpy as np

import oracle
from helpers import SMALL, SMALL_Q8
import synth


def _matvec(variant, w, x, rows, cols):
    L = oracle.lib(variant)
    w = np.ascontiguousarray(w, np.float32)
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(rows, np.float32)
    L.orc_matvec(out.ctypes.data_as(ctypes.c_void_p), w.ctypes.data_as(ctypes.c_void_p),
                 x.ctypes.data_as(ctypes.c_void_p), rows, cols)
    return out


def test_each_build_sums_a_dot_product_in_its_own_order():
    # w . 1 with w = (2^25, 1, -2^25, 1): the spacing of fp32 at 2^25 is 4
    w = np.array([2.0 ** 25, 1.0, -(2.0 ** 25), 1.0], np.float32)
    x = np.ones(4, np.float32)
    # ascending: (2^25 + 1 -> 2^25) - 2^25 + 1 = 1
    assert _matvec("", w, x, 1, 4)[0] == 1.0
    # descending: (1 - 2^25 -> -2^25) + 1 -> -2^25, + 2^25 = 0
    assert _matvec("desc", w, x, 1, 4)[0] == 0.0
    # double: the exact sum 2
    assert _matvec("f64", w, x, 1, 4)[0] == 2.0


def test_the_double_build_accumulates_the_attention_scores_in_double():
    # one head of 4 dims, two cached rows: k_0 = (1, 1, 1, 1), k_1 = 0, v_0 =
    # (1, 1, 1, 1), v_1 = 0; q = (2^25, 1, -2^25, 1). The score of row 0 is
    # q . k_0 / 2: 1/2 in fp32 ascending, 2/2 = 1 in double; row 1 scores 0.
    # The output is then p_0 v_0 with p_0 = e^s / (e^s + 1).
    hd = 4
    q = np.array([2.0 ** 25, 1.0, -(2.0 ** 25), 1.0], np.float32)
    one, zero = oracle.f32_to_f16(1.0), oracle.f32_to_f16(0.0)
    kc = np.array([[one] * hd, [zero] * hd], np.uint16)
    vc = kc.copy()
    for variant, s in (("", 0.5), ("f64", 1.0)):
        L = oracle.lib(variant)
        out = np.empty(hd, np.float32)
        L.orc_attention(out.ctypes.data_as(ctypes.c_void_p), q.ctypes.data_as(ctypes.c_void_p),
                        kc.ctypes.data_as(ctypes.c_void_p), vc.ctypes.data_as(ctypes.c_void_p), 1, 1, hd, 1, None)
        p0 = math.exp(s) / (math.exp(s) + 1.0)
        assert np.allclose(out, p0, rtol=1e-6, atol=0), (variant, out, p0)


def test_the_builds_are_the_same_model_up_to_rounding():
    # the whole forward pass of a two-layer model: every build lands within a
    # few fp32 roundings of the default one, and each really is another build
    for cfg in (SMALL, SMALL_Q8):
        ts = synth.make_tensor_set(cfg)
        toks = synth.prompt(cfg, 6)
        ref = oracle.Model(cfg, ts)
        want = ref.prefill(toks)
        ref.close()
        for variant in ("desc", "f64"):
            m = oracle.Model(cfg, ts, variant=variant)
            got = m.prefill(toks)
            m.close()
            err = float(np.max(np.abs(got.astype(np.float64) - want)))
            assert 0.0 < err < 1e-4, (cfg.name, variant, err)
