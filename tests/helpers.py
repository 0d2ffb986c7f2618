"""Shared helpers for the tests: small model configurations and tensor sets."""
from __future__ import annotations

import numpy as np

import synth
from synth import F16, F32, Q8_0, ModelConfig, Tensor


def f32_tensor(name: str, arr: np.ndarray, ne: tuple) -> Tensor:
    a = np.ascontiguousarray(arr, np.float32).reshape(-1)
    assert a.size == int(np.prod(ne))
    return Tensor(name, F32, tuple(ne), a.view(np.uint8))


def f16_tensor(name: str, bits: np.ndarray, ne: tuple) -> Tensor:
    a = np.ascontiguousarray(bits, np.uint16).reshape(-1)
    return Tensor(name, F16, tuple(ne), a.view(np.uint8))


def replace_tensors(ts, **arrays):
    """Return a copy of tensor set `ts` where each named tensor (dots written as
    '__' in keyword names) is replaced by an F32 tensor of the given values."""
    repl = {k.replace("__", "."): v for k, v in arrays.items()}
    out = []
    for t in ts:
        if t.name in repl:
            out.append(f32_tensor(t.name, repl[t.name], t.ne))
        else:
            out.append(t)
    return out


def drop(ts, *names):
    return [t for t in ts if t.name not in names]


# Small models that the oracle runs in milliseconds. Widths are chosen so the
# GPU kernels see several tiles plus a ragged tail (vocab 1000, ffn 352).
SMALL = ModelConfig("small-f32", dim=128, n_layers=2, n_heads=4, n_kv_heads=2, head_dim=32, ffn=352, vocab=1000,
                    n_ctx=96, eps=1e-5, rope_base=10000.0, mat_dtype="f32", embd_dtype="f32", out_dtype="f32",
                    tied=False, gain_std=0.1, seed=11, prompt_len=7, decode_steps=5)
SMALL_F16 = SMALL.with_(name="small-f16", mat_dtype="f16", embd_dtype="f16", tied=True, seed=12)
SMALL_Q8 = SMALL.with_(name="small-q8_0", mat_dtype="q8_0", embd_dtype="f32", tied=True, seed=13)
SMALL_NEOX_BIAS = SMALL.with_(name="small-neox-bias", rope_neox=True, qkv_bias=True, rope_base=1e6, seed=14)
SMALL_PARTIAL_ROPE = SMALL.with_(name="small-partial-rope", rope_dims=16, seed=15)
SMALL_MHA = SMALL.with_(name="small-mha", n_kv_heads=4, seed=16, head_dim=48, dim=192, n_heads=4)
SMALL_FREQS = SMALL.with_(name="small-rope-freqs", rope_freq_factors=True, rope_base=500000.0, seed=17)
# attention spans and temperature ("The Engine": sliding:N, sink:s,w; Mistral 3's
# temperature with a short original context so that small runs cross it)
SMALL_WINDOW = SMALL_Q8.with_(name="small-window", attn_window=5, seed=18)
SMALL_SINKS = SMALL_F16.with_(name="small-sinks", attn_window=4, attn_sinks=2, seed=19)
SMALL_TEMP = SMALL.with_(name="small-temp", attn_temp_scale=0.1, attn_temp_len=4, seed=20)
SMALL_SPAN_ALL = SMALL_NEOX_BIAS.with_(name="small-window-sinks-temp", attn_window=6, attn_sinks=3,
                                      attn_temp_scale=0.5, attn_temp_len=3, seed=21)
# head_dim 64, the matrix-core prefill attention's size, on a small model
SMALL_HD64 = SMALL.with_(name="small-hd64", dim=256, n_heads=4, n_kv_heads=2, head_dim=64, ffn=704, seed=26)
# llama.cpp's rounding points (numerics 1) on each weight type
SMALL_RND = SMALL.with_(name="small-f32-llamacpp", numerics=1, seed=23)
SMALL_F16_RND = SMALL_F16.with_(name="small-f16-llamacpp", numerics=1, seed=24)
SMALL_Q8_RND = SMALL_Q8.with_(name="small-q8_0-llamacpp", numerics=1, seed=25)
# the rounding mode with a window, sinks and the temperature on Q8_0 weights
SMALL_SPAN_RND = SMALL_SPAN_ALL.with_(name="small-span-q8_0-llamacpp", mat_dtype="q8_0", tied=True, numerics=1,
                                      seed=29)
# YaRN with a short original context, so that small heads have fast, ramped and slow pairs
SMALL_YARN = SMALL.with_(name="small-yarn", yarn_factor=4.0, yarn_orig_ctx=400, rope_base=10000.0, seed=22)


def selftest_config(neox: bool) -> ModelConfig:
    """The synthetic model of Project 18's self-test (width 16, 2 layers)."""
    return ModelConfig("selftest-" + ("qwen2" if neox else "llama"), dim=16, n_layers=2, n_heads=4, n_kv_heads=2,
                       head_dim=4, ffn=32, vocab=24, n_ctx=64, eps=1e-5, rope_base=10000.0, rope_neox=neox,
                       mat_dtype="f32", embd_dtype="f32", out_dtype="f32", tied=False, seed=42)


def selftest_tensors(cfg: ModelConfig):
    """Weights N(0, 1/in), as the self-test draws them; both layouts share them."""
    out = []
    for name, dt, ne, kind in synth.tensor_specs(cfg):
        n = int(np.prod(ne))
        if kind == "gain":
            out.append(f32_tensor(name, np.ones(n, np.float32), ne))
        else:
            out.append(f32_tensor(name, synth.normal(cfg.seed, name, n, std=1.0 / np.sqrt(ne[0])), ne))
    return out
