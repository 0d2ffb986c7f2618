"""Seeded synthetic tensor sets and prompts for the Llama-family decode path.

This package generates inputs only. It is imported by the tests and by the
bench, which hand the same bytes to the oracle and to the HIP library; it holds
no step of the forward pass. Tensor sets follow GGUF conventions: names as in
llama.cpp (``token_embd.weight``, ``blk.{l}.attn_q.weight`` ...), dims listed
innermost first (``ne = [in, out]`` for a matrix, row ``r`` at ``r * ne0``),
type ids 0 = F32, 1 = F16, 8 = Q8_0 (34-byte blocks of fp16 d + 32 int8).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field, replace
from typing import List, Optional

import numpy as np

from . import build as _build

F32, F16, Q8_0 = 0, 1, 8
DTYPE_IDS = {"f32": F32, "f16": F16, "q8_0": Q8_0}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        u64, i64, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double
        vp = ctypes.c_void_p
        L.synth_fnv1a64.argtypes = [ctypes.c_char_p]
        L.synth_fnv1a64.restype = u64
        L.synth_draw.argtypes = [u64, u64, i64]
        L.synth_draw.restype = u64
        L.synth_f16_bits.argtypes = [ctypes.c_float]
        L.synth_f16_bits.restype = ctypes.c_uint16
        L.synth_normal_f32.argtypes = [u64, u64, dbl, dbl, i64, vp]
        L.synth_normal_f16.argtypes = [u64, u64, dbl, dbl, i64, vp]
        L.synth_q8_0.argtypes = [u64, u64, dbl, i64, vp]
        L.synth_uniform_ids.argtypes = [u64, u64, ctypes.c_int32, i64, vp]
        L.synth_uniform_f32.argtypes = [u64, u64, dbl, dbl, i64, vp]
        _lib = L
    return _lib


def fnv1a64(name: str) -> int:
    return int(lib().synth_fnv1a64(name.encode()))


# --------------------------------------------------------------------------
# Model and workload descriptions
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class ModelConfig:
    name: str
    dim: int
    n_layers: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    n_ctx: int
    eps: float
    rope_base: float
    rope_neox: bool = False
    rope_dims: int = 0  # 0 means head_dim
    mat_dtype: str = "f32"  # attention and FFN matrices
    embd_dtype: str = "f32"  # token_embd (also the output projection when tied)
    out_dtype: str = "f32"  # output.weight when untied
    tied: bool = False
    qkv_bias: bool = False
    rope_freq_factors: bool = False  # a rope_freqs.weight tensor (one divisor per RoPE pair)
    attn_window: int = 0  # attend only the last attn_window positions (0: all)
    attn_sinks: int = 0  # ... plus the first attn_sinks positions (with a window)
    attn_temp_scale: float = 0.0  # query scaled by 1 + scale * ln(floor(pos / attn_temp_len) + 1)
    attn_temp_len: int = 16384
    yarn_factor: float = 0.0  # YaRN context scale factor (0: off)
    yarn_orig_ctx: int = 0  # the original context YaRN's ramp is measured against
    yarn_beta_fast: float = 32.0  # pairs with more turns than this over it keep their angle
    yarn_beta_slow: float = 1.0  # pairs with fewer turns are interpolated by the factor
    numerics: int = 0  # 0: float activations; 1: llama.cpp's rounding points
    weight_std: float = 0.02
    q8_scale_std: float = 0.002
    gain_std: float = 0.0  # norm gains are 1 + N(0, gain_std); 0 gives exactly 1.0
    seed: int = 1
    # workload
    prompt_len: int = 8
    decode_steps: int = 8

    @property
    def n_rot(self) -> int:
        return self.rope_dims or self.head_dim

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def with_(self, **kw) -> "ModelConfig":
        return replace(self, **kw)


# The five workloads: shapes, dtypes and seeds. Seed = workload number.
C1 = ModelConfig("llama2c-288-f32", dim=288, n_layers=6, n_heads=6, n_kv_heads=6, head_dim=48, ffn=768,
                 vocab=32000, n_ctx=256, eps=1e-5, rope_base=10000.0, mat_dtype="f32", embd_dtype="f32",
                 out_dtype="f32", tied=False, seed=1, prompt_len=8, decode_steps=64)
C2 = ModelConfig("tiny-qwen2vocab-f32", dim=256, n_layers=4, n_heads=8, n_kv_heads=2, head_dim=32, ffn=704,
                 vocab=151936, n_ctx=512, eps=1e-6, rope_base=1e6, mat_dtype="f32", embd_dtype="f32",
                 out_dtype="f32", tied=False, seed=2, prompt_len=16, decode_steps=256)
_1B = dict(dim=2048, n_layers=16, n_heads=32, n_kv_heads=8, head_dim=64, ffn=8192, vocab=128256, eps=1e-5)
C3 = ModelConfig("llama-1b-f16", n_ctx=2304, rope_base=500000.0, mat_dtype="f16", embd_dtype="f16", tied=True,
                 seed=3, prompt_len=2048, decode_steps=128, **_1B)
C4 = ModelConfig("llama-1b-q8_0", n_ctx=8320, rope_base=500000.0, mat_dtype="q8_0", embd_dtype="f32", tied=True,
                 seed=4, prompt_len=2048, decode_steps=128, **_1B)
C4_LONG = C4.with_(name="llama-1b-q8_0-ctx8192", prompt_len=8192)
C5 = ModelConfig("qwen2-1b-f16-prefill", n_ctx=1024, rope_base=1e6, rope_neox=True, qkv_bias=True,
                 mat_dtype="f16", embd_dtype="f16", tied=True, seed=5, prompt_len=512, decode_steps=0, **_1B)
CONFIGS = {c.name: c for c in (C1, C2, C3, C4, C4_LONG, C5)}


def tensor_specs(cfg: ModelConfig):
    """(name, dtype, ne, kind) for every tensor of the set, in file order."""
    d, qd, kvd, f = cfg.dim, cfg.q_dim, cfg.kv_dim, cfg.ffn
    md = DTYPE_IDS[cfg.mat_dtype]
    out = [("token_embd.weight", DTYPE_IDS[cfg.embd_dtype], (d, cfg.vocab), "matrix")]
    for l in range(cfg.n_layers):
        p = f"blk.{l}."
        out += [
            (p + "attn_norm.weight", F32, (d,), "gain"),
            (p + "attn_q.weight", md, (d, qd), "matrix"),
            (p + "attn_k.weight", md, (d, kvd), "matrix"),
            (p + "attn_v.weight", md, (d, kvd), "matrix"),
        ]
        if cfg.qkv_bias:
            out += [(p + "attn_q.bias", F32, (qd,), "bias"), (p + "attn_k.bias", F32, (kvd,), "bias"),
                    (p + "attn_v.bias", F32, (kvd,), "bias")]
        out += [
            (p + "attn_output.weight", md, (qd, d), "matrix"),
            (p + "ffn_norm.weight", F32, (d,), "gain"),
            (p + "ffn_gate.weight", md, (d, f), "matrix"),
            (p + "ffn_up.weight", md, (d, f), "matrix"),
            (p + "ffn_down.weight", md, (f, d), "matrix"),
        ]
    out.append(("output_norm.weight", F32, (d,), "gain"))
    if cfg.rope_freq_factors:
        out.append(("rope_freqs.weight", F32, (cfg.n_rot // 2,), "rope_freqs"))
    if not cfg.tied:
        out.append(("output.weight", DTYPE_IDS[cfg.out_dtype], (d, cfg.vocab), "matrix"))
    return out


def nbytes_of(dtype: int, n: int) -> int:
    if dtype == F32:
        return 4 * n
    if dtype == F16:
        return 2 * n
    if dtype == Q8_0:
        assert n % 32 == 0
        return n // 32 * 34
    raise ValueError(dtype)


@dataclass
class Tensor:
    name: str
    dtype: int
    ne: tuple
    data: np.ndarray  # raw bytes of the tensor as stored (uint8, contiguous)

    @property
    def nbytes(self) -> int:
        return int(self.data.nbytes)

    @property
    def n(self) -> int:
        return int(np.prod(self.ne))


def gen_tensor(seed: int, name: str, dtype: int, ne: tuple, kind: str, cfg: Optional[ModelConfig] = None) -> Tensor:
    L = lib()
    n = int(np.prod(ne))
    sid = fnv1a64(name)
    std = cfg.weight_std if cfg is not None else 0.02
    if kind == "rope_freqs":
        # Llama-3-style divisors: 1 for the fastest quarter of the pairs, 32 for
        # the slowest quarter, a linear ramp between (synthetic input data)
        assert dtype == F32
        i = np.arange(n, dtype=np.float64)
        lo, hi = n / 4.0, 3.0 * n / 4.0
        t = np.clip((i - lo) / max(hi - lo, 1.0), 0.0, 1.0)
        raw = (1.0 + 31.0 * t).astype(np.float32).view(np.uint8)
    elif kind == "gain":
        assert dtype == F32
        arr = np.empty(n, np.float32)
        gstd = cfg.gain_std if cfg is not None else 0.0
        if gstd == 0.0:
            arr[:] = 1.0
        else:
            L.synth_normal_f32(seed, sid, 1.0, gstd, n, arr.ctypes.data)
        raw = arr.view(np.uint8)
    elif dtype == F32:
        arr = np.empty(n, np.float32)
        L.synth_normal_f32(seed, sid, 0.0, std, n, arr.ctypes.data)
        raw = arr.view(np.uint8)
    elif dtype == F16:
        arr = np.empty(n, np.uint16)
        L.synth_normal_f16(seed, sid, 0.0, std, n, arr.ctypes.data)
        raw = arr.view(np.uint8)
    elif dtype == Q8_0:
        assert ne[0] % 32 == 0, "Q8_0 blocks run along ne0"
        raw = np.empty(n // 32 * 34, np.uint8)
        qstd = cfg.q8_scale_std if cfg is not None else 0.002
        L.synth_q8_0(seed, sid, qstd, n // 32, raw.ctypes.data)
    else:
        raise ValueError(dtype)
    return Tensor(name, dtype, tuple(ne), raw)


def make_tensor_set(cfg: ModelConfig, seed: Optional[int] = None) -> List[Tensor]:
    s = cfg.seed if seed is None else seed
    return [gen_tensor(s, name, dt, ne, kind, cfg) for (name, dt, ne, kind) in tensor_specs(cfg)]


def prompt(cfg: ModelConfig, n: Optional[int] = None, seed: Optional[int] = None, stream: str = "prompt") -> np.ndarray:
    n = cfg.prompt_len if n is None else n
    out = np.empty(n, np.int32)
    lib().synth_uniform_ids(cfg.seed if seed is None else seed, fnv1a64(stream), cfg.vocab, n, out.ctypes.data)
    return out


def normal(seed: int, stream: str, n: int, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_normal_f32(seed, fnv1a64(stream), mean, std, n, out.ctypes.data)
    return out


def normal_f16_bits(seed: int, stream: str, n: int, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    out = np.empty(n, np.uint16)
    lib().synth_normal_f16(seed, fnv1a64(stream), mean, std, n, out.ctypes.data)
    return out


def uniform(seed: int, stream: str, n: int, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_uniform_f32(seed, fnv1a64(stream), lo, hi, n, out.ctypes.data)
    return out


def q8_0_blocks(seed: int, stream: str, n_blocks: int, scale_std: float = 0.002) -> np.ndarray:
    out = np.empty(n_blocks * 34, np.uint8)
    lib().synth_q8_0(seed, fnv1a64(stream), scale_std, n_blocks, out.ctypes.data)
    return out


def ids(seed: int, stream: str, n: int, vocab: int) -> np.ndarray:
    out = np.empty(n, np.int32)
    lib().synth_uniform_ids(seed, fnv1a64(stream), vocab, n, out.ctypes.data)
    return out


def weight_count(cfg: ModelConfig) -> int:
    return sum(int(np.prod(ne)) for (_, _, ne, _) in tensor_specs(cfg))
