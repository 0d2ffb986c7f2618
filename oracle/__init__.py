"""CPU oracle of the Llama-family forward pass (TEST INFRASTRUCTURE ONLY).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It wraps ``liboracle.so`` (plain C, fp32,
built from ``oracle.c``) with ctypes and shares no code with the HIP library.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

from . import build as _build

F32, F16, Q8_0 = 0, 1, 8
_libs = {}


class OrcConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("dim", "n_layers", "n_heads", "n_kv_heads", "head_dim", "ffn", "vocab",
                                               "n_ctx", "rope_dims", "rope_neox")] + [
        ("eps", ctypes.c_float), ("rope_base", ctypes.c_float), ("attn_window", ctypes.c_int32),
        ("attn_sinks", ctypes.c_int32), ("attn_temp_scale", ctypes.c_float), ("attn_temp_len", ctypes.c_int32),
        ("yarn_factor", ctypes.c_float), ("yarn_orig_ctx", ctypes.c_int32), ("yarn_beta_fast", ctypes.c_float),
        ("yarn_beta_slow", ctypes.c_float), ("numerics", ctypes.c_int32)]


class OrcYarn(ctypes.Structure):
    _fields_ = [("factor", ctypes.c_float), ("orig_ctx", ctypes.c_int32), ("beta_fast", ctypes.c_float),
                ("beta_slow", ctypes.c_float)]


class OrcTensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("dtype", ctypes.c_int32), ("n_dims", ctypes.c_int32),
                ("ne", ctypes.c_int64 * 2), ("data", ctypes.c_void_p), ("nbytes", ctypes.c_size_t)]


def lib(variant: str = ""):
    """liboracle.so, or one of its builds that evaluate the same definition in
    another valid way, used only to measure a workload's sensitivity to the
    rounding of its sums: variant "desc" sums every dot product over the input
    index descending, "f64" accumulates every sum in double and rounds it once."""
    if variant not in _libs:
        path = _build.VARIANTS[variant][0]
        if not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f32.restype = f32
        L.orc_f32_to_f16.argtypes = [f32]
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_dequantize.argtypes = [i32, vp, i64, vp]
        L.orc_quantize_q8_0.argtypes = [vp, i64, vp]
        L.orc_rmsnorm.argtypes = [vp, vp, vp, i32, f32]
        L.orc_rmsnorm.restype = None
        L.orc_matvec.argtypes = [vp, vp, vp, i32, i32]
        L.orc_matvec.restype = None
        L.orc_matmul.argtypes = [vp, vp, vp, i32, i32, i32]
        L.orc_matmul.restype = None
        L.orc_rope_cos_sin.argtypes = [i32, i32, f32, vp, vp]
        L.orc_rope_cos_sin.restype = None
        L.orc_rope.argtypes = [vp, i32, i32, i32, i32, f32, i32]
        L.orc_rope.restype = None
        L.orc_rope_cos_sin_ff.argtypes = [i32, i32, f32, vp, vp, vp]
        L.orc_rope_cos_sin_ff.restype = None
        L.orc_rope_ff.argtypes = [vp, i32, i32, i32, i32, f32, i32, vp]
        L.orc_rope_ff.restype = None
        L.orc_rope_cos_sin_y.argtypes = [i32, i32, f32, vp, vp, vp, vp]
        L.orc_rope_cos_sin_y.restype = None
        L.orc_rope_y.argtypes = [vp, i32, i32, i32, i32, f32, i32, vp, vp]
        L.orc_rope_y.restype = None
        L.orc_yarn_ramp.argtypes = [vp, i32, i32, f32]
        L.orc_yarn_ramp.restype = ctypes.c_double
        L.orc_silu.argtypes = [f32]
        L.orc_silu.restype = f32
        L.orc_argmax.argtypes = [vp, i32]
        L.orc_argmax.restype = i32
        L.orc_attention.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, vp]
        L.orc_attention.restype = None
        L.orc_attention_ex.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, vp]
        L.orc_attention_ex.restype = None
        L.orc_attention_nx.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, i32, vp]
        L.orc_attention_nx.restype = None
        L.orc_round_input.argtypes = [vp, i64, i32]
        L.orc_round_input.restype = ctypes.c_int
        L.orc_attn_temp.argtypes = [i32, f32, i32]
        L.orc_attn_temp.restype = f32
        L.orc_attends.argtypes = [i32, i32, i32, i32]
        L.orc_attends.restype = ctypes.c_int
        L.orc_load.argtypes = [ctypes.POINTER(OrcConfig), ctypes.POINTER(OrcTensor), i32, ctypes.POINTER(vp)]
        L.orc_forward.argtypes = [vp, i32, i32, vp]
        L.orc_prefill.argtypes = [vp, vp, i32, vp]
        L.orc_prefill_rows.argtypes = [vp, vp, i32, vp, i32, vp]
        L.orc_prefill_rows.restype = ctypes.c_int
        L.orc_reset.argtypes = [vp]
        L.orc_reset.restype = None
        L.orc_kv_len.argtypes = [vp]
        L.orc_kv_read.argtypes = [vp, i32, i32, vp, vp]
        L.orc_free.argtypes = [vp]
        L.orc_free.restype = None
        L.orc_kv_write.argtypes = [vp, i32, i32, vp, vp]
        L.orc_set_len.argtypes = [vp, i32]
        L.orc_set_threads.argtypes = [i32]
        L.orc_set_threads.restype = None
        L.orc_max_threads.argtypes = []
        L.orc_max_threads.restype = i32
        L.orc_weights_per_layer.argtypes = [i64, i64, i64]
        L.orc_weights_per_layer.restype = i64
        _libs[variant] = L
    return _libs[variant]


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# ---------------------------------------------------------------- operations
def f16_to_f32(h: int) -> float:
    return float(np.float32(lib().orc_f16_to_f32(int(h))))


def f32_to_f16(x: float) -> int:
    return int(lib().orc_f32_to_f16(float(np.float32(x))))


def dequantize(dtype: int, raw: np.ndarray, n: int) -> np.ndarray:
    out = np.empty(n, np.float32)
    rc = lib().orc_dequantize(dtype, _p(np.ascontiguousarray(raw)), n, _p(out))
    if rc:
        raise ValueError(f"orc_dequantize: {rc}")
    return out


def quantize_q8_0(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.size // 32 * 34, np.uint8)
    rc = lib().orc_quantize_q8_0(_p(x), x.size, _p(out))
    if rc:
        raise ValueError(f"orc_quantize_q8_0: {rc}")
    return out


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    w = np.ascontiguousarray(w, np.float32)
    out = np.empty_like(x)
    lib().orc_rmsnorm(_p(out), _p(x), _p(w), x.size, eps)
    return out


def matvec(w: np.ndarray, x: np.ndarray, rows: int, cols: int) -> np.ndarray:
    w = np.ascontiguousarray(w, np.float32)
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(rows, np.float32)
    lib().orc_matvec(_p(out), _p(w), _p(x), rows, cols)
    return out


def matmul(w: np.ndarray, x: np.ndarray, n: int, rows: int, cols: int) -> np.ndarray:
    w = np.ascontiguousarray(w, np.float32)
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty((n, rows), np.float32)
    lib().orc_matmul(_p(out), _p(w), _p(x), n, rows, cols)
    return out


def _yarn(yarn):
    """yarn: None or (factor, orig_ctx, beta_fast, beta_slow)."""
    return None if yarn is None else OrcYarn(float(yarn[0]), int(yarn[1]), float(yarn[2]), float(yarn[3]))


def rope_cos_sin(pos: int, rope_dims: int, base: float, freq=None, yarn=None):
    """(cos, sin) of each pair's angle at pos; freq: optional per-pair divisors;
    yarn: optional (factor, orig_ctx, beta_fast, beta_slow)."""
    c = np.empty(rope_dims // 2, np.float32)
    s = np.empty(rope_dims // 2, np.float32)
    f = None if freq is None else np.ascontiguousarray(freq, np.float32)
    y = _yarn(yarn)
    if y is None:
        lib().orc_rope_cos_sin_ff(pos, rope_dims, base, None if f is None else _p(f), _p(c), _p(s))
    else:
        lib().orc_rope_cos_sin_y(pos, rope_dims, base, None if f is None else _p(f), ctypes.byref(y), _p(c), _p(s))
    return c, s


def rope(vec: np.ndarray, n_heads: int, head_dim: int, rope_dims: int, pos: int, base: float, neox: bool,
         freq=None, yarn=None) -> np.ndarray:
    v = np.array(vec, np.float32, copy=True)
    f = None if freq is None else np.ascontiguousarray(freq, np.float32)
    y = _yarn(yarn)
    if y is None:
        lib().orc_rope_ff(_p(v), n_heads, head_dim, rope_dims, pos, base, int(neox), None if f is None else _p(f))
    else:
        lib().orc_rope_y(_p(v), n_heads, head_dim, rope_dims, pos, base, int(neox), None if f is None else _p(f),
                         ctypes.byref(y))
    return v


def yarn_ramp(yarn, i: int, rope_dims: int, base: float) -> float:
    y = _yarn(yarn)
    return float(lib().orc_yarn_ramp(ctypes.byref(y), i, rope_dims, base))


def silu(z: float) -> float:
    return float(np.float32(lib().orc_silu(float(np.float32(z)))))


def argmax(v: np.ndarray) -> int:
    v = np.ascontiguousarray(v, np.float32)
    return int(lib().orc_argmax(_p(v), v.size))


def attention(q: np.ndarray, kcache: np.ndarray, vcache: np.ndarray, n_heads: int, n_kv_heads: int, head_dim: int,
              pos: int, want_weights: bool = False, window: int = 0, sinks: int = 0, temp_scale: float = 0.0,
              temp_len: int = 0, round16: bool = False):
    """kcache/vcache: binary16 bits, [>= pos+1][n_kv_heads * head_dim]. window /
    sinks: the attended rows (0: all rows up to pos); temp_scale / temp_len:
    the attention temperature (0: none)."""
    q = np.ascontiguousarray(q, np.float32)
    kc = np.ascontiguousarray(kcache, np.uint16)
    vc = np.ascontiguousarray(vcache, np.uint16)
    out = np.empty(n_heads * head_dim, np.float32)
    wts = np.empty((n_heads, pos + 1), np.float32) if want_weights else None
    if round16:
        lib().orc_attention_nx(_p(out), _p(q), _p(kc), _p(vc), n_heads, n_kv_heads, head_dim, pos, window, sinks,
                               temp_scale, temp_len, 1, _p(wts) if wts is not None else None)
    elif window == 0 and sinks == 0 and temp_scale == 0.0:
        lib().orc_attention(_p(out), _p(q), _p(kc), _p(vc), n_heads, n_kv_heads, head_dim, pos,
                            _p(wts) if wts is not None else None)
    else:
        lib().orc_attention_ex(_p(out), _p(q), _p(kc), _p(vc), n_heads, n_kv_heads, head_dim, pos, window, sinks,
                               temp_scale, temp_len, _p(wts) if wts is not None else None)
    return (out, wts) if want_weights else out


def round_input(x: np.ndarray, dtype: int) -> np.ndarray:
    """A product's input as llama.cpp rounds it for weights of type dtype."""
    v = np.array(x, np.float32, copy=True)
    rc = lib().orc_round_input(_p(v), v.size, dtype)
    if rc:
        raise ValueError(f"orc_round_input: {rc}")
    return v


def attn_temp(pos: int, temp_scale: float, temp_len: int) -> float:
    return float(lib().orc_attn_temp(pos, temp_scale, temp_len))


def attends(t: int, pos: int, window: int, sinks: int) -> bool:
    return bool(lib().orc_attends(t, pos, window, sinks))


def set_threads(n: int):
    """Threads of the oracle's OpenMP loops (its results do not depend on it)."""
    lib().orc_set_threads(int(n))


def max_threads() -> int:
    return int(lib().orc_max_threads())


def weights_per_layer(dim: int, kv_dim: int, ffn: int) -> int:
    return int(lib().orc_weights_per_layer(dim, kv_dim, ffn))


# --------------------------------------------------------------------- model
def make_config(cfg) -> OrcConfig:
    c = OrcConfig()
    for f in ("dim", "n_layers", "n_heads", "n_kv_heads", "head_dim", "ffn", "vocab", "n_ctx"):
        setattr(c, f, int(getattr(cfg, f)))
    c.rope_dims = int(cfg.n_rot)
    c.rope_neox = int(bool(cfg.rope_neox))
    c.eps = float(cfg.eps)
    c.rope_base = float(cfg.rope_base)
    c.attn_window = int(getattr(cfg, "attn_window", 0))
    c.attn_sinks = int(getattr(cfg, "attn_sinks", 0))
    c.attn_temp_scale = float(getattr(cfg, "attn_temp_scale", 0.0))
    c.attn_temp_len = int(getattr(cfg, "attn_temp_len", 0))
    c.yarn_factor = float(getattr(cfg, "yarn_factor", 0.0))
    c.yarn_orig_ctx = int(getattr(cfg, "yarn_orig_ctx", 0))
    c.yarn_beta_fast = float(getattr(cfg, "yarn_beta_fast", 32.0))
    c.yarn_beta_slow = float(getattr(cfg, "yarn_beta_slow", 1.0))
    c.numerics = int(getattr(cfg, "numerics", 0))
    return c


class Model:
    """The oracle's forward pass over a tensor set (a list of synth.Tensor)."""

    def __init__(self, cfg, tensors: Sequence, config: Optional[OrcConfig] = None, variant: str = ""):
        self.cfg = cfg
        self.L = lib(variant)
        self._keep = list(tensors)
        arr = (OrcTensor * len(tensors))()
        self._names = []
        for i, t in enumerate(tensors):
            nm = t.name.encode()
            self._names.append(nm)
            arr[i].name = nm
            arr[i].dtype = t.dtype
            arr[i].n_dims = len(t.ne)
            arr[i].ne[0] = t.ne[0]
            arr[i].ne[1] = t.ne[1] if len(t.ne) > 1 else 1
            arr[i].data = t.data.ctypes.data
            arr[i].nbytes = t.nbytes
        self.config = config if config is not None else make_config(cfg)
        h = ctypes.c_void_p()
        rc = self.L.orc_load(ctypes.byref(self.config), arr, len(tensors), ctypes.byref(h))
        if rc:
            raise ValueError(f"orc_load failed: {rc}")
        self.h = h
        self.vocab = self.config.vocab

    def close(self):
        if getattr(self, "h", None):
            self.L.orc_free(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def forward(self, token: int, pos: int) -> np.ndarray:
        out = np.empty(self.vocab, np.float32)
        rc = self.L.orc_forward(self.h, int(token), int(pos), _p(out))
        if rc:
            raise ValueError(f"orc_forward: {rc}")
        return out

    def prefill(self, tokens) -> np.ndarray:
        tk = np.ascontiguousarray(tokens, np.int32)
        out = np.empty(self.vocab, np.float32)
        rc = self.L.orc_prefill(self.h, _p(tk), tk.size, _p(out))
        if rc:
            raise ValueError(f"orc_prefill: {rc}")
        return out

    def prefill_rows(self, tokens, rows) -> np.ndarray:
        """Prefill, returning the logits of the batch rows `rows` ([len(rows), vocab])."""
        tk = np.ascontiguousarray(tokens, np.int32)
        rw = np.ascontiguousarray(rows, np.int32)
        out = np.empty((rw.size, self.vocab), np.float32)
        rc = self.L.orc_prefill_rows(self.h, _p(tk), tk.size, _p(rw), rw.size, _p(out))
        if rc:
            raise ValueError(f"orc_prefill_rows: {rc}")
        return out

    def reset(self):
        self.L.orc_reset(self.h)

    def kv_len(self) -> int:
        return int(self.L.orc_kv_len(self.h))

    def kv_write(self, layer: int, pos: int, k_bits: np.ndarray, v_bits: np.ndarray):
        """Write binary16 K and V bits of one layer at one position."""
        k = np.ascontiguousarray(k_bits, np.uint16)
        v = np.ascontiguousarray(v_bits, np.uint16)
        kvd = self.config.n_kv_heads * self.config.head_dim
        assert k.size == kvd and v.size == kvd
        rc = self.L.orc_kv_write(self.h, int(layer), int(pos), _p(k), _p(v))
        if rc:
            raise ValueError(f"orc_kv_write: {rc}")

    def set_len(self, n: int):
        """Declare cache rows 0..n-1 valid."""
        rc = self.L.orc_set_len(self.h, int(n))
        if rc:
            raise ValueError(f"orc_set_len: {rc}")

    def kv_read(self, layer: int, pos: int):
        kvd = self.config.n_kv_heads * self.config.head_dim
        k = np.empty(kvd, np.uint16)
        v = np.empty(kvd, np.uint16)
        rc = self.L.orc_kv_read(self.h, layer, pos, _p(k), _p(v))
        if rc:
            raise ValueError(f"orc_kv_read: {rc}")
        return k, v
