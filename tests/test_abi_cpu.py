"""The C-ABI library without a GPU: it loads, exports every symbol include/*.h
declares, and rejects malformed configs and tensor sets before any device work
(llm_plan is host-only; llm_load_weights validates before it allocates)."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
from conftest import ROOT
from helpers import SMALL, SMALL_Q8, SMALL_Q8_RND, drop, f32_tensor

llm = pytest.importorskip("llama_family_decode_amd")


def declared_functions():
    names = []
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"\b(llm_[a-z0-9_]+)\s*\(", src)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    L = llm.lib()
    decl = declared_functions()
    assert len(decl) >= 11
    for name in decl:
        assert hasattr(L, name), name
    assert set(llm.EXPORTS) <= set(decl)


def test_library_is_gfx950_code():
    blob = open(llm.LIB_PATH, "rb").read()
    assert b"gfx950" in blob


def plan(cfg, ts):
    c = llm.make_config(cfg)
    arr, keep = llm.make_tensors(ts)
    return llm.llm_plan(c, arr, len(ts))


def plan_rc(cfg, ts, config=None):
    c = config if config is not None else llm.make_config(cfg)
    arr, keep = llm.make_tensors(ts)
    w, k, s = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    return llm.lib().llm_plan(ctypes.byref(c), arr, len(ts), ctypes.byref(w), ctypes.byref(k), ctypes.byref(s))


def tiled_bytes(cfg, q8):
    """The prefill products' tiled binary16 copies of the layer matrices (rows
    padded to 256), plus, for Q8_0, their block scales."""
    pad = lambda r: (r + 255) // 256 * 256
    mats = [(cfg.q_dim + 2 * cfg.kv_dim, cfg.dim), (cfg.dim, cfg.q_dim), (2 * cfg.ffn, cfg.dim), (cfg.dim, cfg.ffn)]
    per = sum(pad(r) * c * 2 + (pad(r) * (c // 32) * 2 if q8 else 0) for r, c in mats)
    return cfg.n_layers * per


def test_plan_sizes():
    ts = synth.make_tensor_set(SMALL)
    w, k, s = plan(SMALL, ts)
    kvd = SMALL.kv_dim
    assert k >= 2 * SMALL.n_layers * SMALL.n_ctx * kvd * 2
    raw = sum(t.nbytes for t in ts)
    assert raw <= w <= raw + 64 * 1024  # packing adds only alignment
    # Q8_0 packing keeps every byte (34 per 32 values) and adds the tiled copies
    ts8 = synth.make_tensor_set(SMALL_Q8)
    w8, _, _ = plan(SMALL_Q8, ts8)
    raw8 = sum(t.nbytes for t in ts8) + tiled_bytes(SMALL_Q8, True)
    assert raw8 <= w8 <= raw8 + 64 * 1024


def test_plan_q8_llamacpp_sizes():
    # under llama.cpp's rounding points a Q8_0 layer matrix gets the tiled int8
    # codes and fp32 block scales of the integer prefill products instead of
    # the binary16 copy, and the scratch arena holds one batch's input codes
    # (int8) and scales (fp32) for the widest product input
    cfg, cfg0 = SMALL_Q8_RND, SMALL_Q8
    ts = synth.make_tensor_set(cfg)
    w, _, s = plan(cfg, ts)
    pad = lambda r: (r + 255) // 256 * 256
    mats = [(cfg.q_dim + 2 * cfg.kv_dim, cfg.dim), (cfg.dim, cfg.q_dim), (2 * cfg.ffn, cfg.dim), (cfg.dim, cfg.ffn)]
    tiled = cfg.n_layers * sum(pad(r) * c + pad(r) * (c // 32) * 4 for r, c in mats)
    raw = sum(t.nbytes for t in ts) + tiled
    assert raw <= w <= raw + 64 * 1024
    _, _, s0 = plan(cfg0, synth.make_tensor_set(cfg0))
    C, kmax = llm.llm_op_prefill_chunk(), max(cfg.dim, cfg.q_dim, cfg.ffn)
    a256 = lambda b: (b + 255) // 256 * 256
    assert s - s0 == a256(C * kmax) + a256(C * (kmax // 32) * 4)


def test_plan_1b_q8_sizes():
    # the 1B-shape Q8_0 set without generating it: byte counts only
    cfg = synth.C4
    specs = synth.tensor_specs(cfg)
    ts = []
    for name, dt, ne, kind in specs:
        n = int(np.prod(ne))
        ts.append(synth.Tensor(name, dt, ne, np.zeros(1, np.uint8)))
        ts[-1].data = np.lib.stride_tricks.as_strided(np.zeros(1, np.uint8), (synth.nbytes_of(dt, n),), (0,))
    c = llm.make_config(cfg)
    arr = (llm.llm_tensor * len(ts))()
    for i, t in enumerate(ts):
        arr[i].name = t.name.encode()
        arr[i].dtype = t.dtype
        arr[i].n_dims = len(t.ne)
        arr[i].ne[0] = t.ne[0]
        arr[i].ne[1] = t.ne[1] if len(t.ne) > 1 else 1
        arr[i].data = 1
        arr[i].nbytes = synth.nbytes_of(t.dtype, int(np.prod(t.ne)))
    w, k, s = llm.llm_plan(c, arr, len(ts))
    layer_q8 = 16 * (2048 * 3072 + 2048 * 2048 + 2 * 8192 * 2048 + 8192 * 2048) * 34 // 32
    embd = 128256 * 2048 * 4
    want = layer_q8 + embd + tiled_bytes(cfg, True)
    assert want <= w <= want + (1 << 20)
    assert k == 2 * 16 * 8 * 8320 * 64 * 2


@pytest.mark.parametrize("case", ["missing", "shape", "dtype_norm", "size", "bias_partial", "mixed_qkv", "freqs_shape"])
def test_plan_rejects_bad_tensor_sets(case):
    ts = synth.make_tensor_set(SMALL)
    want = {"missing": -4, "shape": -2, "dtype_norm": -3, "size": -5, "bias_partial": -4, "mixed_qkv": -3,
            "freqs_shape": -2}[case]
    if case == "missing":
        ts = drop(ts, "blk.1.ffn_down.weight")
    elif case == "shape":
        ts = [f32_tensor(t.name, np.zeros(SMALL.dim * 3, np.float32), (3, SMALL.dim)) if t.name == "blk.0.attn_k.weight"
              else t for t in ts]
    elif case == "dtype_norm":
        ts = [synth.Tensor(t.name, synth.F16, t.ne, np.zeros(t.n * 2, np.uint8)) if t.name == "output_norm.weight"
              else t for t in ts]
    elif case == "size":
        ts = [synth.Tensor(t.name, t.dtype, t.ne, t.data[:-4]) if t.name == "blk.0.ffn_up.weight" else t for t in ts]
    elif case == "bias_partial":
        ts = ts + [f32_tensor("blk.0.attn_q.bias", np.zeros(SMALL.q_dim, np.float32), (SMALL.q_dim,))]
    elif case == "freqs_shape":  # one divisor per pair: n_rot / 2 values
        ts = ts + [f32_tensor("rope_freqs.weight", np.ones(SMALL.n_rot, np.float32), (SMALL.n_rot,))]
    elif case == "mixed_qkv":
        ts = [synth.gen_tensor(9, t.name, synth.F16, t.ne, "matrix", SMALL) if t.name == "blk.0.attn_v.weight" else t
              for t in ts]
    assert plan_rc(SMALL, ts) == want
    assert llm.llm_last_error()


@pytest.mark.parametrize("field,value,want", [
    ("head_dim", 30, -1),     # n_heads * head_dim must match the tensors; 30 is also not a multiple of 8
    ("rope_dims", 33, -1),    # odd
    ("n_kv_heads", 3, -1),    # 4 % 3 != 0
    ("vocab", 0, -1),
    ("n_ctx", 0, -1),
    ("attn_window", -1, -1),
    ("attn_sinks", 2, -1),          # sinks need a window
    ("attn_temp_scale", -0.1, -1),
    ("attn_temp_scale", float("nan"), -1),
    ("yarn_factor", 0.5, -1),        # YaRN factors start at 1
    ("yarn_factor", 4.0, -1),        # ... and need the original context
    ("numerics", 2, -1),
])
def test_plan_rejects_bad_configs(field, value, want):
    ts = synth.make_tensor_set(SMALL)
    c = llm.make_config(SMALL)
    setattr(c, field, value)
    assert plan_rc(SMALL, ts, c) == want


def test_plan_accepts_spans_and_rejects_a_temperature_without_length():
    ts = synth.make_tensor_set(SMALL)
    assert plan_rc(SMALL.with_(attn_window=8, attn_sinks=4, attn_temp_scale=0.1), ts) == 0
    assert plan_rc(SMALL.with_(attn_temp_scale=0.1, attn_temp_len=0), ts) == -1


def test_limits_are_reported():
    cfg = SMALL.with_(n_heads=8, n_kv_heads=8, head_dim=16)  # head_dim 16 ok; group 1 ok -> loads
    ts = synth.make_tensor_set(cfg)
    assert plan_rc(cfg, ts) == 0
    cfg = SMALL.with_(dim=100)  # not a multiple of 32
    c = llm.make_config(cfg)
    assert plan_rc(cfg, synth.make_tensor_set(SMALL), c) == -12


def test_load_validates_before_device_work():
    ts = drop(synth.make_tensor_set(SMALL), "output_norm.weight")
    c = llm.make_config(SMALL)
    arr, keep = llm.make_tensors(ts)
    h = ctypes.c_void_p(123)
    rc = llm.lib().llm_load_weights(ctypes.byref(c), arr, len(ts), None, None, None, None, ctypes.byref(h))
    assert rc == -4 and not h.value
    assert "output_norm" in llm.llm_last_error()


@pytest.mark.parametrize("bad", [0.0, -1.0, float("inf"), float("nan")])
def test_load_rejects_bad_rope_divisors(bad):
    cfg = SMALL.with_(rope_freq_factors=True)
    ts = synth.make_tensor_set(cfg)
    f = np.ones(cfg.n_rot // 2, np.float32)
    f[3] = bad
    ts = [f32_tensor(t.name, f, t.ne) if t.name == "rope_freqs.weight" else t for t in ts]
    assert plan_rc(cfg, ts) == 0  # llm_plan checks shapes only
    c = llm.make_config(cfg)
    arr, keep = llm.make_tensors(ts)
    h = ctypes.c_void_p(123)
    rc = llm.lib().llm_load_weights(ctypes.byref(c), arr, len(ts), None, None, None, None, ctypes.byref(h))
    assert rc == -1 and not h.value
    assert "rope_freqs" in llm.llm_last_error()


def test_null_context_calls():
    L = llm.lib()
    assert L.llm_kv_len(None) == -1
    assert L.llm_reset(None) == -1
    assert L.llm_decode(None, 0, 0, None, None) == -1
    ms = ctypes.c_float()
    assert L.llm_op_time_prefill_product(None, 0, 0, 128, 1, ctypes.byref(ms)) == -1
    assert L.llm_op_prefill_int8(None) == -1
    L.llm_free(None)


def test_prefill_batches_hold_whole_activation_tiles():
    # the batch buffers hold the products' binary16 input planes in 128-row tiles
    c = llm.llm_op_prefill_chunk()
    assert c >= 128 and c % 128 == 0
