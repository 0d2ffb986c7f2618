"""Python binding of libllm, the gfx950 Llama-family forward pass.

Argument marshalling only: every step of the forward pass runs in the HIP
kernels of ``libllm.so``. PyTorch supplies device memory (the three arenas the
library packs weights, KV cache and scratch into) and the stream. Importing
this package loads the built library and raises if it is missing; build it with
``python -m llama_family_decode_amd.build`` (or ``__graft_entry__.build()``).

The functions below carry the C ABI's names (include/llm.h); ``Model`` wraps
them for convenience.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch  # first, so libllm binds to the HIP runtime torch has loaded

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libllm.so")

F32, F16, Q8_0 = 0, 1, 8
ERRORS = {
    0: "OK", -1: "LLM_ERR_ARG", -2: "LLM_ERR_SHAPE", -3: "LLM_ERR_DTYPE", -4: "LLM_ERR_MISSING", -5: "LLM_ERR_SIZE",
    -6: "LLM_ERR_TOKEN", -7: "LLM_ERR_POS", -8: "LLM_ERR_CTX_FULL", -9: "LLM_ERR_NONFINITE", -10: "LLM_ERR_DEVICE",
    -11: "LLM_ERR_OOM", -12: "LLM_ERR_LIMIT",
}
EXPORTS = ["llm_plan", "llm_load_weights", "llm_decode", "llm_prefill", "llm_prefill_rows", "llm_generate", "llm_reset", "llm_free",
           "llm_last_error", "llm_logits", "llm_kv_len", "llm_kv_read", "llm_op_qkv", "llm_op_attention", "llm_op_o",
           "llm_op_ffn_up", "llm_op_down", "llm_op_logits", "llm_op_kv_write", "llm_op_time", "llm_rewind", "llm_op_step_trace",
           "llm_op_step_kind", "llm_op_prefill_chunk", "llm_op_prefill_int8", "llm_op_attention_noalloc",
           "llm_op_time_prefill_product"]
STAGE_QKV, STAGE_ATTN, STAGE_O, STAGE_FFN_UP, STAGE_DOWN, STAGE_LOGITS, STAGE_STEP = range(7)
PRODUCT_QKV, PRODUCT_O, PRODUCT_GATE_UP, PRODUCT_DOWN = range(4)


class LlmError(RuntimeError):
    def __init__(self, code: int, message: str = ""):
        self.code = code
        super().__init__(f"{ERRORS.get(code, code)}: {message}")


class llm_tensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("dtype", ctypes.c_int32), ("n_dims", ctypes.c_int32),
                ("ne", ctypes.c_int64 * 2), ("data", ctypes.c_void_p), ("nbytes", ctypes.c_size_t)]


class llm_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("dim", "n_layers", "n_heads", "n_kv_heads", "head_dim", "ffn", "vocab",
                                               "n_ctx", "rope_dims", "rope_neox")] + [
        ("eps", ctypes.c_float), ("rope_base", ctypes.c_float), ("attn_window", ctypes.c_int32),
        ("attn_sinks", ctypes.c_int32), ("attn_temp_scale", ctypes.c_float), ("attn_temp_len", ctypes.c_int32),
        ("yarn_factor", ctypes.c_float), ("yarn_orig_ctx", ctypes.c_int32), ("yarn_beta_fast", ctypes.c_float),
        ("yarn_beta_slow", ctypes.c_float), ("numerics", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded libllm.so. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run python -m llama_family_decode_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        P = ctypes.POINTER
        L.llm_plan.argtypes = [P(llm_config), P(llm_tensor), i32, P(sz), P(sz), P(sz)]
        L.llm_plan.restype = ctypes.c_int
        L.llm_load_weights.argtypes = [P(llm_config), P(llm_tensor), i32, vp, vp, vp, vp, P(vp)]
        L.llm_load_weights.restype = ctypes.c_int
        L.llm_decode.argtypes = [vp, i32, i32, vp, P(i32)]
        L.llm_decode.restype = ctypes.c_int
        L.llm_prefill.argtypes = [vp, vp, i32, vp, P(i32)]
        L.llm_prefill.restype = ctypes.c_int
        L.llm_prefill_rows.argtypes = [vp, vp, i32, vp, i32, vp]
        L.llm_prefill_rows.restype = ctypes.c_int
        L.llm_generate.argtypes = [vp, i32, i32, vp]
        L.llm_generate.restype = ctypes.c_int
        L.llm_reset.argtypes = [vp]
        L.llm_reset.restype = ctypes.c_int
        L.llm_free.argtypes = [vp]
        L.llm_free.restype = None
        L.llm_last_error.argtypes = [vp]
        L.llm_last_error.restype = ctypes.c_char_p
        L.llm_logits.argtypes = [vp]
        L.llm_logits.restype = vp
        L.llm_kv_len.argtypes = [vp]
        L.llm_kv_len.restype = i32
        L.llm_kv_read.argtypes = [vp, i32, i32, vp, vp]
        L.llm_kv_read.restype = ctypes.c_int
        L.llm_op_qkv.argtypes = [vp, i32, i32, vp, vp]
        L.llm_op_attention.argtypes = [vp, i32, i32, vp, vp]
        L.llm_op_attention_noalloc.argtypes = [vp, i32, i32, vp, vp]
        L.llm_op_o.argtypes = [vp, i32, vp, vp]
        L.llm_op_ffn_up.argtypes = [vp, i32, vp, vp]
        L.llm_op_down.argtypes = [vp, i32, vp, vp]
        L.llm_op_logits.argtypes = [vp, vp, vp, P(i32)]
        L.llm_op_kv_write.argtypes = [vp, i32, i32, i32, vp, vp]
        L.llm_op_time.argtypes = [vp, i32, i32, i32, i32, P(ctypes.c_float)]
        L.llm_op_time_prefill_product.argtypes = [vp, i32, i32, i32, i32, P(ctypes.c_float)]
        L.llm_rewind.argtypes = [vp, i32]
        L.llm_op_step_trace.argtypes = [vp, vp, i32]
        L.llm_op_step_trace.restype = ctypes.c_int
        L.llm_op_step_kind.argtypes = [vp]
        L.llm_op_step_kind.restype = ctypes.c_int
        L.llm_op_prefill_chunk.argtypes = []
        L.llm_op_prefill_chunk.restype = ctypes.c_int
        L.llm_op_prefill_int8.argtypes = [vp]
        L.llm_op_prefill_int8.restype = ctypes.c_int
        for f in ("llm_op_qkv", "llm_op_attention", "llm_op_attention_noalloc", "llm_op_o", "llm_op_ffn_up", "llm_op_down", "llm_op_logits",
                  "llm_op_kv_write", "llm_op_time", "llm_op_time_prefill_product", "llm_rewind"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def make_config(cfg) -> llm_config:
    """llm_config from any object with the config fields (e.g. synth.ModelConfig)."""
    c = llm_config()
    for f in ("dim", "n_layers", "n_heads", "n_kv_heads", "head_dim", "ffn", "vocab", "n_ctx"):
        setattr(c, f, int(getattr(cfg, f)))
    rd = getattr(cfg, "rope_dims", 0) or cfg.head_dim
    c.rope_dims = int(rd)
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


def make_tensors(tensors: Sequence):
    """ctypes array of llm_tensor from objects with name/dtype/ne/data (numpy uint8) fields."""
    arr = (llm_tensor * len(tensors))()
    keep = []
    for i, t in enumerate(tensors):
        nm = t.name.encode()
        keep.append(nm)
        data = np.ascontiguousarray(t.data)
        keep.append(data)
        arr[i].name = nm
        arr[i].dtype = int(t.dtype)
        arr[i].n_dims = len(t.ne)
        arr[i].ne[0] = int(t.ne[0])
        arr[i].ne[1] = int(t.ne[1]) if len(t.ne) > 1 else 1
        arr[i].data = data.ctypes.data
        arr[i].nbytes = int(data.nbytes)
    return arr, keep


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) or None


def llm_last_error(ctx=None) -> str:
    return (lib().llm_last_error(ctx) or b"").decode()


def _check(rc: int, ctx=None):
    if rc != 0:
        raise LlmError(rc, llm_last_error(ctx))


def llm_plan(cfg: llm_config, tarr, n: int):
    w, k, s = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().llm_plan(ctypes.byref(cfg), tarr, n, ctypes.byref(w), ctypes.byref(k), ctypes.byref(s)))
    return int(w.value), int(k.value), int(s.value)


def llm_load_weights(cfg: llm_config, tarr, n: int, d_weights: int, d_kv: int, d_scratch: int, stream: Optional[int]):
    h = ctypes.c_void_p()
    _check(lib().llm_load_weights(ctypes.byref(cfg), tarr, n, d_weights, d_kv, d_scratch, stream, ctypes.byref(h)))
    return h


def llm_decode(ctx, token: int, pos: int, d_logits: Optional[int] = None, want_next: bool = True):
    nxt = ctypes.c_int32(-1)
    rc = lib().llm_decode(ctx, int(token), int(pos), d_logits, ctypes.byref(nxt) if want_next else None)
    _check(rc, ctx)
    return int(nxt.value) if want_next else None


def llm_prefill(ctx, tokens, d_logits: Optional[int] = None, want_next: bool = True):
    tk = np.ascontiguousarray(tokens, np.int32)
    nxt = ctypes.c_int32(-1)
    rc = lib().llm_prefill(ctx, tk.ctypes.data, tk.size, d_logits, ctypes.byref(nxt) if want_next else None)
    _check(rc, ctx)
    return int(nxt.value) if want_next else None


def llm_prefill_rows(ctx, tokens, rows, d_logits: int):
    """Prefill `tokens`; the logits of prompt rows `rows` (None: every row) go
    to the device buffer d_logits, [len(rows)][vocab] fp32. Enqueue only."""
    tk = np.ascontiguousarray(tokens, np.int32)
    if rows is None:
        rc = lib().llm_prefill_rows(ctx, tk.ctypes.data, tk.size, None, tk.size, d_logits)
    else:
        rw = np.ascontiguousarray(rows, np.int32)
        rc = lib().llm_prefill_rows(ctx, tk.ctypes.data, tk.size, rw.ctypes.data if rw.size else None, rw.size,
                                    d_logits)
    _check(rc, ctx)


def llm_generate(ctx, token: int, n_steps: int) -> np.ndarray:
    out = np.empty(n_steps, np.int32)
    _check(lib().llm_generate(ctx, int(token), int(n_steps), out.ctypes.data), ctx)
    return out


def llm_reset(ctx):
    _check(lib().llm_reset(ctx), ctx)


def llm_free(ctx):
    lib().llm_free(ctx)


def llm_logits(ctx) -> int:
    return int(lib().llm_logits(ctx) or 0)


def llm_kv_len(ctx) -> int:
    return int(lib().llm_kv_len(ctx))


def llm_kv_read(ctx, layer: int, pos: int, kv_dim: int):
    k = np.empty(kv_dim, np.uint16)
    v = np.empty(kv_dim, np.uint16)
    _check(lib().llm_kv_read(ctx, int(layer), int(pos), k.ctypes.data, v.ctypes.data), ctx)
    return k, v


def llm_op_qkv(ctx, layer: int, pos: int, d_x: int, d_q: int):
    _check(lib().llm_op_qkv(ctx, layer, pos, d_x, d_q), ctx)


def llm_op_attention(ctx, layer: int, pos: int, d_q: int, d_out: int):
    _check(lib().llm_op_attention(ctx, layer, pos, d_q, d_out), ctx)


def llm_op_attention_noalloc(ctx, layer: int, pos: int, d_q: int, d_out: int):
    _check(lib().llm_op_attention_noalloc(ctx, layer, pos, d_q, d_out), ctx)


def llm_op_o(ctx, layer: int, d_in: int, d_x: int):
    _check(lib().llm_op_o(ctx, layer, d_in, d_x), ctx)


def llm_op_ffn_up(ctx, layer: int, d_x: int, d_u: int):
    _check(lib().llm_op_ffn_up(ctx, layer, d_x, d_u), ctx)


def llm_op_down(ctx, layer: int, d_u: int, d_x: int):
    _check(lib().llm_op_down(ctx, layer, d_u, d_x), ctx)


def llm_op_logits(ctx, d_x: int, d_logits: Optional[int] = None) -> int:
    nxt = ctypes.c_int32(-1)
    _check(lib().llm_op_logits(ctx, d_x, d_logits, ctypes.byref(nxt)), ctx)
    return int(nxt.value)


def llm_op_kv_write(ctx, layer: int, pos0: int, k_bits: np.ndarray, v_bits: np.ndarray, kv_dim: int):
    k = np.ascontiguousarray(k_bits, np.uint16).reshape(-1, kv_dim)
    v = np.ascontiguousarray(v_bits, np.uint16).reshape(-1, kv_dim)
    assert k.shape == v.shape
    _check(lib().llm_op_kv_write(ctx, layer, pos0, k.shape[0], k.ctypes.data, v.ctypes.data), ctx)


def llm_op_time(ctx, stage: int, layer: int = 0, pos: int = 0, n_launch: int = 20) -> float:
    ms = ctypes.c_float()
    _check(lib().llm_op_time(ctx, stage, layer, pos, n_launch, ctypes.byref(ms)), ctx)
    return float(ms.value)


def llm_op_step_kind(ctx) -> int:
    """0: launch graph; 1: persistent step kernel; 2: persistent step kernel compiled for this shape."""
    r = lib().llm_op_step_kind(ctx)
    if r < 0:
        raise LlmError(r, "llm_op_step_kind")
    return r


def llm_op_prefill_chunk() -> int:
    """Rows per prefill batch."""
    return int(lib().llm_op_prefill_chunk())


def llm_op_time_prefill_product(ctx, product: int, layer: int = 0, n_rows: int = 512, n_launch: int = 20) -> float:
    ms = ctypes.c_float()
    _check(lib().llm_op_time_prefill_product(ctx, product, layer, n_rows, n_launch, ctypes.byref(ms)), ctx)
    return float(ms.value)


def llm_op_prefill_int8(ctx) -> int:
    """1 when the context's prefill runs its Q8_0 products as integer matrix-core products."""
    r = lib().llm_op_prefill_int8(ctx)
    if r < 0:
        raise LlmError(r, "llm_op_prefill_int8")
    return r


def llm_op_step_trace(ctx, n_layers: int) -> np.ndarray:
    out = np.zeros(5 * n_layers + 2, np.uint64)
    _check(lib().llm_op_step_trace(ctx, out.ctypes.data, out.size), ctx)
    return out


def llm_rewind(ctx, length: int):
    _check(lib().llm_rewind(ctx, int(length)), ctx)


_hip_rt = None


def _hip():
    """The HIP runtime torch has loaded (for copies out of library-owned buffers)."""
    global _hip_rt
    if _hip_rt is None:
        _hip_rt = ctypes.CDLL("libamdhip64.so")
        _hip_rt.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        _hip_rt.hipMemcpy.restype = ctypes.c_int
    return _hip_rt


class Model:
    """A loaded model on one GPU. `tensors` are objects with name/dtype/ne/data."""

    def __init__(self, cfg, tensors: Sequence, device: str = "cuda:0", stream=None):
        lib()
        self.device = torch.device(device)
        torch.cuda.set_device(self.device)
        self.cfg = cfg
        self.config = make_config(cfg)
        tarr, keep = make_tensors(tensors)
        n = len(tensors)
        wb, kb, sb = llm_plan(self.config, tarr, n)
        self.sizes = (wb, kb, sb)
        # arenas: torch owns the memory, the library packs into it
        self._w = torch.empty(max(wb, 256), dtype=torch.uint8, device=self.device)
        self._kv = torch.empty(max(kb, 256), dtype=torch.uint8, device=self.device)
        self._s = torch.empty(max(sb, 256), dtype=torch.uint8, device=self.device)
        self.stream = stream
        self.ctx = llm_load_weights(self.config, tarr, n, self._w.data_ptr(), self._kv.data_ptr(), self._s.data_ptr(),
                                    _stream_handle(stream))
        del keep
        self.vocab = int(self.config.vocab)
        self.kv_dim = int(self.config.n_kv_heads * self.config.head_dim)
        self.logits_buf = torch.empty(self.vocab, dtype=torch.float32, device=self.device)

    def close(self):
        if getattr(self, "ctx", None):
            llm_free(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def decode(self, token: int, pos: int, want_next: bool = True, copy_logits: bool = True):
        return llm_decode(self.ctx, token, pos, self.logits_buf.data_ptr() if copy_logits else None, want_next)

    def prefill(self, tokens, want_next: bool = True, copy_logits: bool = True):
        return llm_prefill(self.ctx, tokens, self.logits_buf.data_ptr() if copy_logits else None, want_next)

    def prefill_rows(self, tokens, rows=None) -> np.ndarray:
        """Prefill and return the logits of the chosen prompt rows (all rows
        if None) as a [len(rows), vocab] array."""
        n_out = len(tokens) if rows is None else len(rows)
        out = torch.empty((max(n_out, 1), self.vocab), dtype=torch.float32, device=self.device)
        llm_prefill_rows(self.ctx, tokens, rows, out.data_ptr())
        torch.cuda.synchronize(self.device)
        return out[:n_out].cpu().numpy()

    def generate(self, token: int, n_steps: int) -> np.ndarray:
        return llm_generate(self.ctx, token, n_steps)

    def logits(self) -> np.ndarray:
        """The copy of the logits the last decode/prefill call made (d_logits)."""
        torch.cuda.synchronize(self.device)
        return self.logits_buf.cpu().numpy()

    def ctx_logits(self) -> np.ndarray:
        """The context's own logits buffer (llm_logits): the last decode,
        prefill or generate step's logits."""
        torch.cuda.synchronize(self.device)
        out = np.empty(self.vocab, np.float32)
        rc = _hip().hipMemcpy(ctypes.c_void_p(out.ctypes.data), ctypes.c_void_p(llm_logits(self.ctx)),
                              ctypes.c_size_t(out.nbytes), 2)  # hipMemcpyDeviceToHost
        if rc != 0:
            raise RuntimeError(f"hipMemcpy failed: {rc}")
        return out

    def reset(self):
        llm_reset(self.ctx)

    def kv_len(self) -> int:
        return llm_kv_len(self.ctx)

    def kv_read(self, layer: int, pos: int):
        return llm_kv_read(self.ctx, layer, pos, self.kv_dim)

    def rewind(self, length: int):
        llm_rewind(self.ctx, length)

    def kv_write(self, layer: int, pos0: int, k_bits: np.ndarray, v_bits: np.ndarray):
        llm_op_kv_write(self.ctx, layer, pos0, k_bits, v_bits, self.kv_dim)

    def time_stage(self, stage: int, layer: int = 0, pos: int = 0, n_launch: int = 20) -> float:
        return llm_op_time(self.ctx, stage, layer, pos, n_launch)

    def time_product(self, product: int, n_rows: int, layer: int = 0, n_launch: int = 20) -> float:
        return llm_op_time_prefill_product(self.ctx, product, layer, n_rows, n_launch)
