"""Each stage entry point of include/llm_ops.h against the oracle's stage
functions (needs an MI355X).

"The Forward Pass in Java", Example 11 checks a forward pass tensor by tensor;
these tests do the same for the library's per-stage calls, feeding each stage
seeded inputs and comparing its output with the oracle's operations of that
stage: RMSNorm, the matrix-vector products (+ bias), RoPE and the binary16 K/V
store (llm_op_qkv); grouped-query attention over a cache written with
llm_op_kv_write (llm_op_attention); the output product and residual add
(llm_op_o); RMSNorm, gate/up and SwiGLU (llm_op_ffn_up); the down product and
residual add (llm_op_down); the final RMSNorm, the vocabulary product and the
greedy argmax (llm_op_logits).

Tolerance: the GPU sums products in another order than the oracle's sequential
dot, so each product output may differ by the standard bound for any
summation order, n * 2^-24 * sum_i |w_i x_i| (n terms), plus that of its
inputs where they come from an earlier product. With llama.cpp's rounding
points both sides round the same float inputs; where an input is itself
computed (an RMSNorm output) and differs by an ulp, its rounded value may sit
one step away, which the bounds allow twice per output row.
"""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from helpers import SMALL, SMALL_F16, SMALL_NEOX_BIAS, SMALL_PARTIAL_ROPE, SMALL_Q8, SMALL_Q8_RND

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import llama_family_decode_amd as llm

CFGS = [SMALL, SMALL_F16, SMALL_Q8, SMALL_NEOX_BIAS, SMALL_PARTIAL_ROPE, SMALL_Q8_RND]
U = 2.0 ** -24


class Stages:
    """The oracle's stage operations on one tensor set."""

    def __init__(self, cfg, ts):
        self.cfg = cfg
        self.by = {t.name: t for t in ts}

    def mat(self, name):
        t = self.by[name]
        return oracle.dequantize(t.dtype, t.data, t.n).reshape(t.ne[1], t.ne[0]), t.dtype

    def vec(self, name):
        t = self.by.get(name)
        return None if t is None else t.data.view(np.float32)

    def product(self, name, x):
        """(W x, bound on a reordered sum) with x rounded for W's type in the rounding mode."""
        w, dt = self.mat(name)
        aw = np.abs(w.astype(np.float64))
        flip = 0.0
        if self.cfg.numerics and dt != synth.F32:
            # where an input differs by an ulp (an RMSNorm output), its rounded
            # value may sit one step away: allow two such steps per row
            if dt == synth.Q8_0:
                step = np.repeat(np.abs(x.reshape(-1, 32)).max(1) / 127.0, 32)
            else:
                step = _ulp16(x)
            flip = 2.0 * (aw * step[None, :]).max(1)
            x = oracle.round_input(x, dt)
        y = oracle.matvec(np.ascontiguousarray(w), x, w.shape[0], w.shape[1])
        bound = w.shape[1] * U * (aw @ np.abs(x.astype(np.float64))) + flip
        return y, bound


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda")


def _host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _close(got, want, bound, what, slack=0.0):
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    lim = 2.0 * bound + slack + 1e-30
    j = int(np.argmax(err / lim))
    assert np.all(err <= lim), f"{what}: element {j} differs by {err[j]:.3e} (bound {lim[j]:.3e})"


def _rot_bound(bound, cfg, n_heads):
    """A rotated pair mixes two outputs: |dx'| <= |dx_a| + |dx_b| (|cos|, |sin| <= 1)."""
    hd, half = cfg.head_dim, cfg.n_rot // 2
    b = bound.reshape(n_heads, hd).copy()
    for i in range(half):
        a_, b_ = (i, i + half) if cfg.rope_neox else (2 * i, 2 * i + 1)
        s = b[:, a_] + b[:, b_]
        b[:, a_] = s
        b[:, b_] = s
    return b.reshape(-1)


def _ulp16(x):
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -14)))
    return 2.0 ** (e - 10)


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
def test_stage_qkv(cfg):
    ts = synth.make_tensor_set(cfg)
    gpu, o = llm.Model(cfg, ts), Stages(cfg, ts)
    H, KVH, hd = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    for layer, pos in ((0, 0), (cfg.n_layers - 1, 37)):
        print(f"[{cfg.name}] qkv layer {layer} pos {pos}", flush=True)
        x = synth.normal(cfg.seed, f"stage-x{layer}", cfg.dim, std=1.0)
        dq = torch.zeros(cfg.q_dim, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        llm.llm_op_qkv(gpu.ctx, layer, pos, _dev(x).data_ptr(), dq.data_ptr())
        q_gpu = _host(dq)
        k_bits, v_bits = gpu.kv_read(layer, pos)
        p = f"blk.{layer}."
        h = oracle.rmsnorm(x, o.vec(p + "attn_norm.weight"), cfg.eps)
        out = {}
        for n in "qkv":
            y, b = o.product(p + f"attn_{n}.weight", h)
            bias = o.vec(p + f"attn_{n}.bias")
            out[n] = (y if bias is None else (y + bias).astype(np.float32), b)
        q = oracle.rope(out["q"][0], H, hd, cfg.n_rot, pos, cfg.rope_base, cfg.rope_neox)
        k = oracle.rope(out["k"][0], KVH, hd, cfg.n_rot, pos, cfg.rope_base, cfg.rope_neox)
        qb = _rot_bound(out["q"][1], cfg, H)
        kb = _rot_bound(out["k"][1], cfg, KVH)
        # a cos/sin table entry may differ by an ulp from the oracle's: |x| 2^-23 per rotated value
        rot_slack = lambda v: 4 * U * np.repeat(np.abs(v).reshape(-1, 2).sum(1), 2) if not cfg.rope_neox else \
            8 * U * np.abs(v).max()
        _close(q_gpu, q, qb, "q", rot_slack(out["q"][0]))
        kf = k_bits.astype(np.uint16).view(np.float16).astype(np.float64)
        vf = v_bits.astype(np.uint16).view(np.float16).astype(np.float64)
        _close(kf, k, kb, "k (binary16)", _ulp16(k) + rot_slack(out["k"][0]))
        _close(vf, out["v"][0], out["v"][1], "v (binary16)", _ulp16(out["v"][0]))
    gpu.close()


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
def test_stage_attention(cfg):
    ts = synth.make_tensor_set(cfg)
    gpu = llm.Model(cfg, ts)
    H, KVH, hd, kvd = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.kv_dim
    layer = cfg.n_layers - 1
    P = 70
    kc = synth.normal_f16_bits(cfg.seed, "stage-k", P * kvd, std=1.0).reshape(P, kvd)
    vc = synth.normal_f16_bits(cfg.seed, "stage-v", P * kvd, std=1.0).reshape(P, kvd)
    gpu.kv_write(layer, 0, kc, vc)
    for pos in (0, 1, 31, P - 1):
        print(f"[{cfg.name}] attention pos {pos}", flush=True)
        q = synth.normal(cfg.seed, f"stage-q{pos}", cfg.q_dim, std=1.0)
        dout = torch.zeros(cfg.q_dim, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        llm.llm_op_attention(gpu.ctx, layer, pos, _dev(q).data_ptr(), dout.data_ptr())
        got = _host(dout)
        want, wts = oracle.attention(q, kc, vc, H, KVH, hd, pos, want_weights=True, round16=bool(cfg.numerics))
        # scores in another order: |ds_t| <= hd 2^-24 (|K_t| . |q_h|) / sqrt(hd)
        # + one rounding; the probabilities then move by at most 2 max|ds| +
        # a few roundings relative, and the weighted sum by the summation
        # bound; a rounded probability (rounding mode) may sit one binary16
        # step away
        K = np.abs(kc[:pos + 1].view(np.float16).astype(np.float64)).reshape(pos + 1, KVH, hd)
        V = np.abs(vc[:pos + 1].view(np.float16).astype(np.float64)).reshape(pos + 1, KVH, hd)
        qa = np.abs(q.astype(np.float64)).reshape(H, hd)
        bound = np.zeros((H, hd))
        for h in range(H):
            g = h // (H // KVH)
            sc = K[:, g] @ qa[h]
            ds = (hd * U * sc + U * sc) / np.sqrt(hd)
            pv = wts[h].astype(np.float64) @ V[:, g]
            rel = 2 * ds.max() + (pos + 16) * U + (2.0 ** -11 if cfg.numerics else 0.0)
            bound[h] = rel * pv
        _close(got, want, bound.reshape(-1) / 2, f"attention at {pos}")
    gpu.close()


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c.name)
def test_stage_output_ffn_down_and_logits(cfg):
    ts = synth.make_tensor_set(cfg)
    gpu, o = llm.Model(cfg, ts), Stages(cfg, ts)
    layer = cfg.n_layers - 1
    p = f"blk.{layer}."
    x = synth.normal(cfg.seed, "stage-res", cfg.dim, std=1.0)
    a = synth.normal(cfg.seed, "stage-att", cfg.q_dim, std=1.0)
    print(f"[{cfg.name}] output, ffn, down, logits", flush=True)
    # output product + residual
    dx = _dev(x)
    torch.cuda.synchronize()
    llm.llm_op_o(gpu.ctx, layer, _dev(a).data_ptr(), dx.data_ptr())
    y, b = o.product(p + "attn_output.weight", a)
    _close(_host(dx), (x + y).astype(np.float32), b, "x + W_o a", 2 * U * np.abs(x))
    # RMSNorm + gate/up + SwiGLU
    du = torch.zeros(cfg.ffn, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    llm.llm_op_ffn_up(gpu.ctx, layer, _dev(x).data_ptr(), du.data_ptr())
    h = oracle.rmsnorm(x, o.vec(p + "ffn_norm.weight"), cfg.eps)
    g, gb = o.product(p + "ffn_gate.weight", h)
    u, ub = o.product(p + "ffn_up.weight", h)
    sw = np.array([oracle.silu(z) for z in g], np.float32) * u
    # d(silu(g) u) <= |silu'(g)| |dg| |u| + |silu(g)| |du|, |silu'| <= 1.1
    sb = 1.1 * gb * np.abs(u) + np.abs(g) * ub
    _close(_host(du), sw, sb, "silu(W_g h) * (W_u h)", 8 * U * np.abs(sw))
    # down product + residual
    uu = synth.normal(cfg.seed, "stage-u", cfg.ffn, std=0.5)
    dx = _dev(x)
    torch.cuda.synchronize()
    llm.llm_op_down(gpu.ctx, layer, _dev(uu).data_ptr(), dx.data_ptr())
    y, b = o.product(p + "ffn_down.weight", uu)
    _close(_host(dx), (x + y).astype(np.float32), b, "x + W_down u", 2 * U * np.abs(x))
    # final RMSNorm + vocabulary product + argmax
    dl = torch.zeros(cfg.vocab, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    nxt = llm.llm_op_logits(gpu.ctx, _dev(x).data_ptr(), dl.data_ptr())
    got = _host(dl)
    hn = oracle.rmsnorm(x, o.vec("output_norm.weight"), cfg.eps)
    wname = "output.weight" if "output.weight" in o.by else "token_embd.weight"
    y, b = o.product(wname, hn)
    _close(got, y, b, "logits")
    assert nxt == int(np.flatnonzero(got == got.max())[0])  # the first strict maximum of the GPU logits
    gpu.close()


def test_stage_argument_errors():
    cfg = SMALL
    gpu = llm.Model(cfg, synth.make_tensor_set(cfg))
    L = llm.lib()
    buf = torch.zeros(cfg.ffn + cfg.q_dim, dtype=torch.float32, device="cuda")
    d = buf.data_ptr()
    assert L.llm_op_qkv(gpu.ctx, cfg.n_layers, 0, d, d) == -1
    assert L.llm_op_qkv(gpu.ctx, 0, cfg.n_ctx, d, d) == -1
    assert L.llm_op_attention(gpu.ctx, -1, 0, d, d) == -1
    assert L.llm_op_o(gpu.ctx, 0, None, d) == -1
    assert L.llm_op_ffn_up(gpu.ctx, 0, d, None) == -1
    assert L.llm_op_down(gpu.ctx, 0, None, None) == -1
    assert L.llm_op_logits(gpu.ctx, None, None, None) == -1
    assert gpu.kv_len() == 0
    gpu.close()


@pytest.mark.parametrize("cfg", [SMALL_F16, SMALL_Q8_RND], ids=lambda c: c.name)
def test_time_prefill_product(cfg):
    # every prompt-pass product times over one row, a whole 128-row tile and a
    # ragged 300 rows; the cache is untouched, and a prompt pass afterwards
    # gives the logits of a context that never ran the timing
    ts = synth.make_tensor_set(cfg)
    toks = synth.prompt(cfg, 6)
    gpu, ref = llm.Model(cfg, ts), llm.Model(cfg, ts)
    ref.prefill(toks)
    gpu.prefill(toks)
    for prod in (llm.PRODUCT_QKV, llm.PRODUCT_O, llm.PRODUCT_GATE_UP, llm.PRODUCT_DOWN):
        for n in (1, 128, 300):
            ms = gpu.time_product(prod, n, cfg.n_layers - 1, 2)
            assert 0.0 < ms < 100.0, (prod, n, ms)
    assert gpu.kv_len() == len(toks)
    gpu.reset()
    gpu.prefill(toks)
    assert np.array_equal(gpu.logits().view(np.uint32), ref.logits().view(np.uint32))
    L = llm.lib()
    ms = ctypes.c_float()
    chunk = llm.llm_op_prefill_chunk()
    for args in ((4, 0, 1, 1), (-1, 0, 1, 1), (0, cfg.n_layers, 1, 1), (0, 0, 0, 1), (0, 0, chunk + 1, 1),
                 (0, 0, 1, 0)):
        assert L.llm_op_time_prefill_product(gpu.ctx, *args, ctypes.byref(ms)) == -1, args
    assert L.llm_op_time_prefill_product(gpu.ctx, 0, 0, 1, 1, None) == -1
    gpu.close()
    ref.close()
