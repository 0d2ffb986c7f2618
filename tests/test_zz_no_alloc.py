"""The allocation-free attention entry point against llm_op_attention (needs an MI355X).

llm_op_attention_noalloc runs the same kernels as llm_op_attention with its
scratch in a file-scope device array instead of the context's arena, so its
output must equal llm_op_attention's bit for bit. Two calls in a row, the
second over fewer cache rows (a smaller input), check that the array's
contents left by one call do not leak into the next; the float and the
rounding numerics and two shapes (a small GQA model and the 1B shape) are
covered.
"""
import numpy as np
import pytest

import synth
from helpers import SMALL_Q8, SMALL_Q8_RND

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import llama_family_decode_amd as llm

CASES = [SMALL_Q8.with_(n_ctx=300), SMALL_Q8_RND.with_(n_ctx=300), synth.C4.with_(n_ctx=600)]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_noalloc_attention_equals_llm_op_attention(cfg):
    ts = synth.make_tensor_set(cfg)
    gpu = llm.Model(cfg, ts)
    L = llm.lib()
    layer = cfg.n_layers - 1
    P = cfg.n_ctx - 10
    kvd = cfg.kv_dim
    kc = synth.normal_f16_bits(cfg.seed, "noalloc-k", P * kvd, std=1.0).reshape(P, kvd)
    vc = synth.normal_f16_bits(cfg.seed, "noalloc-v", P * kvd, std=1.0).reshape(P, kvd)
    gpu.kv_write(layer, 0, kc, vc)
    for pos in (P - 1, 37):  # the second call attends fewer rows
        print(f"[{cfg.name}] noalloc attention at pos {pos}", flush=True)
        q = torch.from_numpy(synth.normal(cfg.seed, f"noalloc-q{pos}", cfg.q_dim, std=1.0)).to("cuda")
        want = torch.full((cfg.q_dim,), float("nan"), dtype=torch.float32, device="cuda")
        got = torch.full((cfg.q_dim,), float("nan"), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        assert L.llm_op_attention(gpu.ctx, layer, pos, q.data_ptr(), want.data_ptr()) == 0
        assert L.llm_op_attention_noalloc(gpu.ctx, layer, pos, q.data_ptr(), got.data_ptr()) == 0
        torch.cuda.synchronize()
        w, g = want.cpu().numpy(), got.cpu().numpy()
        assert np.all(np.isfinite(g))
        assert np.array_equal(g.view(np.uint32), w.view(np.uint32)), f"pos {pos}: outputs differ"
    # argument errors change nothing and name themselves
    assert L.llm_op_attention_noalloc(gpu.ctx, cfg.n_layers, 0, q.data_ptr(), got.data_ptr()) == -1
    assert L.llm_op_attention_noalloc(gpu.ctx, 0, cfg.n_ctx, q.data_ptr(), got.data_ptr()) == -1
    assert L.llm_op_attention_noalloc(gpu.ctx, 0, 0, None, got.data_ptr()) == -1
    assert gpu.kv_len() == 0
    gpu.close()
