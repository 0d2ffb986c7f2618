"""Prefill with chosen output rows against the oracle (needs an MI355X).

"What a Llama model computes, and why", section 4: the prompt pass yields a
logit row for every prompt position, and the last layer's output product and
FFN are only needed for the rows that are read. llm_prefill_rows runs that
pruned last layer and returns the chosen rows' logits; the oracle computes the
same rows with the whole last layer. Every chosen row is held to the logit
tolerance of the weight type (and to the oracle's greedy token where its top-2
gap exceeds it); the cache the pruned pass leaves is checked by the decode
steps that follow and by the K/V rows themselves.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import (SMALL, SMALL_F16, SMALL_FREQS, SMALL_MHA, SMALL_NEOX_BIAS, SMALL_PARTIAL_ROPE, SMALL_Q8,
                     SMALL_F16_RND, SMALL_Q8_RND, SMALL_SPAN_ALL, SMALL_SPAN_RND)
from test_gpu_parity import check_kv, check_step, first_max, tol, top2_gap

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import llama_family_decode_amd as llm

    CHUNK = llm.llm_op_prefill_chunk()


@pytest.fixture(autouse=True)
def graph_path(monkeypatch):
    monkeypatch.setenv("LLM_STEP", "graph")


def check_rows(cfg, got, want, where):
    t = tol(cfg)
    assert got.shape == want.shape
    assert np.all(np.isfinite(got)), f"{where}: non-finite logits"
    err = np.max(np.abs(got.astype(np.float64) - want), axis=1)
    j = int(np.argmax(err))
    assert err[j] <= t, f"{where}: output {j} max |dlogit| = {err[j]:.3e} > {t}"
    for j in range(want.shape[0]):
        if top2_gap(want[j]) > t:
            assert first_max(got[j]) == oracle.argmax(want[j]), f"{where}: output {j} greedy token differs"
    return float(err.max())


def run_rows(cfg, n_prompt, rows, n_steps=2, split=None):
    """Prefill n_prompt tokens (in two calls at `split` if given) asking for
    `rows` of each call, then decode n_steps, all against the oracle."""
    ts = synth.make_tensor_set(cfg)
    toks = synth.prompt(cfg, n_prompt)
    gpu = llm.Model(cfg, ts)
    ref = oracle.Model(cfg, ts)
    parts = [toks] if split is None else [toks[:split], toks[split:]]
    print(f"[{cfg.name}] prompt {n_prompt} split {split} rows {rows if rows is not None else 'all'}", flush=True)
    worst = 0.0
    for part in parts:
        r = list(range(len(part))) if rows is None else [x for x in rows if x < len(part)]
        got = gpu.prefill_rows(part, None if rows is None else r)
        want = ref.prefill_rows(part, r)
        worst = max(worst, check_rows(cfg, got, want, f"prefill of {len(part)}"))
    assert gpu.kv_len() == ref.kv_len() == n_prompt
    # the pruned last layer must still leave every cache row in place:
    # teacher-forced decode steps read all of them
    tok = int(toks[-1])
    pos = n_prompt
    for step in range(n_steps):
        w = ref.forward(tok, pos)
        nxt = gpu.decode(tok, pos)
        worst = max(worst, check_step(cfg, gpu.logits(), w, nxt, f"step {step} pos {pos}"))
        tok, pos = oracle.argmax(w), pos + 1
    check_kv(cfg, gpu, ref, sorted({0, n_prompt // 2, n_prompt - 1}), None)
    print(f"[{cfg.name}] rows: max |dlogit| {worst:.3e}", flush=True)
    gpu.close()
    ref.close()
    return worst


SMALLS = [SMALL, SMALL_F16, SMALL_Q8, SMALL_NEOX_BIAS, SMALL_PARTIAL_ROPE, SMALL_MHA, SMALL_FREQS, SMALL_SPAN_ALL,
          SMALL_F16_RND, SMALL_Q8_RND, SMALL_SPAN_RND]


@pytest.mark.parametrize("cfg", SMALLS, ids=lambda c: c.name)
def test_rows_small_unsorted_with_repeats(cfg):
    run_rows(cfg, 13, [12, 0, 5, 5, 7, 11])


@pytest.mark.parametrize("cfg", [SMALL, SMALL_Q8], ids=lambda c: c.name)
def test_every_row_small(cfg):
    run_rows(cfg, 13, None)


def test_rows_continue_a_sequence():
    # the second call's rows are indices into its own prompt, at positions 7..
    run_rows(SMALL_F16, 13, [0, 5, 3], split=7)


def test_rows_across_chunks_and_ragged_tail():
    # three chunks, the last one 76 rows; rows on both sides of each edge
    n = 2 * CHUNK + 76
    cfg = SMALL_Q8.with_(n_ctx=n + 24)
    run_rows(cfg, n, [n - 1, 0, CHUNK - 1, CHUNK, 2 * CHUNK - 1, 2 * CHUNK, 700, 700, n - 2], n_steps=1)


def test_rows_repeated_past_one_chunk():
    # more wanted rows in one chunk than the chunk holds (repeats): the last
    # layer runs them in batches of at most one chunk
    n = CHUNK + 52
    rows = [5, CHUNK - 1, 0] * ((CHUNK + 600) // 3) + [CHUNK, n - 1]
    cfg = SMALL_Q8.with_(n_ctx=len(rows) + 8)
    assert cfg.n_ctx > CHUNK + 600
    run_rows(cfg, n, rows, n_steps=1)


def test_rows_1b_q8_shape():
    cfg = synth.C4.with_(n_ctx=160)
    run_rows(cfg, 40, [39, 0, 17, 38], n_steps=1)


def test_rows_1b_f16_neox_bias_shape():
    cfg = synth.C5.with_(n_ctx=160)
    run_rows(cfg, 40, [20, 39, 1], n_steps=1)


def test_last_row_matches_llm_prefill():
    # llm_prefill computes only the last row, through the decode vocabulary
    # kernel; the chosen-rows call through the batched product
    cfg = SMALL_Q8
    ts = synth.make_tensor_set(cfg)
    toks = synth.prompt(cfg, 21)
    a = llm.Model(cfg, ts)
    nxt = a.prefill(toks)
    la = a.logits()
    b = llm.Model(cfg, ts)
    lb = b.prefill_rows(toks, [20])[0]
    assert nxt == first_max(la)
    assert float(np.max(np.abs(la.astype(np.float64) - lb))) <= tol(cfg) / 4
    for l in range(cfg.n_layers):
        for p in (0, 10, 20):
            ka, va = a.kv_read(l, p)
            kb, vb = b.kv_read(l, p)
            assert np.array_equal(ka, kb) and np.array_equal(va, vb), f"KV differs at layer {l} pos {p}"
    a.close()
    b.close()


def test_rows_argument_errors():
    cfg = SMALL
    ts = synth.make_tensor_set(cfg)
    toks = np.ascontiguousarray(synth.prompt(cfg, 6), np.int32)
    m = llm.Model(cfg, ts)
    out = torch.empty((8, cfg.vocab), dtype=torch.float32, device="cuda")
    L = llm.lib()

    def call(rows, n_rows, d=out.data_ptr(), tokens=toks):
        rw = None if rows is None else np.ascontiguousarray(rows, np.int32)
        return L.llm_prefill_rows(m.ctx, tokens.ctypes.data, tokens.size, None if rw is None else rw.ctypes.data,
                                  n_rows, d)

    assert call([6], 1) == -1          # row past the prompt
    assert call([-1], 1) == -1         # negative row
    assert call([0], 0) == -1          # no rows
    assert call(None, 5) == -1         # all rows needs n_rows == n
    assert call([0], 1, d=None) == -1  # no output buffer
    bad = toks.copy()
    bad[2] = cfg.vocab
    assert call([0], 1, tokens=bad) == -6
    assert m.kv_len() == 0
    got = m.prefill_rows(toks, [5])
    assert m.kv_len() == 6
    ref = oracle.Model(cfg, ts)
    check_rows(cfg, got, ref.prefill_rows(toks, [5]), "after rejected calls")
    m.close()
    ref.close()
