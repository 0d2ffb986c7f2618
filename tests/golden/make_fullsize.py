"""Writes the oracle's expected values for the full-size workloads.

Calls only the CPU oracle (``oracle/``) and the seeded input generator
(``synth/``); nothing here comes from the GPU library. For each workload the
oracle prefills the seeded prompt ("What a Llama model computes, and why",
section 4), then decodes greedily, each step feeding the previous step's first
strict maximum ("The Forward Pass in Java", Examples 9 and 12). Stored per
workload (``fullsize_<name>.npz``):

* ``tokens[i]``: the token fed at decode step i+1 (teacher forcing for the GPU);
* ``full_steps`` / ``full_logits``: whole logit vectors at a few steps (step 0
  is the prompt's last row, step i the i-th decode step);
* ``sample_idx`` / ``sample_logits``: a fixed sample of logit indices at every
  step, plus ``top2`` (largest two logits) and ``argmax`` per step;
* ``kv_pos`` / ``kv_k`` / ``kv_v``: binary16 K and V of every layer at a few
  positions;
* for the prompt-only workload, the logits of chosen prompt rows
  (``row_idx`` / ``row_logits``).

The rounding-mode workload (c4_q8_0_llamacpp_ctx2048: the headline model with
llama.cpp's rounding points, "What a Llama model computes, and why", section 8)
runs 16 decode steps.

With --variant V the script runs a workload again on another build of the
oracle that evaluates the same definition in another valid way (V = desc:
every dot product summed over the input index descending, liboracle_desc.so;
V = f64: every sum accumulated in double and rounded once, liboracle_f64.so),
teacher-forced with the stored tokens, and writes ``fullsize_<name>_<V>.npz``:
at every step the largest |difference| of its logits from the stored ones over
the sample (``sample_dist``) and over the whole vector at the stored steps
(``full_dist``), and its own binary16 K and V of every layer at the stored
positions (``kv_k`` / ``kv_v``). That is how far the rounding of the sums alone
moves this workload's logits and cache.

Usage: python tests/golden/make_fullsize.py [--variant desc|f64] [workload ...]   (default: all)
The 8192-position prompt takes the oracle about 70 minutes on 8 cores.
"""
import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

N_SAMPLE = 1024
# workload -> (config, decode steps, steps with whole logit vectors, prompt rows with logits)
WORKLOADS = {
    "c3_f16_ctx2048": (synth.C3, 128, (0, 1, 128), None),
    "c4_q8_0_ctx2048": (synth.C4, 128, (0, 1, 128), None),
    "c4_q8_0_ctx8192": (synth.C4_LONG, 128, (0, 1, 128), None),
    "c5_qwen2_prefill512": (synth.C5, 0, (0,), (0, 255, 511)),
    # the headline workload with llama.cpp's rounding points (numerics 1)
    "c4_q8_0_llamacpp_ctx2048": (synth.C4.with_(name="llama-1b-q8_0-llamacpp", numerics=1), 16, (0, 1, 16), None),
}


def out_path(name: str) -> str:
    return os.path.join(HERE, f"fullsize_{name}.npz")


VARIANTS = ("desc", "f64")


def variant_path(name: str, variant: str) -> str:
    return os.path.join(HERE, f"fullsize_{name}_{variant}.npz")


def sample_indices(vocab: int) -> np.ndarray:
    return np.unique(np.linspace(0, vocab - 1, N_SAMPLE).round().astype(np.int32))


def kv_positions(P: int, steps: int):
    last = P + steps - 1
    return sorted({0, P // 2, P - 1, P + steps // 2, last} if steps else {0, P // 2, P - 1})


def top2(v: np.ndarray):
    i = int(oracle.argmax(v))
    rest = np.delete(v, i)
    return i, float(v[i]), float(rest.max())


def make(name: str):
    cfg, steps, full_steps, rows = WORKLOADS[name]
    P = cfg.prompt_len
    t0 = time.time()
    ts = synth.make_tensor_set(cfg)
    toks = synth.prompt(cfg, P)
    m = oracle.Model(cfg, ts)
    print(f"[{name}] loaded in {time.time() - t0:.1f}s; prefill of {P} rows", flush=True)
    sidx = sample_indices(cfg.vocab)
    n_full = len(full_steps)
    full = np.zeros((n_full, cfg.vocab), np.float32)
    samp = np.zeros((steps + 1, sidx.size), np.float32)
    tt = np.zeros((steps + 1, 2), np.float32)
    am = np.zeros(steps + 1, np.int32)
    fed = np.zeros(steps, np.int32)
    extra = {}
    t1 = time.time()
    if rows is not None:
        rl = m.prefill_rows(toks, list(rows))
        extra["row_idx"] = np.array(rows, np.int32)
        extra["row_logits"] = rl
        logits = rl[list(rows).index(P - 1)]
    else:
        logits = m.prefill(toks)
    print(f"[{name}] prefill {time.time() - t1:.1f}s", flush=True)

    def record(step, v):
        i, a, b = top2(v)
        am[step], tt[step] = i, (a, b)
        samp[step] = v[sidx]
        if step in full_steps:
            full[list(full_steps).index(step)] = v

    record(0, logits)
    t2 = time.time()
    for s in range(1, steps + 1):
        fed[s - 1] = am[s - 1]
        logits = m.forward(int(fed[s - 1]), P + s - 1)
        record(s, logits)
        if s % 16 == 0:
            print(f"[{name}] decode step {s}/{steps} ({time.time() - t2:.1f}s)", flush=True)
    kvp = kv_positions(P, steps)
    kvd = cfg.n_kv_heads * cfg.head_dim
    kk = np.zeros((len(kvp), cfg.n_layers, kvd), np.uint16)
    vv = np.zeros_like(kk)
    for i, p in enumerate(kvp):
        for l in range(cfg.n_layers):
            kk[i, l], vv[i, l] = m.kv_read(l, p)
    np.savez_compressed(
        out_path(name), config=np.array(cfg.name), prompt_len=np.int32(P), steps=np.int32(steps),
        vocab=np.int32(cfg.vocab), prompt_sha256=np.array(hashlib.sha256(toks.tobytes()).hexdigest()),
        tokens=fed, full_steps=np.array(full_steps, np.int32), full_logits=full, sample_idx=sidx,
        sample_logits=samp, top2=tt, argmax=am, kv_pos=np.array(kvp, np.int32), kv_k=kk, kv_v=vv, **extra)
    m.close()
    print(f"[{name}] written in {time.time() - t0:.1f}s total", flush=True)


def make_variant(name: str, variant: str):
    """The workload on another build of the oracle, against the stored values."""
    cfg, steps, full_steps, rows = WORKLOADS[name]
    with np.load(out_path(name), allow_pickle=False) as z:
        g = {k: z[k] for k in z.files}
    P = int(g["prompt_len"])
    t0 = time.time()
    toks = synth.prompt(cfg, P)
    assert hashlib.sha256(toks.tobytes()).hexdigest() == str(g["prompt_sha256"])
    m = oracle.Model(cfg, synth.make_tensor_set(cfg), variant=variant)
    sidx = g["sample_idx"]
    full = {int(s_): g["full_logits"][i] for i, s_ in enumerate(g["full_steps"])}
    sd = np.zeros(steps + 1, np.float32)
    fd = np.zeros(len(full_steps), np.float32)

    def record(step, v):
        sd[step] = np.max(np.abs(v[sidx].astype(np.float64) - g["sample_logits"][step]))
        if step in full:
            fd[list(full_steps).index(step)] = np.max(np.abs(v.astype(np.float64) - full[step]))

    print(f"[{name} {variant}] prefill of {P} rows", flush=True)
    record(0, m.prefill(toks))
    for s_ in range(1, steps + 1):
        record(s_, m.forward(int(g["tokens"][s_ - 1]), P + s_ - 1))
        if s_ % 16 == 0:
            print(f"[{name} {variant}] decode step {s_}/{steps}", flush=True)
    kvp = [int(p) for p in g["kv_pos"]]
    kk = np.zeros_like(g["kv_k"])
    vv = np.zeros_like(g["kv_v"])
    for i, p in enumerate(kvp):
        for l in range(cfg.n_layers):
            kk[i, l], vv[i, l] = m.kv_read(l, p)
    np.savez_compressed(variant_path(name, variant), config=np.array(cfg.name), sample_dist=sd,
                        full_steps=np.array(full_steps, np.int32), full_dist=fd, kv_pos=np.array(kvp, np.int32),
                        kv_k=kk, kv_v=vv)
    m.close()
    print(f"[{name} {variant}] median {np.median(sd):.2e} max {sd.max():.2e}; written in {time.time() - t0:.1f}s",
          flush=True)


if __name__ == "__main__":
    args = sys.argv[1:]
    variant = None
    if "--variant" in args:
        i = args.index("--variant")
        variant = args[i + 1]
        assert variant in VARIANTS, f"--variant takes one of {VARIANTS}"
        del args[i:i + 2]
    for n in args or list(WORKLOADS):
        if variant:
            make_variant(n, variant)
        else:
            make(n)
