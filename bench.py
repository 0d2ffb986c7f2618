#!/usr/bin/env python3
"""Benchmark of the Llama-family forward pass on one MI355X.

Headline workload: the 1B-shape model (16 layers, d 2048, 32/8 heads of 64,
FFN 8192, vocab 128256) with Q8_0 matrices and a tied F32 embedding, seeded
random weights; the KV cache is prefilled with 2048 seeded prompt ids, then K
greedy decode steps run at positions 2048 .. 2048+K-1 (device-side token
feedback, llm_generate). A step is one token's full forward pass.

Decode runs the persistent step kernel (one cooperative launch per token,
compiled for this shape). The line also reports
  - roofline: that kernel, the only one a decode step launches, timed with HIP
    events on the context's stream; its algorithmic bytes are the step's
    (every weight once, the K/V rows 0..pos, the new K/V row); HBM traffic
    from the committed rocprofv3 counter runs;
  - prefill: llm_prefill of 512 seeded ids on the Qwen2-style F16 variant
    (also with every row's logits, and with llama.cpp's rounding points);
  - decode_reports: the same decode with F16 matrices at context 2048, with
    Q8_0 at context 8192 (attention a larger share of the bytes), with
    Llama 3's RoPE frequency factors (rope_freqs.weight), at context 8192
    with a 1024-row sliding window plus 4 sink rows, with llama.cpp's
    rounding points (the step kernel's rounding variant), and with YaRN
    (factor 16);
  - cpu_baseline: the CPU oracle on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps 128] [--warmup 8]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
F16_MFMA_PEAK_TFLOPS = 2500.0  # dense
INT8_MFMA_PEAK_TOPS = 5000.0  # dense


def span_rows(cfg, pos):
    """Cache rows the query at pos attends: 0..pos, or with a window w the last
    w rows plus the sink rows below them."""
    w = getattr(cfg, "attn_window", 0)
    if w <= 0:
        return pos + 1
    lo = max(0, pos - w + 1)
    return min(getattr(cfg, "attn_sinks", 0), lo) + pos - lo + 1


def algorithmic_step_bytes(cfg, pos):
    """Bytes one decode step at position pos must move: every weight once, the
    attended K and V rows read (0..pos, or the window and sinks), one K/V row
    written, the embedding row (tied: the table is also the output matrix,
    read once by the vocabulary product)."""
    import synth

    total = 0
    for name, dt, ne, kind in synth.tensor_specs(cfg):
        n = 1
        for e in ne:
            n *= e
        if name == "rope_freqs.weight":  # consumed at load into the RoPE table
            continue
        if name == "token_embd.weight":
            total += synth.nbytes_of(dt, cfg.dim * cfg.vocab) if cfg.tied else synth.nbytes_of(dt, cfg.dim)
            continue
        total += synth.nbytes_of(dt, n)
    kv_row = 2 * cfg.n_layers * cfg.kv_dim * 2  # K and V, f16
    total += kv_row * span_rows(cfg, pos)  # attended rows (row pos written then read)
    return total


def read_traffic():
    """HBM bytes per launch of the step kernel from the committed counter runs
    (profiles/step_q8_1b_ctx2048_counters.txt), or None when absent."""
    p = os.path.join(ROOT, "profiles", "step_q8_1b_ctx2048_counters.txt")
    if not os.path.exists(p):
        return None
    for line in open(p):
        if line.startswith("traffic_bytes_per_launch:"):
            try:
                return float(line.split(":", 1)[1])
            except ValueError:
                return None
    return None


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, ctx_len, budget_s=8.0):
    """The oracle, untuned, on bounded samples of the same workloads:
      - decode steps of the headline model at positions ctx_len.. over a
        ctx_len-row cache (seeded binary16 rows written into the oracle's
        cache: the oracle's step time does not depend on the cached values,
        and its own 2048-row prompt pass takes minutes), with every thread
        the process may use and with one thread;
      - the prompt pass of the Qwen2-style F16 model on the first rows of its
        512-id prompt, with every thread and with one thread.
    Each sample runs about budget_s seconds (at least one step)."""
    import numpy as np

    import oracle
    import synth

    def timed(fn, budget, cap):
        n, t0 = 0, time.perf_counter()
        while True:
            fn(n)
            n += 1
            if time.perf_counter() - t0 > budget or n >= cap:
                return n, time.perf_counter() - t0

    all_threads = oracle.max_threads()
    ts = synth.make_tensor_set(cfg)
    m = oracle.Model(cfg, ts)
    del ts
    kvd = cfg.kv_dim
    for l in range(cfg.n_layers):
        k = synth.normal_f16_bits(cfg.seed, f"cpu-baseline-k{l}", ctx_len * kvd, std=1.0).reshape(ctx_len, kvd)
        v = synth.normal_f16_bits(cfg.seed, f"cpu-baseline-v{l}", ctx_len * kvd, std=1.0).reshape(ctx_len, kvd)
        for p in range(ctx_len):
            m.kv_write(l, p, k[p], v[p])
    toks = synth.prompt(cfg, 64, stream="cpu-baseline")
    decode = {}
    for threads in (all_threads, 1):
        oracle.set_threads(threads)
        m.set_len(ctx_len)
        n, dt = timed(lambda i: m.forward(int(toks[i % 64]), ctx_len + i), budget_s, 64)
        decode[threads] = (n, dt)
    m.close()
    c5 = synth.C5
    ts = synth.make_tensor_set(c5)
    pm = oracle.Model(c5, ts)
    del ts
    p5 = synth.prompt(c5, 512)
    prefill = {}
    for threads, rows in ((all_threads, 32), (1, 4)):
        oracle.set_threads(threads)
        pm.reset()
        t0 = time.perf_counter()
        pm.prefill(p5[:rows])
        prefill[threads] = (rows, time.perf_counter() - t0)
    pm.close()
    oracle.set_threads(all_threads)
    n_all, dt_all = decode[all_threads]
    n_one, dt_one = decode[1]
    return {"value": round(n_all / dt_all, 4), "unit": "tok/s", "cores": all_threads, "kind": "oracle",
            "cpu_model": _cpu_model(), "host_cpus": os.cpu_count(),
            "one_thread_tok_s": round(n_one / dt_one, 4),
            "prefill_tok_s": round(prefill[all_threads][0] / prefill[all_threads][1], 3),
            "prefill_one_thread_tok_s": round(prefill[1][0] / prefill[1][1], 3),
            "sample": f"decode: {n_all} steps on {all_threads} threads and {n_one} on 1 thread of the same 1B Q8_0 "
                      f"model at positions {ctx_len}.. over a {ctx_len}-row cache (seeded binary16 rows written "
                      f"into the oracle's cache); prefill: the first {prefill[all_threads][0]} rows "
                      f"({all_threads} threads) and {prefill[1][0]} rows (1 thread) of the 512-id prompt of the "
                      f"Qwen2-style F16 1B model, as one prompt pass"}


def product_fractions(llm, model, cfg, n_rows, peak, n_launch=20):
    """Each prefill product of layer 0 over n_rows rows, timed with HIP events
    on the context's stream (llm_op_time_prefill_product): average us per
    launch, algorithmic TFLOP/s (2 * rows * outputs * inputs, the lo pass not
    counted) and its fraction of the dense matrix-core peak."""
    shapes = {"qkv": (llm.PRODUCT_QKV, cfg.q_dim + 2 * cfg.kv_dim, cfg.dim),
              "o": (llm.PRODUCT_O, cfg.dim, cfg.q_dim),
              "gate_up": (llm.PRODUCT_GATE_UP, 2 * cfg.ffn, cfg.dim),
              "down": (llm.PRODUCT_DOWN, cfg.dim, cfg.ffn)}
    out = {}
    for name, (prod, n_out, n_in) in shapes.items():
        ms = model.time_product(prod, n_rows, 0, n_launch)
        tf = 2.0 * n_rows * n_out * n_in / (ms * 1e-3) / 1e12
        out[name] = {"us": round(ms * 1e3, 1), "tflops": round(tf, 1), "frac": round(tf / peak, 4)}
    return out


def measure_prefill(llm, synth, np, torch, reps=5, products=True):
    """llm_prefill of 512 seeded ids on the Qwen2-style F16 1B model from an
    empty cache, median of `reps`, and llm_prefill_rows of the same ids with
    every row's logits; MFMA fraction = algorithmic GEMM FLOPs / time / F16
    dense peak."""
    c5 = synth.C5
    ts = synth.make_tensor_set(c5)
    pm = llm.Model(c5, ts)
    del ts
    p5 = synth.prompt(c5, 512)
    pm.prefill(p5)
    pm.reset()
    ptimes = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        pm.prefill(p5)
        torch.cuda.synchronize()
        ptimes.append(time.perf_counter() - t0)
        pm.reset()
    pt = float(np.median(ptimes))
    # the same prompt with the logits of every row (llm_prefill_rows)
    out = torch.empty((512, c5.vocab), dtype=torch.float32, device="cuda")
    rtimes = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        llm.llm_prefill_rows(pm.ctx, p5, None, out.data_ptr())
        torch.cuda.synchronize()
        rtimes.append(time.perf_counter() - t0)
        pm.reset()
    rt = float(np.median(rtimes))
    products = product_fractions(llm, pm, c5, 512, F16_MFMA_PEAK_TFLOPS) if products else {}
    # GEMM FLOPs the pass needs: the last layer's output product and FFN run
    # on the one row whose logits are read (on all 512 for every row's logits)
    qkv = c5.dim * (c5.q_dim + 2 * c5.kv_dim)
    rest = c5.q_dim * c5.dim + 3 * c5.dim * c5.ffn
    gemm_flop = 2.0 * (512 * c5.n_layers * qkv + 512 * (c5.n_layers - 1) * rest + rest)
    rows_flop = 2.0 * 512 * (c5.n_layers * (qkv + rest) + c5.vocab * c5.dim)
    pm.close()
    del pm, out
    torch.cuda.empty_cache()
    # the same prompt with llama.cpp's rounding points (numerics 1)
    c5n = c5.with_(numerics=1)
    ts = synth.make_tensor_set(c5n)
    pn = llm.Model(c5n, ts)
    del ts
    pn.prefill(p5)
    pn.reset()
    ntimes = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        pn.prefill(p5)
        torch.cuda.synchronize()
        ntimes.append(time.perf_counter() - t0)
        pn.reset()
    nt = float(np.median(ntimes))
    pn.close()
    del pn
    torch.cuda.empty_cache()
    print(f"# prefill 512: {pt * 1e3:.2f} ms, {512 / pt:.0f} tok/s; with all 512 logit rows {rt * 1e3:.2f} ms; "
          f"with llama.cpp's rounding points {nt * 1e3:.2f} ms"
          + ("; products at 512 rows: " + ", ".join(f"{k} {v['us']} us ({v['frac']:.3f})" for k, v in products.items())
             if products else ""), file=sys.stderr, flush=True)
    return {"config": c5.name, "tokens": 512, "ms": round(pt * 1e3, 3), "tok_s": round(512 / pt, 1),
            "gemm_tflop": round(gemm_flop / 1e12, 4), "products_512_rows": products,
            "whole_prefill_mfma_frac": round(gemm_flop / pt / 1e12 / F16_MFMA_PEAK_TFLOPS, 4),
            "all_rows_ms": round(rt * 1e3, 3), "all_rows_gemm_tflop": round(rows_flop / 1e12, 4),
            "all_rows_mfma_frac": round(rows_flop / rt / 1e12 / F16_MFMA_PEAK_TFLOPS, 4),
            "llamacpp_numerics_ms": round(nt * 1e3, 3), "llamacpp_numerics_tok_s": round(512 / nt, 1),
            "llamacpp_numerics_mfma_frac": round(gemm_flop / nt / 1e12 / F16_MFMA_PEAK_TFLOPS, 4)}


def measure_decode_report(llm, synth, np, torch, cfg, ctx_len, steps=64, reps=3):
    """A reported (not headline) decode workload: llm_prefill of ctx_len seeded
    ids, then `steps` greedy steps by llm_generate, median of `reps`."""
    ts = synth.make_tensor_set(cfg)
    m = llm.Model(cfg, ts)
    del ts
    nxt = m.prefill(synth.prompt(cfg, ctx_len))
    m.generate(nxt, 4)
    m.rewind(ctx_len)
    times = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        m.generate(nxt, steps)
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
        m.rewind(ctx_len)
    kind = llm.llm_op_step_kind(m.ctx)
    m.close()
    del m
    torch.cuda.empty_cache()
    dt = float(np.median(times))
    tok_s = steps / dt
    b = algorithmic_step_bytes(cfg, ctx_len + steps // 2)
    print(f"# report {cfg.name} ctx {ctx_len}: {tok_s:.1f} tok/s, {b * tok_s / 1e9:.0f} GB/s", file=sys.stderr,
          flush=True)
    return {"config": cfg.name, "ctx": ctx_len, "steps": steps, "tok_s": round(tok_s, 1),
            "ms_per_token": round(1e3 * dt / steps, 4), "bytes_per_token": b,
            "hbm_frac": round(b * tok_s / 1e9 / HBM_PEAK_GBS, 4), "step_kind": kind}


def measure_prefill_q8_llamacpp(llm, synth, np, torch, n=2048, reps=3, products=True):
    """llm_prefill of the headline workload's 2048 ids with llama.cpp's
    rounding points: the Q8_0 products on the integer matrix cores."""
    cfg = synth.C4.with_(name="llama-1b-q8_0-llamacpp", numerics=1)
    m = llm.Model(cfg, synth.make_tensor_set(cfg))
    int8 = llm.llm_op_prefill_int8(m.ctx)
    toks = synth.prompt(cfg, n)
    m.prefill(toks)
    m.reset()
    times = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        m.prefill(toks)
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
        m.reset()
    products = product_fractions(llm, m, cfg, n, INT8_MFMA_PEAK_TOPS if int8 else F16_MFMA_PEAK_TFLOPS) if products else {}
    m.close()
    del m
    torch.cuda.empty_cache()
    dt = float(np.median(times))
    print(f"# prefill {n} (Q8_0, llama.cpp rounding points, integer products {int8}): {dt * 1e3:.2f} ms"
          + ("; products " + ", ".join(f"{k} {v['us']} us ({v['frac']:.3f} of the int8 peak)"
                                        for k, v in products.items()) if products else ""),
          file=sys.stderr, flush=True)
    return {"config": cfg.name, "tokens": n, "ms": round(dt * 1e3, 3), "tok_s": round(n / dt, 1),
            "integer_products": int8, "products": products}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill measurement")
    ap.add_argument("--reps", type=int, default=5, help="repetitions of the timed decode run (median)")
    ap.add_argument("--no-reports", action="store_true",
                    help="skip the reported decode workloads (F16 1B at ctx 2048, Q8_0 1B at ctx 8192, "
                         "Q8_0 1B with RoPE frequency factors)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only run the prefill measurement (512 ids, Qwen2-style F16 1B) and print it as JSON")
    ap.add_argument("--no-products", action="store_true",
                    help="skip timing the prompt passes' products one by one")
    ap.add_argument("--prefill-llamacpp", action="store_true",
                    help="only run the 2048-id prompt pass of the Q8_0 1B model with llama.cpp's rounding points "
                         "(integer matrix-core products) and print it as JSON")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run 5 device-to-device copies of this many bytes (the reference kernel that scales "
                         "the HBM counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the decode path is not sharded across GPUs "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import llama_family_decode_amd as llm
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_bytes:
        src = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"# copied {args.copy_bytes} bytes 5 times", file=sys.stderr)
        return
    if args.prefill_llamacpp:
        print(json.dumps({"prefill_q8_0_2048_llamacpp": measure_prefill_q8_llamacpp(llm, synth, np, torch,
                                                                                     products=not args.no_products)}))
        return
    if args.prefill_only:
        print(json.dumps({"prefill": measure_prefill(llm, synth, np, torch, products=not args.no_products)}))
        return
    cfg = synth.C4  # 1B shape, Q8_0 matrices, tied F32 embedding
    ctx_len = 2048
    t_load = time.perf_counter()
    ts = synth.make_tensor_set(cfg)
    model = llm.Model(cfg, ts)
    del ts
    prompt = synth.prompt(cfg, ctx_len)
    nxt = model.prefill(prompt)
    torch.cuda.synchronize()
    print(f"# loaded + prefilled {ctx_len} in {time.perf_counter() - t_load:.1f}s", file=sys.stderr, flush=True)
    # the workload's own prompt pass (Q8_0 products on the matrix cores), median of 3
    q8_times = []
    for _ in range(3):
        model.reset()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        nxt = model.prefill(prompt)
        torch.cuda.synchronize()
        q8_times.append(time.perf_counter() - t0)
    q8_prefill = float(np.median(q8_times))
    print(f"# prefill {ctx_len} (Q8_0): {q8_prefill * 1e3:.2f} ms, {ctx_len / q8_prefill:.0f} tok/s", file=sys.stderr,
          flush=True)
    # each of its layer products alone (the batch buffers only; the cache is untouched)
    q8_products = None
    if not args.no_products:
        q8_products = product_fractions(llm, model, cfg, ctx_len, F16_MFMA_PEAK_TFLOPS)
        print("# prefill products at 2048 rows: " + ", ".join(f"{k} {v['us']} us ({v['frac']:.3f} of the f16 peak)"
                                                               for k, v in q8_products.items()), file=sys.stderr,
              flush=True)

    # warmup (then rewind to the prefilled length)
    if args.warmup > 0:
        model.generate(nxt, args.warmup)
        model.rewind(ctx_len)
    times = []
    toks = None
    for r in range(max(1, args.reps)):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        out = model.generate(nxt, args.steps)
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
        model.rewind(ctx_len)
        if toks is None:
            toks = out
        else:
            assert np.array_equal(toks, out), "greedy decode is not deterministic"
    dt = float(np.median(times))
    tok_s = args.steps / dt
    mid_pos = ctx_len + args.steps // 2
    step_bytes = algorithmic_step_bytes(cfg, mid_pos)
    print(f"# decode {tok_s:.1f} tok/s ({1e3 * dt / args.steps:.3f} ms/token), step bytes {step_bytes / 1e6:.1f} MB "
          f"-> {step_bytes * tok_s / 1e9:.0f} GB/s", file=sys.stderr, flush=True)

    # ABI-level decode: one llm_decode call per token, each returning the next
    # token to the host (a 4-byte copy and a stream synchronisation), logits
    # left on the device
    abi_steps = min(64, args.steps)
    t = nxt
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(abi_steps):
        t = model.decode(int(t), ctx_len + i, want_next=True, copy_logits=False)
    abi_dt = time.perf_counter() - t0
    model.rewind(ctx_len)
    print(f"# llm_decode per token (host round trip each): {abi_steps / abi_dt:.1f} tok/s", file=sys.stderr,
          flush=True)

    # the dominant (only) decode kernel, timed with HIP events on its stream
    kind = llm.llm_op_step_kind(model.ctx)
    ms_step = model.time_stage(llm.STAGE_STEP, 0, mid_pos, 50)
    achieved = step_bytes / (ms_step * 1e-3) / 1e9
    kernel = {2: "k_step (persistent decode step compiled for this shape: whole forward pass of one token)",
              1: "k_step (persistent decode step: whole forward pass of one token)",
              0: "launch graph of the decode step"}[kind]
    print(f"# step kernel {ms_step * 1e3:.1f} us per launch -> {achieved:.0f} GB/s", file=sys.stderr, flush=True)
    model.rewind(ctx_len)
    model.close()
    del model
    torch.cuda.empty_cache()

    # device-to-device copy of 1 GiB (reads and writes it): the chip's measured
    # streaming rate beside the 8 TB/s specification
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(10):
        dst.copy_(src)
    ev1.record()
    ev1.synchronize()
    copy_gbs = 2 * src.numel() * 4 * 10 / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()

    prefill = None
    if not args.no_prefill:
        prefill = measure_prefill(llm, synth, np, torch, products=not args.no_products)

    reports = None
    if not args.no_reports:
        reports = [measure_decode_report(llm, synth, np, torch, synth.C3, 2048),
                   measure_decode_report(llm, synth, np, torch, synth.C4_LONG, 8192),
                   measure_decode_report(llm, synth, np, torch,
                                         synth.C4.with_(name="llama-1b-q8_0-rope-freqs", rope_freq_factors=True), 2048),
                   measure_decode_report(llm, synth, np, torch,
                                         synth.C4_LONG.with_(name="llama-1b-q8_0-window1024-sinks4", attn_window=1024,
                                                             attn_sinks=4), 8192),
                   measure_decode_report(llm, synth, np, torch,
                                         synth.C4.with_(name="llama-1b-q8_0-llamacpp-numerics", numerics=1), 2048),
                   measure_decode_report(llm, synth, np, torch,
                                         synth.C4.with_(name="llama-1b-q8_0-yarn16", yarn_factor=16.0,
                                                        yarn_orig_ctx=16384), 2048)]
        reports.append({"prefill_q8_0_2048_llamacpp": measure_prefill_q8_llamacpp(llm, synth, np, torch)})

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, ctx_len)
        print(f"# cpu oracle {cpu['value']} tok/s on {cpu['cores']} threads ({cpu['one_thread_tok_s']} on 1), "
              f"prefill {cpu['prefill_tok_s']} tok/s; {cpu['cpu_model']}", file=sys.stderr, flush=True)

    line = {
        "metric": "decode tok/s (1B-shape Q8_0, tied F32 embedding, KV cache prefilled to 2048)",
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * dt / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q8_0 weights, fp32 arithmetic, f16 KV",
        "data": "synthetic: seeded random weights and prompt ids",
        "config": {"workload": "llama-1b-q8_0 decode at positions 2048..2175 after a 2048-id prefill",
                   "dim": cfg.dim, "layers": cfg.n_layers, "heads": cfg.n_heads, "kv_heads": cfg.n_kv_heads,
                   "ffn": cfg.ffn, "vocab": cfg.vocab, "ctx": ctx_len, "parallelism": "single GPU"},
        "step_roofline": {"bytes_per_token": step_bytes, "achieved_GBs": round(step_bytes * tok_s / 1e9, 1),
                          "peak_GBs": HBM_PEAK_GBS, "frac": round(step_bytes * tok_s / 1e9 / HBM_PEAK_GBS, 4)},
        "roofline": {"kernel": kernel, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": read_traffic(),
                     "bytes_per_launch": step_bytes, "ms_per_launch": round(ms_step, 5), "position": mid_pos},
        "abi_decode": {"tok_s": round(abi_steps / abi_dt, 1), "steps": abi_steps,
                       "note": "llm_decode once per token, next token returned to the host each call"},
        "device_copy_GBs": round(copy_gbs, 1),
        "prefill": prefill,
        "prefill_q8_0_2048": {"config": cfg.name, "tokens": ctx_len, "ms": round(q8_prefill * 1e3, 3),
                              "tok_s": round(ctx_len / q8_prefill, 1), "products": q8_products},
        "decode_reports": reports,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
