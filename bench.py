#!/usr/bin/env python3
"""Benchmark of the MI355X forward pass of a Qwen3 dense decoder over Q8_0
weights.

Default workload (one "step"): the Qwen3-0.6B shape with synthetic Q8_0
weights (N(0, 0.02) quantised; f32 norm weights 1 + N(0, 0.1)), one prefill
of a 512-token uniform-random prompt, then 256 greedy decode steps fed their
own argmax on the device, f32 KV cache, batch 1.  Timed with HIP events on
the stream the library launches on; inputs are resident in HBM before timing.

Prints ONE JSON line: decode tokens/s (`value`), the whole-step decode HBM
rate, prefill tokens/s, the roofline of the dominant decode kernel (its
algorithmic bytes per launch over its event-timed average duration), the
prefill-dominated variant (4096 tokens in one call, same weights) and the
CPU oracle timed on a bounded sample of the same workload.

Other workloads (`--workload`): `8b-longctx` (Qwen3-8B shape, bf16 KV --
`--kv q8_0` for the Q8_0 cache -- decode at KV lengths 2048/16384/32768)
and `0.6b-bf16-batch64` (bf16 weights, 64 ragged sequences, batched
decode)."""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_step_traffic.json")
# the one-launch decode kernel and the headers it includes
PERSISTENT_SRC = [os.path.join(ROOT, "quantized_q8_dequant_amd", "csrc", f)
                  for f in ("k_decode_persistent.hip", "persist.h", "qdevice.h")]
INT8_PEAK_OPS = 5.0e15  # dense int8 MFMA
KIND_NAMES = ["qkv_gemv", "attention", "o_proj_gemv", "gate_up_swiglu_gemv", "down_gemv", "lm_head_argmax_gemv"]


def q8_bytes(n_weights: int) -> float:
    return n_weights * 34 / 32


def kernel_bytes(shape, kind: int, ctx: int) -> float:
    """Algorithmic HBM bytes of one launch of a decode kernel at KV length ctx."""
    H, F, V = shape.hidden_size, shape.intermediate_size, shape.vocab_size
    qw, kvw = shape.q_width, shape.kv_width
    nqkv = qw + 2 * kvw
    if kind == 0:
        return q8_bytes(nqkv * H) + 4 * (2 * H + nqkv)
    if kind == 1:
        kv_elem = 4 if shape.kv_type == "f32" else 2
        return 2 * kvw * (ctx + 1) * kv_elem + 4 * (nqkv + qw)
    if kind == 2:
        return q8_bytes(H * qw) + 4 * (qw + 2 * H)
    if kind == 3:
        return q8_bytes(2 * F * H) + 4 * (2 * H + F)
    if kind == 4:
        return q8_bytes(H * F) + 4 * (F + 2 * H)
    return q8_bytes(V * H) + 4 * (2 * H)


def decode_token_bytes(shape, ctx: int) -> float:
    """Algorithmic HBM bytes of one decode step whose new token sits at ctx."""
    per_layer = sum(kernel_bytes(shape, k, ctx) for k in range(5))
    return shape.num_layers * per_layer + kernel_bytes(shape, 5, ctx) + 4 * shape.vocab_size


def source_sha(paths) -> str:
    """SHA-256 over the concatenated bytes of `paths`, in order."""
    import hashlib

    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter runs
    (FETCH_SIZE + WRITE_SIZE, scaled by a copy of known size), or None if
    there are none or the kernel source changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    k = t.get("kernels", {}).get(kernel)
    if not k or k.get("source_sha256") != source_sha(PERSISTENT_SRC):
        return None
    return k.get("bytes_per_launch")


def prefill_int8_ops(shape, T: int) -> int:
    """int8 MACs x 2 of the projection GEMMs of a T-token prefill (the
    lm_head runs on the last row only and is left out)."""
    H, F = shape.hidden_size, shape.intermediate_size
    per_layer = (shape.q_width + 2 * shape.kv_width) * H + H * shape.q_width + 2 * F * H + H * F
    return 2 * T * per_layer * shape.num_layers


def weight_bytes(shape) -> float:
    """Bytes of all projection and embedding weights (read once per decode step)."""
    H, F, V = shape.hidden_size, shape.intermediate_size, shape.vocab_size
    per_layer = (shape.q_width + 2 * shape.kv_width) * H + H * shape.q_width + 2 * F * H + H * F
    n = per_layer * shape.num_layers + V * H
    return q8_bytes(n) if shape.weight_type == "q8_0" else 2.0 * n


def kv_bytes_per_position(shape) -> float:
    per = {"f32": 4.0, "bf16": 2.0, "q8_0": 34.0 / 32.0}[shape.kv_type]  # q8_0: codes + f16 scale per 32
    return shape.num_layers * 2 * shape.kv_width * per


def timed(fn, reps: int) -> float:
    """Median milliseconds of fn() over reps runs, HIP events on the current stream."""
    import torch

    out = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b))
    return sorted(out)[len(out) // 2]


def bench_8b(args) -> int:
    """Qwen3-8B shape, Q8_0, bf16 KV: prefill 2048, decode at 2048/16384/32768."""
    import torch

    from quantized_q8_dequant_amd import Qwen3Config, Qwen3Model
    from synthetic import WORKLOADS, gen_prompt, gen_weights

    wl = WORKLOADS["8b-longctx"]
    shape = wl.shape if args.kv is None else wl.shape.with_(kv_type=args.kv)
    weights = gen_weights(shape, wl.weight_seed)
    model = Qwen3Model(Qwen3Config.from_shape(shape), weights, [wl.kv_capacity], max_batch_tokens=2048)
    torch.cuda.synchronize()
    cpu = None
    if not args.no_cpu_baseline:
        p0 = gen_prompt(shape.vocab_size, wl.prompt_len, wl.prompt_seed)[:16]
        cpu = cpu_baseline(
            shape, weights, p0, 2,
            "prefill of the first 16 prompt tokens then 2 greedy decode steps (KV length 16-18; at 8B the "
            "weights, not the KV length, set the oracle's time per token)",
        )
    del weights
    steps = max(args.steps, 1) * 4
    out = {}
    t0 = time.perf_counter()
    for L in wl.decode_contexts:
        prompt = gen_prompt(shape.vocab_size, L, wl.prompt_seed if L == wl.prompt_len else wl.prompt_seed + L)
        model.reset()
        model.prefill(prompt[:1024])  # warm-up
        model.reset()
        pre_ms = timed(lambda: (model.reset(), model.prefill(prompt, logits=False)), 1)
        for _ in range(args.warmup):
            model.decode_step()
        ctx0 = model.kv_len()
        n_steps = max(1, min(steps, wl.kv_capacity - ctx0))
        ms = timed(lambda: [model.decode_step() for _ in range(n_steps)], 1) / n_steps
        nbytes = weight_bytes(shape) + kv_bytes_per_position(shape) * (ctx0 + n_steps / 2)
        out[str(L)] = {
            "prefill_ms": round(pre_ms, 2),
            "prefill_tokens_per_s": round(L / (pre_ms / 1000.0), 1),
            "prefill_int8_frac_of_whole_prefill": round(prefill_int8_ops(shape, L) / (pre_ms / 1000.0) / INT8_PEAK_OPS, 4),
            "decode_steps_timed": n_steps,
            "decode_ms_per_token": round(ms, 4),
            "decode_tokens_per_s": round(1000.0 / ms, 2),
            "decode_hbm_GBps": round(nbytes / (ms / 1000.0) / 1e9, 1),
            "decode_hbm_frac": round(nbytes / (ms / 1000.0) / 1e9 / HBM_PEAK_GBPS, 4),
        }
    t1 = time.perf_counter()
    line = {
        "metric": "decode tokens/s and HBM GB/s at KV lengths 2048/16384/32768; prefill tokens/s, Qwen3-8B Q8_0",
        "value": out[str(wl.decode_contexts[0])]["decode_tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round((t1 - t0) * 1000.0, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": f"Qwen3-8B shape, Q8_0 weights, {shape.kv_type} KV cache: a prompt of L random tokens in "
            "2048-row chunks, then greedy decode steps at KV length L, L = 2048, 16384, 32768, batch 1",
            "weights": "q8_0",
            "kv_cache": shape.kv_type,
            "parallelism": "single GPU",
        },
        "contexts": out,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_batch64(args) -> int:
    """bf16 0.6B: 64 sequences with lengths 1024..16384, lockstep greedy steps."""
    import numpy as np
    import torch

    from quantized_q8_dequant_amd import Qwen3Config, Qwen3Model
    from synthetic import WORKLOADS, gen_lengths, gen_prompts, gen_weights

    wl = WORKLOADS["0.6b-bf16-batch64"]
    shape = wl.shape
    lengths = gen_lengths(wl.n_seqs, wl.min_len, wl.max_len, wl.length_seed)
    prompts = gen_prompts(shape.vocab_size, lengths, wl.prompt_seed)
    weights = gen_weights(shape, wl.weight_seed)
    caps = [int(n) + wl.decode_steps for n in lengths]
    model = Qwen3Model(Qwen3Config.from_shape(shape), weights, caps)
    torch.cuda.synchronize()
    cpu = None
    if not args.no_cpu_baseline:
        s0 = int(np.argmin(lengths))
        cpu = cpu_baseline(
            shape, weights, prompts[s0][:32], 4,
            "one sequence: prefill of 32 prompt tokens then 4 greedy decode steps; the oracle steps sequences "
            "one at a time, so its tokens/s is that of a batched step of any size (at this short KV length)",
        )
    del weights
    n = wl.n_seqs
    t0 = time.perf_counter()
    first = [int(model.prefill(p, seq=s, logits=False)[1].item()) for s, p in enumerate(prompts)]
    fill_s = time.perf_counter() - t0
    toks = torch.tensor(first, dtype=torch.int32, device="cuda:0")
    am = torch.empty(n, dtype=torch.int32, device="cuda:0")
    seqs = list(range(n))
    steps = min(wl.decode_steps, max(1, args.steps) * 32)
    warm = min(args.warmup * 4, wl.decode_steps - steps)

    def step():
        nonlocal toks
        model.decode_batch(seqs, toks, None, am)
        toks = am.clone()

    for _ in range(warm):
        step()
    ctx0 = np.asarray(lengths, np.float64) + warm
    ms = timed(lambda: [step() for _ in range(steps)], 1) / steps
    kv = kv_bytes_per_position(shape) * float(np.sum(ctx0 + steps / 2.0))
    nbytes = weight_bytes(shape) + kv
    line = {
        "metric": "batched decode tokens/s (64 ragged sequences) + achieved HBM GB/s, Qwen3-0.6B bf16",
        "value": round(n / (ms / 1000.0), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {
            "workload": "Qwen3-0.6B shape with bf16 weights and bf16 KV: 64 independent sequences, KV lengths "
            "uniform in 1024..16384 (each filled by prefill), lockstep greedy batched decode steps",
            "weights": "bf16",
            "kv_cache": "bf16",
            "parallelism": "single GPU",
        },
        "hbm_GBps": round(nbytes / (ms / 1000.0) / 1e9, 1),
        "hbm_frac": round(nbytes / (ms / 1000.0) / 1e9 / HBM_PEAK_GBPS, 4),
        "bytes_per_step": int(nbytes),
        "cache_fill_s": round(fill_s, 2),
        "mean_kv_length": float(np.mean(ctx0)),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


VERIFY_TOKENS = 16


def event_ms(fn, warmup: int, reps: int) -> float:
    """Median event-timed duration of fn() on the current stream, in ms."""
    import torch

    for _ in range(warmup):
        fn()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    return sorted(times)[len(times) // 2]


def bench_verify(model, prompt, shape, decode_ms_per_token: float, args) -> dict:
    """The speculative seams: an all-logits verify of VERIFY_TOKENS drafted
    tokens after the prompt plus the rewind that drops them, set against as
    many sequential decode steps; and the whole prompt with every row's
    logits, set against the ordinary last-row prefill."""
    from synthetic import gen_prompt

    draft = gen_prompt(shape.vocab_size, VERIFY_TOKENS, 80)
    P = len(prompt)
    model.reset()
    model.prefill(prompt, logits=False)

    def verify():
        model.prefill_all_logits(draft)
        model.truncate(P)

    v_ms = event_ms(verify, args.warmup, max(args.steps, 5))

    def all_rows():
        model.reset()
        model.prefill_all_logits(prompt)

    a_ms = event_ms(all_rows, args.warmup, args.steps)
    return {
        "verify_tokens": VERIFY_TOKENS,
        "verify_ms": round(v_ms, 3),
        "sequential_decode_ms": round(VERIFY_TOKENS * decode_ms_per_token, 3),
        "verify_speedup_vs_sequential_decode": round(VERIFY_TOKENS * decode_ms_per_token / v_ms, 2),
        "all_logits_prompt_tokens": P,
        "all_logits_prefill_ms": round(a_ms, 3),
        "all_logits_tokens_per_s": round(P / (a_ms / 1000.0), 1),
    }


BATCH_SIZES = (16, 64)


def bench_batched(shape, weights, prompt, args) -> dict:
    """Lockstep batched greedy decode (one token for each of n streams per
    step) at KV length len(prompt), every stream prefilled with the prompt."""
    import torch

    from quantized_q8_dequant_amd import Qwen3Config, Qwen3Model

    nmax = max(BATCH_SIZES)
    P = len(prompt)
    steps = 8
    model = Qwen3Model(Qwen3Config.from_shape(shape), weights, [P + steps * (args.warmup + args.steps + 1) + 1] * nmax)
    for s in range(nmax):
        model.prefill(prompt, seq=s, logits=False)
    out = {}
    for n in BATCH_SIZES:
        seqs = list(range(n))
        am = torch.zeros(n, dtype=torch.int32, device="cuda:0")

        def run():
            for _ in range(steps):
                model.decode_batch(seqs, am, None, am)

        ms = event_ms(run, args.warmup, args.steps) / steps
        for s in seqs:
            model.truncate(P, seq=s)
        out[str(n)] = {
            "ms_per_step": round(ms, 4),
            "tokens_per_s": round(n * 1000.0 / ms, 1),
            "weight_GBps": round(weight_bytes(shape) / (ms / 1000.0) / 1e9, 1),
        }
    model.close()
    # the same 64-stream step over a q8_0 KV cache (a quarter of the f32
    # cache's bytes), the per-step KV reads being the largest part at 64
    qshape = shape.with_(kv_type="q8_0")
    model = Qwen3Model(Qwen3Config.from_shape(qshape), weights, [P + steps * (args.warmup + args.steps + 1) + 1] * nmax)
    for s in range(nmax):
        model.prefill(prompt, seq=s, logits=False)
    seqs = list(range(nmax))
    am = torch.zeros(nmax, dtype=torch.int32, device="cuda:0")

    def runq():
        for _ in range(steps):
            model.decode_batch(seqs, am, None, am)

    ms = event_ms(runq, args.warmup, args.steps) / steps
    out[f"{nmax}_q8_0_kv"] = {"ms_per_step": round(ms, 4), "tokens_per_s": round(nmax * 1000.0 / ms, 1)}
    model.close()
    return out


def bench_sampling(V: int, args) -> dict:
    """The device sampling pipeline on rows of V logits: a Qwen3-style
    setting (temperature 0.7, top-k 20, top-p 0.95, repetition penalty over
    64 tokens) and the exact nucleus (top-k 0, top-p 0.9: on these N(0, 4^2)
    logits its window grows past 256 candidates), for 1 and 64 rows; and the
    exact nucleus on flat N(0, 1) rows, whose window grows to the whole
    vocabulary (the wide window sorted in scratch), for 1 and 8 rows."""
    import torch

    from quantized_q8_dequant_amd import sample

    g = torch.Generator(device="cuda:0").manual_seed(11)
    out = {}
    for rows in (1, 64):
        base = torch.randn((rows, V), device="cuda:0", generator=g) * 4.0
        uni = torch.rand(rows, device="cuda:0", generator=g)
        hist = torch.randint(0, V, (rows, 64), device="cuda:0", dtype=torch.int32, generator=g)
        hlen = torch.full((rows,), 64, device="cuda:0", dtype=torch.int32)
        for name, kw in (
            ("top_k20_top_p0.95", dict(temperature=0.7, top_k=20, top_p=0.95, repeat_penalty=1.1)),
            ("nucleus_top_p0.9", dict(temperature=1.0, top_k=0, top_p=0.9)),
        ):
            lg = base.clone()

            def run():
                sample(lg, uni, history=hist, history_len=hlen, **kw)

            out[f"{name}_rows{rows}_us"] = round(event_ms(run, args.warmup, max(args.steps, 5)) * 1000.0, 1)
    for rows in (1, 8):
        base = torch.randn((rows, V), device="cuda:0", generator=g)
        uni = torch.rand(rows, device="cuda:0", generator=g)
        lg = base.clone()

        def run_wide():
            sample(lg, uni, temperature=1.0, top_k=0, top_p=0.9)

        out[f"nucleus_whole_vocab_top_p0.9_rows{rows}_us"] = round(
            event_ms(run_wide, args.warmup, max(args.steps, 5)) * 1000.0, 1
        )
    return out


def bench_prefill_gemms(shape, args) -> dict:
    """Each projection GEMM of a 4096-token prefill timed alone: the op-level
    Q8_0 linear (qwen3_q8_0_linear: the activation rows quantised, then the
    MFMA GEMM the prefill runs) on 4096 random rows against a random Q8_0
    matrix of the layer's shape, event-timed (median of repeats).  The int8
    ops are 2 M N K; the rate includes the row quantisation, a few percent."""
    import torch

    from quantized_q8_dequant_amd import encode_q8_0, q8_0_linear, repack_q8_0

    H, F = shape.hidden_size, shape.intermediate_size
    M = 4096
    g = torch.Generator(device="cuda:0").manual_seed(13)
    out = {}
    for name, N, K in (
        ("qkv", shape.q_width + 2 * shape.kv_width, H),
        ("o_proj", H, shape.q_width),
        ("gate_up", 2 * F, H),
        ("down", H, F),
    ):
        w = torch.randn((N, K), device="cuda:0", generator=g) * 0.02
        qs, sc = repack_q8_0(encode_q8_0(w), N, K)
        x = torch.randn((M, K), device="cuda:0", generator=g)
        del w
        ms = event_ms(lambda: q8_0_linear(x, qs, sc), max(args.warmup, 1), max(args.steps, 5))
        ops = 2.0 * M * N * K
        out[name] = {
            "M": M, "N": N, "K": K,
            "us": round(ms * 1000.0, 1),
            "int8_TOPS": round(ops / (ms / 1000.0) / 1e12, 1),
            "frac_of_int8_peak": round(ops / (ms / 1000.0) / INT8_PEAK_OPS, 4),
        }
        del qs, sc, x
    torch.cuda.empty_cache()
    return out


def measure_peaks(args) -> dict:
    """Achievable peaks on this GPU, measured with the library's own probes:
    a streaming copy of 1 GiB (read plus write bytes over its event-timed
    duration), a streaming read of 1 GiB and a loop of int8 MFMAs (2048
    workgroups, operands in registers)."""
    import torch

    from quantized_q8_dequant_amd import peak_copy, peak_mfma_i8, peak_read, peak_read_partials

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    src.fill_(1)
    dst = torch.empty_like(src)
    copy_ms = event_ms(lambda: peak_copy(src, dst), max(args.warmup, 1), 10)
    parts = torch.zeros(peak_read_partials(), dtype=torch.int32, device="cuda:0")
    read_ms = event_ms(lambda: peak_read(src, parts), max(args.warmup, 1), 10)
    del src, dst, parts
    torch.cuda.empty_cache()
    wgs, iters = 2048, 4000
    out = torch.empty(256 * wgs, dtype=torch.int32, device="cuda:0")
    ops = [0.0]

    def run():
        ops[0] = peak_mfma_i8(out, wgs, iters)

    mfma_ms = event_ms(run, 1, 5)
    return {
        "copy_GBps": round(2 * n / (copy_ms / 1000.0) / 1e9, 1),
        "copy_frac_of_vendor_peak": round(2 * n / (copy_ms / 1000.0) / 1e9 / HBM_PEAK_GBPS, 4),
        "read_GBps": round(n / (read_ms / 1000.0) / 1e9, 1),
        "read_frac_of_vendor_peak": round(n / (read_ms / 1000.0) / 1e9 / HBM_PEAK_GBPS, 4),
        "mfma_int8_TOPS": round(ops[0] / (mfma_ms / 1000.0) / 1e12, 1),
        "mfma_int8_frac_of_vendor_peak": round(ops[0] / (mfma_ms / 1000.0) / INT8_PEAK_OPS, 4),
    }


def host_info() -> dict:
    """The host the CPU baseline runs on: CPU model, logical CPUs, and the
    BLAS library numpy calls (its threads are the cores the oracle uses)."""
    from threadpoolctl import threadpool_info

    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = [
        {
            "api": i.get("internal_api"),
            "version": i.get("version"),
            "threads": i.get("num_threads"),
            "library": os.path.basename(i.get("filepath", "")),
        }
        for i in threadpool_info()
        if i.get("user_api") == "blas"
    ]
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "blas": blas}


def cpu_baseline(shape, weights, prompt, decode_steps: int, sample: str | None = None) -> dict:
    """The CPU oracle (as it stands, not tuned) on a bounded sample of the
    same workload: a prefill of `prompt`, then `decode_steps` greedy steps."""
    from oracle import model as om

    ref = om.Model(shape, weights, threads=min(16, os.cpu_count() or 1))
    cache = ref.new_cache(len(prompt) + decode_steps + 1)
    t0 = time.perf_counter()
    logits = ref.forward(prompt, cache)[0]
    t1 = time.perf_counter()
    tok = int(logits.argmax())
    for _ in range(decode_steps):
        tok = int(ref.forward([tok], cache)[0].argmax())
    t2 = time.perf_counter()
    info = host_info()
    threads = max([b["threads"] or 1 for b in info["blas"]] or [1])
    return {
        "value": decode_steps / (t2 - t1),
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": sample or f"prefill of the {len(prompt)}-token prompt then {decode_steps} greedy decode steps",
        "prefill_tokens_per_s": len(prompt) / (t1 - t0),
        "host": info,
    }


def counters_decode(args) -> int:
    """The default workload's decode steps alone, for hardware-counter runs.

    The prompt enters the KV cache through one-token decode steps (the
    prompt's own tokens fed in order), so no prefill kernel is launched; then
    the workload's greedy decode steps (KV lengths prompt_len ..
    prompt_len + steps - 1) as one qwen3_decode_greedy call, the one launch
    the benchmark times; then one 1 GiB device-to-device copy whose bytes are
    known (the counters' scale).
    A line is printed after each part."""
    import torch

    from quantized_q8_dequant_amd import Qwen3Config, Qwen3Model
    from synthetic import WORKLOADS, gen_prompt, gen_weights

    wl = WORKLOADS["0.6b-decode"]
    shape = wl.shape
    model = Qwen3Model(Qwen3Config.from_shape(shape), gen_weights(shape, wl.weight_seed), [wl.kv_capacity])
    if model.decode_launches() != 1:
        print("the decode step is not one launch on this build", file=sys.stderr)
        return 1
    prompt = torch.tensor(gen_prompt(shape.vocab_size, wl.prompt_len, wl.prompt_seed), dtype=torch.int32,
                          device="cuda:0")
    for i in range(wl.prompt_len):
        model.decode_step(token=prompt[i : i + 1], logits=False)
    torch.cuda.synchronize()
    model.step_status()
    print(f"cache filled by {wl.prompt_len} decode steps", flush=True)
    model.decode_greedy(wl.decode_steps)  # from the token the last fill step chose
    torch.cuda.synchronize()
    model.step_status()
    print(f"{wl.decode_steps} greedy decode steps in one launch (KV length {wl.prompt_len}.."
          f"{wl.prompt_len + wl.decode_steps - 1})", flush=True)
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print("1 GiB device-to-device copy", flush=True)
    model.close()
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="0.6b-decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-decode-steps", type=int, default=8)
    ap.add_argument("--kernel-reps", type=int, default=50)
    ap.add_argument(
        "--kv",
        choices=["f32", "bf16", "q8_0"],
        default=None,
        help="KV cache type of the 8b-longctx workload (default: its bf16)",
    )
    ap.add_argument(
        "--counters-decode",
        action="store_true",
        help="counter runs: only the default workload's decode steps (the cache filled by decode steps, no "
        "prefill kernel), then a 1 GiB device-to-device copy of known size",
    )
    ap.add_argument(
        "--pmc-calibrate",
        action="store_true",
        help="finish with a 1 GiB device-to-device copy (the known-size kernel hardware counters are scaled by)",
    )
    args = ap.parse_args()
    if args.gpus != 1:
        print(
            f"bench.py runs on exactly one GPU (asked for {args.gpus}); the path is single-GPU by design",
            file=sys.stderr,
        )
        return 2

    if args.counters_decode:
        return counters_decode(args)

    import torch

    from quantized_q8_dequant_amd import Qwen3Config, Qwen3Model
    from synthetic import WORKLOADS, gen_prompt, gen_weights

    if args.workload == "8b-longctx":
        return bench_8b(args)
    if args.workload == "0.6b-bf16-batch64":
        return bench_batch64(args)
    wl = WORKLOADS[args.workload]
    shape = wl.shape
    weights = gen_weights(shape, wl.weight_seed)
    prompt = gen_prompt(shape.vocab_size, wl.prompt_len, wl.prompt_seed)
    model = Qwen3Model(Qwen3Config.from_shape(shape), weights, [wl.kv_capacity])
    torch.cuda.synchronize()

    # the greedy decode steps are one qwen3_decode_greedy call (with the
    # one-launch step: one launch, the token handed between steps on the
    # device); the same steps as single qwen3_decode_step calls are timed
    # after the timed region
    def one_step():
        model.reset()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        model.prefill(prompt)
        e[1].record()
        model.decode_greedy(wl.decode_steps)
        e[2].record()
        return e

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs = [one_step() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prefill_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    decode_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    ms_per_step = (t1 - t0) * 1000.0 / args.steps
    decode_tps = wl.decode_steps / (decode_ms / 1000.0)
    prefill_tps = wl.prompt_len / (prefill_ms / 1000.0)
    step_bytes = sum(decode_token_bytes(shape, wl.prompt_len + i) for i in range(wl.decode_steps))
    decode_gbps = step_bytes / (decode_ms / 1000.0) / 1e9

    # the same decode steps as single calls (one launch each)
    single = []
    for _ in range(2):
        model.reset()
        model.prefill(prompt)
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record()
        for _ in range(wl.decode_steps):
            model.decode_step()
        b_.record()
        torch.cuda.synchronize()
        single.append(a_.elapsed_time(b_))
    model.step_status()
    single_ms = single[-1]

    # per-kernel durations at the mean decode length (replayed in the step's
    # launch configuration, timed with events on the launch stream)
    model.reset()
    model.prefill(prompt)
    mid = wl.decode_steps // 2
    for _ in range(mid):
        model.decode_step()
    torch.cuda.synchronize()
    ctx = wl.prompt_len + mid
    kernels = {}
    for kind in range(6):
        layer = shape.num_layers // 2
        model.replay_kernel(kind, layer, 3)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        model.replay_kernel(kind, layer, args.kernel_reps)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1000.0 / args.kernel_reps
        launches = 1 if kind == 5 else shape.num_layers
        nbytes = kernel_bytes(shape, kind, ctx)
        kernels[KIND_NAMES[kind]] = {
            "us_per_launch": round(us, 3),
            "launches_per_token": launches,
            "bytes_per_launch": int(nbytes),
            "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
        }
    verify = None
    if args.workload == "0.6b-decode":
        verify = bench_verify(model, prompt, shape, single_ms / wl.decode_steps, args)
    launches = model.decode_launches()
    if launches == 1:
        # the decode steps are one kernel launch: its algorithmic bytes (every
        # step at its KV length) over its event-timed duration
        us = decode_ms * 1000.0
        dom = f"decode_step (one launch running the {wl.decode_steps} greedy steps)"
        achieved = round(step_bytes / (us * 1e-6) / 1e9, 1)
        traffic = measured_traffic("decode_step")
        kernel_info = {"us_per_launch": round(us, 1), "bytes_per_launch": int(step_bytes),
                       "steps_per_launch": wl.decode_steps, "us_per_step": round(us / wl.decode_steps, 3)}
    else:
        dom = max(kernels, key=lambda k: kernels[k]["us_per_launch"] * kernels[k]["launches_per_token"])
        achieved = kernels[dom]["GBps"]
        traffic = None
        kernel_info = kernels[dom]
    roofline = {
        "kernel": dom,
        "bound": "hbm",
        "achieved": achieved,
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": traffic,
        "launch": kernel_info,
    }

    # the prefill-dominated workload on the same weights: 4096 tokens in one call
    p4 = None
    if args.workload == "0.6b-decode":
        model.close()
        del model
        torch.cuda.empty_cache()
        wl4 = WORKLOADS["0.6b-prefill4096"]
        prompt4 = gen_prompt(shape.vocab_size, wl4.prompt_len, wl4.prompt_seed)
        m4 = Qwen3Model(Qwen3Config.from_shape(shape), weights, [wl4.kv_capacity], max_batch_tokens=wl4.prompt_len)
        times = []
        for _ in range(args.warmup + args.steps):
            m4.reset()
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record()
            m4.prefill(prompt4)
            b_.record()
            torch.cuda.synchronize()
            times.append(a_.elapsed_time(b_))
        t4 = sorted(times[args.warmup:])[len(times[args.warmup:]) // 2]
        ops = prefill_int8_ops(shape, wl4.prompt_len)
        p4 = {
            "prompt_tokens": wl4.prompt_len,
            "ms": round(t4, 3),
            "tokens_per_s": round(wl4.prompt_len / (t4 / 1000.0), 1),
            "projection_int8_ops": ops,
            "int8_mfma_frac_of_whole_prefill": round(ops / (t4 / 1000.0) / INT8_PEAK_OPS, 4),
        }
        m4.close()
        del m4
        torch.cuda.empty_cache()
        p4["per_gemm"] = bench_prefill_gemms(shape, args)
    else:
        model.close()
        del model
        torch.cuda.empty_cache()

    batched = sampling = None
    if args.workload == "0.6b-decode":
        batched = bench_batched(shape, weights, prompt, args)
        torch.cuda.empty_cache()
        sampling = bench_sampling(shape.vocab_size, args)
    peaks = measure_peaks(args)

    if args.pmc_calibrate:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(shape, weights, prompt, args.cpu_decode_steps)

    line = {
        "metric": "decode tokens/sec + achieved HBM GB/s (% peak); prefill tokens/sec, Qwen3-0.6B Q8_0",
        "value": round(decode_tps, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": f"{shape.name} Q8_0: prefill {wl.prompt_len} random tokens then "
            f"{wl.decode_steps} greedy decode steps, {shape.kv_type} KV cache, batch 1",
            "prompt_tokens": wl.prompt_len,
            "decode_steps": wl.decode_steps,
            "kv_cache": shape.kv_type,
            "weights": shape.weight_type,
            "parallelism": "single GPU",
        },
        "decode_ms": round(decode_ms, 3),
        "decode_tokens_per_s": round(decode_tps, 2),
        "decode_hbm_GBps": round(decode_gbps, 1),
        "decode_hbm_frac": round(decode_gbps / HBM_PEAK_GBPS, 4),
        "decode_frac_of_measured_read_peak": round(decode_gbps / peaks["read_GBps"], 4),
        "prefill_ms": round(prefill_ms, 3),
        "prefill_tokens_per_s": round(prefill_tps, 1),
        "decode_launches_per_token": launches,
        "decode_call": "qwen3_decode_greedy (all steps in one call)",
        "decode_single_step_calls_ms": round(single_ms, 3),
        "decode_single_step_calls_tokens_per_s": round(wl.decode_steps / (single_ms / 1000.0), 2),
        "kernels_at_mean_ctx": kernels,
        "prefill_4096_one_call": p4,
        "verify": verify,
        "batched_decode": batched,
        "sampling": sampling,
        "measured_peaks": peaks,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    rc = main()
    if rc:  # success ends the interpreter normally (a profiler writes its results during that shutdown)
        sys.exit(rc)
