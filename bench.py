#!/usr/bin/env python3
"""Benchmark of the MI355X forward pass of a Qwen3 dense decoder over Q8_0
weights.

Workload (one "step"): the Qwen3-0.6B shape with synthetic Q8_0 weights
(N(0, 0.02) quantised; f32 norm weights 1 + N(0, 0.1)), one prefill of a
512-token uniform-random prompt, then 256 greedy decode steps fed their own
argmax on the device, f32 KV cache, batch 1.  Timed with HIP events on the
stream the library launches on; inputs are resident in HBM before timing.

Prints ONE JSON line: decode tokens/s (`value`), the whole-step decode HBM
rate, prefill tokens/s, the roofline of the dominant decode kernel (its
algorithmic bytes per launch over its event-timed average duration) and the
CPU oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
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


def cpu_baseline(shape, weights, prompt, decode_steps: int) -> dict:
    """The CPU oracle on a bounded sample of the same workload."""
    from threadpoolctl import threadpool_info

    from oracle import model as om

    ref = om.Model(shape, weights)
    cache = ref.new_cache(len(prompt) + decode_steps + 1)
    t0 = time.perf_counter()
    logits = ref.forward(prompt, cache)[0]
    t1 = time.perf_counter()
    tok = int(logits.argmax())
    for _ in range(decode_steps):
        tok = int(ref.forward([tok], cache)[0].argmax())
    t2 = time.perf_counter()
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {
        "value": decode_steps / (t2 - t1),
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"prefill of the {len(prompt)}-token prompt then {decode_steps} greedy decode steps",
        "prefill_tokens_per_s": len(prompt) / (t1 - t0),
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="0.6b-decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-decode-steps", type=int, default=8)
    ap.add_argument("--kernel-reps", type=int, default=50)
    args = ap.parse_args()
    if args.gpus != 1:
        print(
            f"bench.py runs on exactly one GPU (asked for {args.gpus}); the path is single-GPU by design",
            file=sys.stderr,
        )
        return 2

    import torch

    from quantized_q8_dequant_amd import Qwen3Config, Qwen3Model
    from synthetic import WORKLOADS, gen_prompt, gen_weights

    wl = WORKLOADS[args.workload]
    shape = wl.shape
    weights = gen_weights(shape, wl.weight_seed)
    prompt = gen_prompt(shape.vocab_size, wl.prompt_len, wl.prompt_seed)
    model = Qwen3Model(Qwen3Config.from_shape(shape), weights, [wl.kv_capacity])
    torch.cuda.synchronize()

    def one_step():
        model.reset()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        model.prefill(prompt)
        e[1].record()
        for _ in range(wl.decode_steps):
            model.decode_step()
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
    dom = max(kernels, key=lambda k: kernels[k]["us_per_launch"] * kernels[k]["launches_per_token"])
    dk = kernels[dom]
    achieved = dk["GBps"]
    roofline = {
        "kernel": dom,
        "bound": "hbm",
        "achieved": achieved,
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": None,
    }

    cpu = None
    if not args.no_cpu_baseline:
        model.close()
        del model
        torch.cuda.empty_cache()
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
        "prefill_ms": round(prefill_ms, 3),
        "prefill_tokens_per_s": round(prefill_tps, 1),
        "kernels_at_mean_ctx": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
