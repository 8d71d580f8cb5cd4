"""Benchmark: batch-1 greedy decode of the ~2B decoder on one MI355X.

Workload: the ~2B Llama-style decoder (24 layers, d 2048, 16 query / 8 KV
heads of 128, SwiGLU 8192, vocab 128256, untied head), random-init fp16
weights ~ N(0, 0.02^2), 512-token uniform-random prompt prefilled (MFMA prefill launch,
timed as time to first token), then
one bench step = one monokernel launch that decodes 512 greedy tokens from
position 512 (the generation state is rewound to the end of the prompt before
each step; the KV cache of the prompt stays in HBM).

Prints one JSON line on stdout (progress goes to stderr):
  value        decode tokens/s (whole job = this one GPU)
  roofline     algorithmic bytes per launch (all weights + one embedding row +
               the K/V of every attended position, per step) over the
               monokernel's mean duration measured with HIP events on the
               stream it is launched on, against the 8 TB/s HBM peak
  cpu_baseline the CPU oracle on this host on a bounded sample
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(model, w, P: int, n: int, steps: int = 8, steps_1t: int = 2, max_prompt: int = 1024) -> dict:
    """Time the CPU oracle on every host core of this process: the prefill of the workload's own
    prompt (its TTFT baseline), then `steps` decode tokens -- the first `steps` of the timed launch's
    positions -- and `steps_1t` more on one thread.  Prompts longer than `max_prompt` (the float64
    prefill would take minutes) are cut to min(64, max_prompt) tokens and the sample says so."""
    import numpy as np
    import threadpoolctl
    from decode_megakernel_wave_amd import inputs
    from oracle import decoder as od

    prompt_len = P if P <= max_prompt else min(64, max_prompt)
    ids = inputs.make_prompt(model, P, seed=1)[:prompt_len]
    cores = len(os.sched_getaffinity(0))
    dec = od.Decoder(w, model.n_heads, model.n_kv_heads, model.rms_eps, model.rope_theta,
                     max_seq=prompt_len + steps + steps_1t + 1)
    with threadpoolctl.threadpool_limits(cores):
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        tp = time.perf_counter()
        t = int(np.argmax(dec.prefill(ids)))
        prefill_s = time.perf_counter() - tp
        t0 = time.perf_counter()
        for s in range(steps):
            t = int(np.argmax(dec.step(t, prompt_len + s)))
        dt = time.perf_counter() - t0
    with threadpoolctl.threadpool_limits(1):
        t1 = time.perf_counter()
        for s in range(steps, steps + steps_1t):
            t = int(np.argmax(dec.step(t, prompt_len + s)))
        dt1 = time.perf_counter() - t1
    if prompt_len == P:
        where = (f"after the workload's own {P}-token prompt (KV context {P + 1}..{P + steps}, the first {steps} of "
                 f"the timed launch's {P + 1}..{P + n})")
    else:
        kv = 2 * model.n_layers * model.n_kv_heads * model.head_dim * 2 * (P + (n + 1) / 2)
        kv_share = kv / (kv + 2 * model.n_params() - 2 * model.vocab * model.d_model + 2 * model.d_model)
        where = (f"after a {prompt_len}-token prompt (KV context {prompt_len}..{prompt_len + steps} instead of "
                 f"{P}..{P + n}: a float64 prefill of {P} tokens takes minutes; K/V are {100 * kv_share:.1f}% of the "
                 f"bytes per token at the full context)")
    return {"value": steps / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "prefill_s": prefill_s, "prefill_tokens": prompt_len,
            "one_thread": {"value": steps_1t / dt1, "unit": "tokens/s", "cores": 1, "steps": steps_1t},
            "sample": f"float64 oracle decode of {steps} greedy tokens of the same {model.name} decoder {where}, "
                      f"then {steps_1t} tokens on one thread; prefill_s = the oracle's prefill of that prompt"}


# sources that decide what the monokernel reads and writes: the device code and the schedule
KERNEL_SOURCES = ("mk_device.h", "mk_kernel.hip", "mk_layout.h", "mk_plan.cpp", "mk_plan.h")


def kernel_sources_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update(name.encode())
        with open(os.path.join(ROOT, "decode_megakernel_wave_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, n: int, launch: dict):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE passes, scaled
    by the copy-kernel calibration; None unless they were taken on these exact kernel sources
    and this launch shape."""
    path = os.path.join(ROOT, "profiles", f"mk_monokernel_{workload}_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sources_sha256_16") != kernel_sources_hash() or rec.get("decode_tokens_per_launch") != n:
        return None
    if any(rec.get("launch", {}).get(k) != v for k, v in launch.items()):
        return None
    return rec


def traced_decode(model, w, ids, P: int, n: int, opts, trace_steps: int, top_k: int = 1,
                  temperature: float = 1.0) -> dict:
    """One extra launch (not timed) with the time journal on for its first steps: handoff latency per op."""
    import torch
    import decode_megakernel_wave_amd as mk
    from decode_megakernel_wave_amd import synclat

    opts.trace_steps = trace_steps
    ctx = mk.mk_create(model, max_seq=P + n + 1, opts=opts)
    try:
        wd = mk.to_device(w)
        mk.mk_load_weights(ctx, wd)
        del wd
        torch.cuda.empty_cache()
        if top_k > 1:
            mk.mk_set_sampling(ctx, top_k, temperature, seed=3)
        mk.mk_prefill(ctx, ids)
        mk.mk_decode(ctx, min(n, max(trace_steps, 8)))
        rec = mk.mk_read_trace(ctx)
    finally:
        mk.mk_destroy(ctx)
    res = synclat.handoffs(rec)
    log(f"[bench] handoff latency over {trace_steps} traced steps (us, median/p99): "
        + ", ".join(f"{k} {v['median_us']:.2f}/{v['p99_us']:.2f}" for k, v in res.items() if v["median_us"] is not None))
    log("[bench] critical-path span per stage (us, mean): "
        + ", ".join(f"{k} {v['span_mean_us']:.2f}" for k, v in res.items() if v["span_mean_us"] is not None))
    return {"traced_steps": trace_steps, "definition": "last producer's publish (its output stores issued) -> a "
            "waiting consumer's inputs staged, device wall clock (10 ns ticks); median / p99 over (stage, consumer) "
            "pairs; critical = last consumer ready - last producer's publish, per stage; early_consumers = consumers "
            "staged before the last producer published (they needed only earlier producers); span = last consumer "
            "done - last producer done", "per_op": res}


def fine_mark_decode(model, w, ids, P: int, opts) -> dict:
    """One extra launch (not timed) of 4 decode steps with the fine marks of step 0 recorded
    (MK_DEBUG_TS): median phase durations of each instruction, per op, over layers 1..L-1."""
    import torch
    import decode_megakernel_wave_amd as mk
    from decode_megakernel_wave_amd import synclat

    L = model.n_layers
    os.environ["MK_DEBUG_TS"] = "1"
    ctx = mk.mk_create(model, max_seq=P + 5, opts=opts)
    try:
        wd = mk.to_device(w)
        mk.mk_load_weights(ctx, wd)
        del wd
        torch.cuda.empty_cache()
        mk.mk_prefill(ctx, ids)
        mk.mk_decode(ctx, 4)
        grid = mk.mk_stats(ctx)["grid"]
        max_ins = mk.mk_plan_check(model, P + 5, grid)["max_ins_per_cta"]
        if max_ins != 5 * L + 2:
            raise RuntimeError(f"fine marks expect 5 instructions per layer and workgroup, got {max_ins} in all")
        ts = mk.mk_debug_ts(ctx, grid, max_ins)
        if not (ts[:, -1, 0] > 0).all():
            raise RuntimeError("fine marks expect every workgroup to run all 5 ops of every layer")
        kernel = mk.mk_kernel_name(ctx)
    finally:
        mk.mk_destroy(ctx)
        del os.environ["MK_DEBUG_TS"]
    names = ["qkv", "attention", "o_proj", "up_gate", "down"]
    ops = [None] * 5 + names * (L - 1) + ["lm_head", "argmax"]  # layer 0 stages the embedding row
    res = synclat.fine_marks(ts, ops)
    for k, v in res.items():
        log(f"[bench] fine marks {k}: " + ", ".join(f"{p} {x:.2f}" for p, x in v.items()))
    return {"kernel": kernel, "unit": "us", "definition": "median over workgroups and layers 1..L-1 of the phases "
            "between the marks wavefront 0 takes per instruction in step 0 (mk_debug_ts)", "per_op": res}


MFMA_PEAK_TFLOPS = 2500.0  # dense fp16 matrix cores of one MI355X


def time_prefill(mk, ctx, model, ids, reps: int = 3) -> dict:
    """Time to first token: mk_prefill of the prompt, wall clock (ids upload, the MFMA prefill launch over
    positions 0..P-2, the decode step of the last token, t0 back), median of `reps` calls after one
    warm-up; with the prefill kernel's GPU time and its matrix-core throughput."""
    import numpy as np
    P = len(ids)
    mk.mk_prefill(ctx, ids)
    walls, kern, last = [], [], []
    for _ in range(reps):
        t = time.perf_counter()
        t0 = mk.mk_prefill(ctx, ids)
        walls.append((time.perf_counter() - t) * 1e3)
        st = mk.mk_stats(ctx)
        kern.append(st["prefill_ms"])
        last.append(st["gpu_ms"])
    n = st["prefill_positions"]
    stages = None
    if n:
        # device-clock (100 MHz) marks of the last launch's grid barriers: embedding, then 5 stages per layer
        marks = mk.mk_debug_prefill_marks(ctx, model.n_layers).astype(np.int64)
        per = (np.diff(marks) / 100.0).reshape(model.n_layers, 5)
        stages = {name: float(per[:, i].mean()) for i, name in
                  enumerate(["qkv", "attention", "o_proj", "up_gate", "down"])}
        log("[bench] prefill stages, mean us per layer: " + ", ".join(f"{k} {v:.1f}" for k, v in stages.items()))
    qd, kvd, d, f = model.n_heads * model.head_dim, model.n_kv_heads * model.head_dim, model.d_model, model.ffn
    per_pos = 2 * model.n_layers * ((qd + 2 * kvd) * d + d * qd + 3 * f * d)  # GEMM flops per position
    gemm_flops = per_pos * n
    k_ms = float(np.median(kern))
    out = {"prompt_len": P, "ttft_ms": float(np.median(walls)), "prefill_kernel_ms": k_ms,
           "last_token_decode_ms": float(np.median(last)), "prefill_positions": n, "t0": t0,
           "prefill_grid": st["prefill_grid"], "stage_us_per_layer": stages,
           "gemm": {"bound": "mfma", "algorithmic_flops": gemm_flops,
                    "achieved": gemm_flops / (k_ms * 1e-3) / 1e12 if n else None, "unit": "TFLOP/s",
                    "peak": MFMA_PEAK_TFLOPS, "frac": gemm_flops / (k_ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS if n else None,
                    "note": "algorithmic [P x K] x [K x N] flops of every layer's projections over the whole prefill "
                            "launch (its attention and barriers included in the time); the fp32 activations run "
                            "as fp16 hi + lo halves, two MFMAs per product"}}
    log(f"[bench] prefill of {P} tokens: TTFT {out['ttft_ms']:.2f} ms wall (prefill kernel {k_ms:.2f} ms over "
        f"{n} positions, last-token decode step {out['last_token_decode_ms']:.2f} ms); t0={t0}")
    return out


def chain_bench(args) -> int:
    """GEMV-tanh chain y_i = tanh(W_i y_{i-1}), 256 dependent stages in one persistent launch, run with
    NaN-sentinel and with atomic-counter inter-stage sync: microseconds per stage, GB/s, handoff latency."""
    import numpy as np
    import torch
    import decode_megakernel_wave_amd as mk
    from decode_megakernel_wave_amd import inputs, synclat

    n = 2048 if args.workload == "chain" else 256
    stages = 256
    W = inputs.make_chain_weights(n=n, stages=stages)
    x0 = inputs.make_chain_x0(n)
    Wd = torch.from_numpy(W).cuda()
    xd = torch.from_numpy(x0).cuda()
    y = torch.empty((stages, n), dtype=torch.float32, device="cuda")
    results, outs = {}, {}
    for name, mode in (("sentinel", mk.MK_SYNC_SENTINEL), ("counter", mk.MK_SYNC_COUNTER)):
        ch = mk.mk_chain_create(n, stages, Wd, mk.mk_default_options(sync_mode=mode, xcd_replicas=args.replicas))
        try:
            for _ in range(args.warmup):
                mk.mk_chain_run(ch, xd, y)
            ms = []
            for _ in range(args.steps):
                mk.mk_chain_run(ch, xd, y)
                ms.append(mk.mk_chain_stats(ch)["gpu_ms"])
            st = mk.mk_chain_stats(ch)
            outs[name] = y.cpu().numpy().copy()
        finally:
            mk.mk_chain_destroy(ch)
        ch = mk.mk_chain_create(n, stages, Wd, mk.mk_default_options(sync_mode=mode, xcd_replicas=args.replicas,
                                                                      trace_steps=1))
        try:
            mk.mk_chain_run(ch, xd, y)
            lat = synclat.handoffs(mk.mk_chain_read_trace(ch)).get("chain")
        finally:
            mk.mk_chain_destroy(ch)
        mean_ms = float(np.mean(ms))
        results[name] = {"us_per_stage": mean_ms * 1e3 / stages, "launch_ms": mean_ms,
                         "GB_per_s": st["weight_bytes"] / (mean_ms * 1e-3) / 1e9, "handoff_latency": lat}
        log(f"[bench] chain {n}x{n} {name}: {results[name]['us_per_stage']:.3f} us/stage, "
            f"{results[name]['GB_per_s']:.0f} GB/s, handoff median {lat['median_us']:.2f} us")
    same = bool(np.array_equal(outs["sentinel"].view(np.uint32), outs["counter"].view(np.uint32)))
    stream_us = stages * n * n * 2 / (HBM_PEAK_GBS * 1e3) / stages
    out = {"metric": f"GEMV-tanh chain, {stages} dependent stages of {n}x{n} fp16 in one launch: us per stage",
           "value": results["sentinel"]["us_per_stage"], "unit": "us/stage", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": False, "vs_baseline": None, "dtype": "f16 weights, f32 accumulate",
           "data": "synthetic: W_i ~ N(0,0.02^2) fp16, x0 ~ N(0,1) fp32",
           "config": {"workload": f"chain {stages} x {n}x{n}", "xcd_replicas": args.replicas},
           "sentinel": results["sentinel"], "counter": results["counter"],
           "counter_over_sentinel": results["counter"]["us_per_stage"] / results["sentinel"]["us_per_stage"],
           "bitwise_equal_modes": same, "streaming_floor_us_per_stage": stream_us}
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="2b", choices=["2b", "2b-long", "2b-tp8-shard", "0.5b", "tiny", "chain", "chain-s"],
                    help="decoder workloads, or the GEMV-tanh chain microbenchmark (chain: 256 stages of "
                         "2048x2048; chain-s: 256 stages of 256x256, cache-resident, to isolate sync latency)")
    ap.add_argument("--decode-steps", type=int, default=0, help="tokens per launch (default: the workload's)")
    ap.add_argument("--sync", default="sentinel", choices=["sentinel", "counter"])
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--top-k", type=int, default=1, help="1 = greedy (the benchmark); 2..16 = top-k sampling")
    ap.add_argument("--temperature", type=float, default=1.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--trace-steps", type=int, default=0,
                    help="after the timed launches, run one more launch that records the per-instruction time "
                         "journal of its first N steps and report the inter-stage handoff latency")
    ap.add_argument("--fine-marks", action="store_true",
                    help="after the timed launches, run one more launch with the fine per-instruction marks of "
                         "its first step recorded and report the median phase durations per op")
    ap.add_argument("--probes", action="store_true",
                    help="only run the calibration probes (empty-kernel launch cost, nontemporal read ceiling "
                         "over 4 GiB, naive atomic grid barrier) and print one JSON line")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 device-to-device copies of MIB MiB (torch) and exit: the reference "
                         "kernel for scaling the HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the monokernel runs on a single "
              "MI355X; the multi-GPU tensor-parallel path is a design note, not part of this build.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.copy_calibration:
        n = args.copy_calibration << 18  # fp32 elements
        x = torch.ones(n, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()
        log(f"[bench] copied {args.copy_calibration} MiB 5 times")
        return 0

    import decode_megakernel_wave_amd as mk
    from decode_megakernel_wave_amd import inputs

    if args.probes:
        buf = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
        buf.fill_(1)
        launch = mk.mk_probe_launch(2000)
        read = mk.mk_probe_read(buf, repeats=5)
        del buf
        barrier = mk.mk_probe_barrier(2000)
        handoff = {}
        for name, mode, same in (("idle_cross_xcd", 0, False), ("idle_same_xcd", 0, True),
                                 ("streaming_cus_ringless_poller", 1, False),
                                 ("streaming_cus_poller_streams_too", 2, False),
                                 ("streaming_cus_same_xcd", 1, True),
                                 ("quiet_pair_cus_rest_streaming", 3, False),
                                 ("quiet_pair_cus_rest_streaming_same_xcd", 3, True)):
            handoff[name] = mk.mk_probe_handoff(mode, same)
            log(f"[bench] handoff probe {name}: {handoff[name]['us_per_handoff']:.3f} us, "
                f"{handoff[name]['stream_GB_per_s']:.0f} GB/s streamed, same-XCD pairs {handoff[name]['same_xcd_pairs']:.2f}")
        out = {"probes": "calibration", "launch": launch, "read_4GiB_GB_per_s": read,
               "read_frac_of_8TBps": read / HBM_PEAK_GBS, "naive_grid_barrier_us": barrier,
               "handoff_under_streaming": handoff,
               "note": "pages' MI300X context: ~4.5 us launch, 7.59-7.88 us atomic grid sync"}
        log(f"[bench] probes: launch {launch['us_per_launch_pipelined']:.2f} us pipelined / "
            f"{launch['us_per_launch_round_trip']:.2f} us round trip; read {read:.0f} GB/s; barrier {barrier:.2f} us")
        print(json.dumps(out), flush=True)
        return 0

    if args.workload.startswith("chain"):
        return chain_bench(args)

    wl = inputs.WORKLOADS[args.workload]
    model, P = wl.model, wl.prompt_len
    n = args.decode_steps or wl.decode_steps
    max_seq = P + n + 1
    log(f"[bench] workload {args.workload}: generating {model.n_params() / 1e9:.2f}B fp16 weights")
    t = time.time()
    w = inputs.make_weights(model, seed=0)
    ids = inputs.make_prompt(model, P, seed=1)
    log(f"[bench] weights ready in {time.time() - t:.1f}s; uploading")
    opts = mk.mk_default_options(sync_mode=mk.MK_SYNC_COUNTER if args.sync == "counter" else mk.MK_SYNC_SENTINEL,
                                 xcd_replicas=args.replicas)
    ctx = mk.mk_create(model, max_seq=max_seq, opts=opts)
    wd = mk.to_device(w)
    mk.mk_load_weights(ctx, wd)
    del wd
    torch.cuda.empty_cache()
    if args.top_k > 1:
        mk.mk_set_sampling(ctx, args.top_k, args.temperature, seed=3)
    prefill = time_prefill(mk, ctx, model, ids)
    t0 = prefill.pop("t0")

    def step():
        mk.mk_rewind(ctx, P)
        toks = mk.mk_decode(ctx, n)
        return toks, mk.mk_stats(ctx)

    for i in range(args.warmup):
        toks, st = step()
        log(f"[bench] warmup {i}: {st['gpu_ms']:.2f} ms GPU for {n} tokens")
    torch.cuda.synchronize()
    kernel_ms, algo = [], []
    t_start = time.perf_counter()
    for i in range(args.steps):
        toks, st = step()
        kernel_ms.append(st["gpu_ms"])
        algo.append(st["algo_bytes"])
        log(f"[bench] step {i}: {st['gpu_ms']:.2f} ms GPU, {n / st['gpu_ms'] * 1e3:.0f} tok/s")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    sent = mk.mk_count_sentinels(ctx)
    stats = mk.mk_stats(ctx)
    kernel_name = mk.mk_kernel_name(ctx)
    mk.mk_destroy(ctx)
    sync_latency = None
    if args.trace_steps > 0:
        sync_latency = traced_decode(model, w, ids, P, n, opts, args.trace_steps, args.top_k, args.temperature)
    fine = fine_mark_decode(model, w, ids, P, opts) if args.fine_marks else None

    mean_ms = float(np.mean(kernel_ms))
    achieved = float(np.mean(algo)) / (mean_ms * 1e-3) / 1e9
    traffic = measured_traffic(args.workload, n, {"grid": stats["grid"], "block": stats["block"],
                                                  "lds_bytes": stats["lds_bytes"], "ring_depth": stats["ring_depth"],
                                                  "sync": args.sync, "xcd_replicas": args.replicas,
                                                  "kernel": kernel_name})
    out = {
        "metric": "batch-1 decode tokens/s per request on 1 MI355X; achieved HBM TB/s of 8",
        "value": n * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 weights, f32 accumulate",
        "data": "synthetic: random-init fp16 weights N(0,0.02^2), uniform-random prompt ids",
        "config": {"workload": f"{args.workload} decoder greedy decode", "layers": model.n_layers,
                   "d_model": model.d_model, "heads": f"{model.n_heads}q/{model.n_kv_heads}kv x {model.head_dim}",
                   "ffn": model.ffn, "vocab": model.vocab, "prompt_len": P, "decode_tokens_per_step": n,
                   "batch": 1, "sync": args.sync, "xcd_replicas": args.replicas,
                   "token_choice": "greedy" if args.top_k == 1 else f"top-{args.top_k} sampling, T={args.temperature}",
                   "grid": stats["grid"],
                   "block": stats["block"], "lds_bytes": stats["lds_bytes"], "ring_depth": stats["ring_depth"]},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic["traffic_bytes_per_launch"] if traffic else None,
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "traffic_read_write": [traffic["fetch_bytes_per_launch"], traffic["write_bytes_per_launch"]]
                     if traffic else None,
                     "kernel": kernel_name, "kernel_ms": mean_ms, "kernel_ms_median": float(np.median(kernel_ms)),
                     "algo_bytes_per_launch": float(np.mean(algo))},
        "kernel_tokens_per_s": n / mean_ms * 1e3,
        "prefill": prefill,
        "residual_sentinels": sent,
    }
    if sync_latency is not None:
        out["sync_latency"] = sync_latency
    if fine is not None:
        out["fine_marks"] = fine
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle (bounded sample)")
        try:
            out["cpu_baseline"] = cpu_baseline(model, w, P, n)
        except MemoryError:
            out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
