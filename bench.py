#!/usr/bin/env python3
"""Benchmark of the canvas-denoising hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload full|sampler|blockar|prefill|tiny|stream|copy]
                    [--no-cpu-baseline]
                    [--sampler-mode M] [--experts bf16|fp8] [--prefill-rows R]

Prints ONE JSON line (see the keys below). A step is one pass of the
workload's hot path over one batch of synthetic input that is already
resident in HBM:

* ``sampler``: one entropy-bounded sampling step (temperature-scaled
  softmax, entropy, argmax, accept / Philox re-noise, mean-entropy and
  stability stop) over a bf16 logits canvas [256 x 262144] whose background
  is N(0, 3)-like with a +12 peak planted in 70% of the rows. 48 distinct
  logits buffers (6.4 GB) rotate with the 48-step temperature schedule, so
  every step reads cold HBM rather than the 256 MB Infinity Cache.

* ``full`` (default): the whole denoising loop of a 30-layer MoE model
  over a 256-token canvas with an 8192-token prompt in the KV cache:
  self-conditioning, 30 layers, LM head over 262144 tokens, the sampler,
  the 16-byte stop read-back and a block commit whenever a canvas stops.
  ``--experts fp8`` runs it with the routed experts' weights stored as FP8
  E4M3 with per-row scales (an opt-in mode at reduced weight precision,
  reported under its own metric name, never as the bf16 figure).
* ``blockar``: block-autoregressive generation, a 32768-token prompt
  prefilled (timed and reported separately), then 8 canvases denoised and
  committed one after another; the value is committed tokens/s.
* ``prefill``: encoder mode at scale, the 32768-token prompt of the
  block-autoregressive workload prefilled into an empty cache in chunks of
  ``--prefill-rows`` rows.
* ``tiny``: the small fp32 configuration (1 layer, d_model 256, 16 experts
  top-2, vocab 4096, 64 prompt tokens, 8-step canvases over the prompt, one
  canvas plus its commit timed on its own); a correctness configuration,
  bound by launches, not by HBM.
* ``stream``: a plain streaming read of 4 GiB (libdg's calibration kernel),
  the ceiling a bandwidth-bound kernel can reach on the box.
* ``copy``: a plain 1 GiB device copy, the calibration run for the HBM
  byte counters of the profiles.

The roofline entry is for the dominant kernel, timed live with HIP events
(marker packets before and after each launch, on the kernel's own stream)
through libdg's profiling hooks. The cpu_baseline entry
times the CPU oracle (tests-only code) on a bounded sample of the same
workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(name: str, src_hash: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if the kernel is unchanged."""
    p = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("source_hash") != src_hash:
        return None
    return d.get("bytes_per_launch")


# --------------------------------------------------------------------- sampler
def bench_sampler(args):
    import torch
    from canvas_denoising_amd import _lib as L
    from canvas_denoising_amd.runtime import SamplerState

    rows, V, S = 256, 262144, 48
    sched = L.make_sched(max_steps=S, seed=0, mode=args.sampler_mode)
    log(f"[bench] generating {S} logits buffers {rows}x{V} bf16")
    bufs = []
    for s in range(S):
        t = torch.empty(rows, V, dtype=torch.bfloat16, device="cuda")
        L.dg_synth_planted_logits(0, s, rows, V, 3.0, 12.0, t)
        bufs.append(t)
    st = SamplerState(rows, V)
    torch.cuda.synchronize()

    def run(n, first):
        for i in range(first, first + n):
            s = i % S
            if s == 0:
                st.init(sched, (i // S) % 1024)
            st.sample(bufs[s], sched, s, (i // S) % 1024)

    log(f"[bench] warmup {args.warmup}")
    run(args.warmup, 0)
    torch.cuda.synchronize()
    L.dg_profile_enable(True, 4 * (args.steps + 64))
    L.dg_profile_only("sample_partial")
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(args.steps, 0)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    live = L.dg_profile_report()
    L.dg_profile_only(None)
    run(min(args.steps, 48), 0)
    torch.cuda.synchronize()
    prof = L.dg_profile_report()
    L.dg_profile_enable(False)
    stop = st.stop_state()
    part = live["sample_partial"]
    part_us = part["avg_us"]
    bytes_per_launch = rows * V * 2
    achieved = bytes_per_launch / (part_us * 1e-6) / 1e9
    src = kernel_source_hash(["canvas_denoising_amd/csrc/sampler.hip"])
    steps_per_s = args.steps / dt
    out = {
        "metric": "sampler steps/s (256 x 262144 bf16 logits)",
        "value": steps_per_s,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dt * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "sampler-only: bf16 logits 256x262144, N(0,3)-like background, +12 peak in 70% "
                               "of rows, 48-step linear 0.8->0.4 schedule, 48 rotating buffers",
                   "canvas": rows, "vocab": V, "max_steps": S, "sampler_mode": args.sampler_mode,
                   "canvas_tokens_per_s": steps_per_s * rows,
                   "kernels_us": {k: v["avg_us"] for k, v in prof.items()},
                   "stopped_at_end": stop["stopped"]},
        "roofline": {"kernel": "sample_partial", "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": load_traffic("sample_partial", src),
                     "algorithmic_bytes_per_launch": bytes_per_launch, "avg_us": part_us,
                     "timed_with": "HIP events (marker packets) around each launch of the partial kernel in the "
                                   "timed region"},
    }
    del bufs
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_sampler(rows, V, S, args.cpu_seconds)
    return out


def cpu_baseline_sampler(rows, V, S, budget_s):
    """Oracle sampler on a row sample of the same logits; scaled to whole-canvas steps/s."""
    sys.path.insert(0, ROOT)
    import numpy as np
    import synthetic
    from oracle.sampler import Schedule, sample_step

    sample_rows = 32
    sched = Schedule(max_steps=S, seed=0)
    t_total, rows_done, steps = 0.0, 0, 0
    prev, stable = None, 0
    while t_total < budget_s and steps < S:
        bits = synthetic.planted_logits_rows(0, steps, rows, V, range(sample_rows))
        lg = synthetic.bf16_bits_to_f32(bits).astype(np.float64)
        t0 = time.perf_counter()
        res = sample_step(lg, steps, 0, sched, prev, stable)
        t_total += time.perf_counter() - t0
        prev, stable = res.pred, res.stable
        rows_done += sample_rows
        steps += 1
    canvas_steps = rows_done / rows
    return {"value": canvas_steps / t_total, "unit": "steps/s", "cores": 1, "kind": "oracle",
            "sample": f"oracle sample_step (NumPy fp64, single-threaded ufuncs) on {sample_rows} of {rows} rows "
                      f"for {steps} steps ({t_total:.1f} s of CPU time), scaled to whole 256-row canvas steps"}


# ------------------------------------------------------------- full denoise step
EXPERT_KERNELS = ("expert_gateup", "expert_down")


def bench_full(args):
    """Whole hot path: self-conditioning, 30 MoE layers, LM head, sampler, stop read-back, block commit."""
    import numpy as np
    import torch
    from canvas_denoising_amd import _lib as L
    from canvas_denoising_amd import configs
    from canvas_denoising_amd.runtime import Model, SamplerState, stop_dict

    w = configs.full_loop_bf16(args.layers)
    d = w.desc
    d.prefill_rows = args.prefill_rows
    C, V, S = d.canvas, d.vocab, w.max_steps
    n_blocks = (args.steps + S - 1) // S + 1
    capacity = w.prompt + (n_blocks + 2) * C  # + the separately timed committed canvas
    log(f"[bench] model {d.n_layers} layers, weights {L.dg_weights_bytes(d) / 1e9:.1f} GB, KV capacity {capacity}")
    model = Model(d, capacity, seed=0)
    fp8 = args.experts == "fp8"
    if fp8:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        model.use_expert_fp8(True)
        torch.cuda.synchronize()
        log(f"[bench] FP8 experts: {L.dg_expert_fp8_bytes(d) / 1e9:.1f} GB quantized in {time.perf_counter() - t0:.2f} s")
    gu_name = "expert_gateup_fp8" if fp8 else "expert_gateup"
    prompt = torch.empty(w.prompt, dtype=torch.int32, device="cuda")
    L.dg_synth_uniform_ids(4, 10, w.prompt, V, prompt)
    t0 = time.perf_counter()
    model.prefill(prompt)
    torch.cuda.synchronize()
    prefill_s = time.perf_counter() - t0
    log(f"[bench] prefill {w.prompt} tokens: {prefill_s:.2f} s")
    placement = None
    if args.placement_tries > 1:
        # load-time choice among allocations of the weights: each copy is timed over a few steps
        probe = torch.empty(C, dtype=torch.int32, device="cuda")
        L.dg_synth_uniform_ids(5, 11, C, V, probe)

        def measure(n=10):
            model.denoise_step(probe, 0, logits=model.logits)
            torch.cuda.synchronize()
            t = time.perf_counter()
            for _ in range(n):
                model.denoise_step(probe, 0, logits=model.logits)
            torch.cuda.synchronize()
            return (time.perf_counter() - t) / n

        t0 = time.perf_counter()
        times, kept = model.place_weights(measure, args.placement_tries)
        placement = {"tries": args.placement_tries, "ms_per_step": [round(1e3 * x, 3) for x in times],
                     "kept": kept, "seconds": round(time.perf_counter() - t0, 2),
                     "note": "the weights' speed follows their allocation; each candidate (the original and "
                             "device copies) timed over 10 steps without self-conditioning, the fastest kept"}
        log(f"[bench] weight placement: {placement['ms_per_step']} ms/step, kept {kept}")
    sched = L.make_sched(max_steps=S, seed=0)
    if args.sampler_records == "lm_head":
        model.fuse_sampler_stats(sched)
    st = SamplerState(C, V)
    logits = model.logits
    block_ids = torch.empty(C, dtype=torch.int32, device="cuda")
    counters = {"steps": 0, "commits": 0, "stopped": 0}

    def run(n_steps, block0):
        """n_steps denoising steps; a canvas ends at its stop or after S steps and is then committed.
        The 16-byte stop state of a step is read back whenever that step could have stopped
        (Model.denoise_canvas)."""
        block, left = block0, n_steps
        while left > 0:
            steps, stopped = model.denoise_canvas(st, sched, block, limit=left, logits=logits)
            counters["steps"] += steps
            left -= steps
            if stopped or steps == S:
                counters["stopped"] += int(stopped)
                block_ids.copy_(st.pred)
                model.commit(block_ids)
                counters["commits"] += 1
                block += 1
        return block

    def one_canvas(block):
        """One canvas from its init to its stop (or S steps), then its commit: the pages' unit of output."""
        steps, stopped = model.denoise_canvas(st, sched, block, logits=logits)
        block_ids.copy_(st.pred)
        model.commit(block_ids)
        return steps, int(stopped)

    log(f"[bench] warmup {args.warmup}")
    blk = run(args.warmup, 0)
    torch.cuda.synchronize()
    counters.update(steps=0, commits=0, stopped=0)
    # timed region 1: the throughput, steps replayed from HIP graphs, no events
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    blk = run(args.steps, blk)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    commits, stops = counters["commits"], counters["stopped"]
    # timed region 4 (committed output): one whole canvas, init to stop or S steps, plus its commit
    blk += 1
    log(f"[bench] timing one committed canvas")
    torch.cuda.synchronize()
    t4 = time.perf_counter()
    steps4, stopped4 = one_canvas(blk)
    torch.cuda.synchronize()
    dt4 = time.perf_counter() - t4
    blk += 1
    # timed region 2: the same loop with launches issued directly and HIP events (marker packets) around
    # every launch, on each kernel's stream: the per-kernel table and the roofline kernel's live
    # per-launch duration. (Recording every launch site keeps the launches as spread as in a replayed
    # step; rocprofv3 measured the routed-expert kernel 4% slower when only its own launches carried
    # events.)
    n_ev = min(args.steps, 16)
    L.dg_profile_only(None)
    L.dg_profile_enable(True, 2000 * (n_ev + 2))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    blk = run(n_ev, blk)
    torch.cuda.synchronize()
    dt_ev = time.perf_counter() - t1
    prof = L.dg_profile_report()
    n_prof = n_ev
    live = prof
    L.dg_profile_enable(False)
    steps_per_s = args.steps / dt
    # algorithmic bytes of the routed-expert kernels: every expert's weights, once per launch (FP8:
    # one byte per weight plus a float32 scale per row)
    es = 2
    if fp8:
        gu_bytes = d.n_experts * 2 * d.d_expert * (d.d_model + 4)
        dn_bytes = d.n_experts * d.d_model * (d.d_expert + 4)
    else:
        gu_bytes = d.n_experts * 2 * d.d_expert * d.d_model * es
        dn_bytes = d.n_experts * d.d_model * d.d_expert * es
    gu = live[gu_name]
    gu_us = gu["avg_us"]
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9
    src = kernel_source_hash(["canvas_denoising_amd/csrc/moe.hip"])
    metric = "canvas denoise steps/s (256-token canvas)"
    if fp8:
        metric = "canvas denoise steps/s (256-token canvas, FP8 E4M3 routed-expert weights)"
    # roofline of the whole step (derived bytes; activations excluded)
    layer_bytes = (gu_bytes + dn_bytes + ((d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim * d.d_model +
                   d.n_q_heads * d.head_dim * d.d_model + d.n_experts * d.d_model + 3 * d.d_shared * d.d_model) * es)
    kv_len = w.prompt + C
    attn_bytes = 2 * d.n_kv_heads * kv_len * d.head_dim * es
    step_bytes = d.n_layers * (layer_bytes + attn_bytes) + 2 * V * d.d_model * es + 3 * C * V * es
    step_roof_s = step_bytes / (HBM_PEAK_GBS * 1e9)
    out = {
        "metric": metric,
        "value": steps_per_s,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dt * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"full denoise loop: {d.n_layers} MoE layers d_model {d.d_model}, 16q/8kv x 128 heads, "
                               f"128 experts top-8 (704, gated GeLU) + shared 2816, tied vocab {V}, self-conditioning "
                               f"FFN {d.d_selfcond}, prompt KV {w.prompt}, canvas {C}, up to {S} steps per canvas, "
                               "block commit after each canvas; random-init weights",
                   "expert_weights": "fp8 e4m3, per-row float32 scales" if fp8 else "bf16",
                   "sampler_records": args.sampler_records,
                   "weights_placement": placement,
                   "canvas_tokens_per_s": steps_per_s * C,
                   "committed_tokens_per_s": C / dt4,
                   "committed_canvas": {"steps": steps4, "stopped": stopped4, "seconds": dt4,
                                        "note": "one canvas from init to its stop (or the step budget) plus "
                                                "its commit, timed on its own"},
                   "commits_in_timed_steps": commits, "stops": stops,
                   "prefill_tokens_per_s": w.prompt / prefill_s, "prefill_rows": d.prefill_rows,
                   "step_roofline_ms": step_roof_s * 1e3,
                   "step_roofline_frac": step_roof_s / (dt / args.steps),
                   "kernels_us": {k: v["avg_us"] for k, v in sorted(prof.items())},
                   "kernels_total_us_per_step": {k: v["total_us"] / n_prof for k, v in sorted(prof.items())}},
        "roofline": {"kernel": gu_name, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": load_traffic(gu_name, src),
                     "algorithmic_bytes_per_launch": gu_bytes, "avg_us": gu_us, "launches": gu["count"],
                     "timed_with": f"HIP events (marker packets) around every launch over {n_ev} steps issued "
                                   f"directly ({dt_ev * 1e3 / n_ev:.2f} ms/step)"},
    }
    model.close()
    del model
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_full(d, w.prompt, args.cpu_seconds)
    return out


def cpu_baseline_full(d, prompt, budget_s):
    """Oracle time of one denoising step, extrapolated from one layer (x n_layers) plus LM head,
    self-conditioning and sampler on a row sample; weights drawn with NumPy (values do not change the
    oracle's arithmetic cost)."""
    sys.path.insert(0, ROOT)
    import numpy as np
    from oracle import model as OM
    from oracle.sampler import Schedule, sample_step
    rng = np.random.default_rng(0)
    shape = OM.ModelShape(n_layers=1, d_model=d.d_model, n_q_heads=d.n_q_heads, n_kv_heads=d.n_kv_heads,
                          head_dim=d.head_dim, n_experts=d.n_experts, top_k=d.top_k, d_expert=d.d_expert,
                          d_shared=d.d_shared, gated=bool(d.gated), vocab=d.vocab, d_selfcond=d.d_selfcond)
    D, hd, F, Fs = d.d_model, d.head_dim, d.d_expert, d.d_shared
    g = lambda *s: rng.standard_normal(s) * 0.02
    lw = {"wq": g(d.n_q_heads * hd, D), "wk": g(d.n_kv_heads * hd, D), "wv": g(d.n_kv_heads * hd, D),
          "wo": g(D, d.n_q_heads * hd), "wr": g(d.n_experts, D), "sh_gate": g(Fs, D), "sh_up": g(Fs, D),
          "sh_down": g(D, Fs), "experts": [{"gate": g(F, D), "up": g(F, D), "down": g(D, F)}
                                           for _ in range(d.n_experts)]}
    C = d.canvas
    L = prompt + C
    kc = rng.standard_normal((d.n_kv_heads, L, hd))
    vc = rng.standard_normal((d.n_kv_heads, L, hd))
    x = rng.standard_normal((C, D))
    t0 = time.perf_counter()
    OM.layer_forward(lw, x, kc, vc, prompt, shape, causal=False)
    t_layer = time.perf_counter() - t0
    rows = 16
    E = rng.standard_normal((d.vocab, D)) * 0.02
    W = {"embed": E, "sc_w1": g(d.d_selfcond, D), "sc_w2": g(D, d.d_selfcond)}
    t0 = time.perf_counter()
    lg = OM.lm_head(W, x[:rows], shape)
    t_lm = (time.perf_counter() - t0) * C / rows
    res = None
    t0 = time.perf_counter()
    res = sample_step(lg, 1, 0, Schedule(), None, 0, keep_probs=True)
    t_samp = (time.perf_counter() - t0) * C / rows
    t0 = time.perf_counter()
    OM.self_condition(W, res.probs)
    t_sc = (time.perf_counter() - t0) * C / rows
    step_s = d.n_layers * t_layer + t_lm + t_samp + t_sc
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas = 1
    cores = len(os.sched_getaffinity(0))
    return {"value": 1.0 / step_s, "unit": "steps/s", "cores": min(cores, blas), "kind": "oracle",
            "sample": f"oracle (NumPy fp64) one MoE layer over the {C}-row canvas with {L} keys "
                      f"({t_layer:.2f} s) x {d.n_layers} layers, plus LM head ({t_lm:.2f} s), sampler "
                      f"({t_samp:.2f} s) and self-conditioning ({t_sc:.2f} s) timed on {rows} rows and scaled to "
                      f"{C}; host cores {cores}, BLAS threads {blas}"}


def bench_blockar(args):
    """Block-autoregressive generation: a 32768-token prompt prefilled (timed separately), then 8
    canvases of 256, each denoised until its two-fold stop or 48 steps and committed to the KV cache
    before the next one starts. Reports committed tokens/s over the 8 canvases (denoising + commits)."""
    import torch
    from canvas_denoising_amd import _lib as L
    from canvas_denoising_amd import configs
    from canvas_denoising_amd.runtime import Model, SamplerState

    w = configs.block_ar_bf16()
    d = w.desc
    d.prefill_rows = args.prefill_rows
    C, V, S = d.canvas, d.vocab, w.max_steps
    log(f"[bench] model {d.n_layers} layers, KV capacity {w.capacity}")
    model = Model(d, w.capacity, seed=0)
    prompt = torch.empty(w.prompt, dtype=torch.int32, device="cuda")
    L.dg_synth_uniform_ids(5, 10, w.prompt, V, prompt)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    model.prefill(prompt)
    torch.cuda.synchronize()
    prefill_s = time.perf_counter() - t0
    log(f"[bench] prefill {w.prompt} tokens: {prefill_s:.2f} s")
    sched = L.make_sched(max_steps=S, seed=0)
    st = SamplerState(C, V)
    logits = model.logits
    block_ids = torch.empty(C, dtype=torch.int32, device="cuda")

    def canvas(block, max_steps, commit):
        steps, stopped = model.denoise_canvas(st, sched, block, limit=max_steps, logits=logits)
        if commit:
            block_ids.copy_(st.pred)
            model.commit(block_ids)
        return steps, int(stopped)

    log(f"[bench] warmup {args.warmup} steps (not committed)")
    canvas(0, max(1, args.warmup), False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    steps = stops = 0
    for b in range(w.blocks):
        n, stopped = canvas(b, S, True)
        steps += n
        stops += stopped
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    out = {
        "metric": "committed tokens/s (block-autoregressive, 8 canvases of 256)",
        "value": w.blocks * C / dt,
        "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": args.warmup, "ms_per_step": dt * 1e3 / steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"block-AR: {d.n_layers} MoE layers as the full loop, prompt {w.prompt} prefilled "
                               f"(untimed), {w.blocks} canvases of {C} denoised (<= {S} steps, two-fold stop) and "
                               f"committed one after another, KV length {w.prompt} -> {w.prompt + w.blocks * C}; "
                               "random-init weights",
                   "denoise_steps_per_s": steps / dt, "canvas_tokens_per_s": steps * C / dt, "stops": stops,
                   "prefill_tokens_per_s": w.prompt / prefill_s, "prefill_s": prefill_s,
                   "prefill_rows": d.prefill_rows},
    }
    model.close()
    return out


def bench_prefill(args):
    """Encoder mode at scale: the 30-layer model prefills a 32768-token prompt (config 4's prologue) in
    chunks of --prefill-rows rows; a step is one whole prefill into an empty cache."""
    import torch
    from canvas_denoising_amd import _lib as L
    from canvas_denoising_amd import configs
    from canvas_denoising_amd.runtime import Model

    w = configs.block_ar_bf16()
    d = w.desc
    d.prefill_rows = args.prefill_rows
    log(f"[bench] model {d.n_layers} layers, prompt {w.prompt}, chunks of {max(d.canvas, d.prefill_rows)} rows")
    model = Model(d, w.prompt, seed=0)
    fp8 = args.experts == "fp8"
    if fp8:
        model.use_expert_fp8(True)
    prompt = torch.empty(w.prompt, dtype=torch.int32, device="cuda")
    L.dg_synth_uniform_ids(5, 10, w.prompt, d.vocab, prompt)

    def run(n):
        for _ in range(n):
            L.dg_kv_set_length(model.ctx, 0)
            model.prefill(prompt)

    run(args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(args.steps)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    model.close()
    return {
        "metric": "prefill tokens/s (32768-token prompt" + (", FP8 E4M3 routed-expert weights)" if fp8 else ")"),
        "value": args.steps * w.prompt / dt, "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": dt * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"encoder prefill of {w.prompt} uniform token ids, {d.n_layers} MoE layers "
                               f"d_model {d.d_model}, 128 experts top-8, causal, random-init weights",
                   "prefill_rows": max(d.canvas, d.prefill_rows),
                   "expert_weights": "fp8 e4m3, per-row float32 scales" if fp8 else "bf16"},
    }


def bench_tiny(args):
    """The tiny fp32 configuration: 1 layer, d_model 256, 4 heads x 64, 16 experts top-2 (plain GeLU FFN 512)
    + shared 512, vocab 4096, self-conditioning 256; 64 prompt tokens prefilled; canvases of 8 steps
    (temperature 0.8 -> 0.4), each committed before the next. A step = self-conditioning + the layer + LM
    head + sampler + the 16-byte stop read-back."""
    import torch
    from canvas_denoising_amd import _lib as L
    from canvas_denoising_amd import configs
    from canvas_denoising_amd.runtime import Model, SamplerState

    w = configs.tiny_f32()
    d = w.desc
    C, V, S = d.canvas, d.vocab, w.max_steps
    model = Model(d, w.prompt + C, seed=0)
    prompt = torch.empty(w.prompt, dtype=torch.int32, device="cuda")
    L.dg_synth_uniform_ids(1, 10, w.prompt, V, prompt)
    model.prefill(prompt)
    sched = L.make_sched(max_steps=S, seed=0)
    st = SamplerState(C, V)
    logits = model.logits
    block_ids = torch.empty(C, dtype=torch.int32, device="cuda")
    state = {"block": 0}

    def run(n):
        """n steps of canvases over the 64-token prompt (a canvas restarts after its stop or S steps;
        a canvas cut short by n starts afresh on the next call)."""
        left = n
        while left > 0:
            steps, _ = model.denoise_canvas(st, sched, state["block"], limit=left, logits=logits)
            left -= steps
            state["block"] += 1

    run(args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(args.steps)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    # one canvas from init to its end plus its commit, timed on its own (the context then grows by it)
    t1 = time.perf_counter()
    run(S)
    block_ids.copy_(st.pred)
    model.commit(block_ids)
    torch.cuda.synchronize()
    dt_canvas = time.perf_counter() - t1
    L.dg_kv_set_length(model.ctx, w.prompt)
    # per-kernel table (events) over one more canvas, issued directly
    L.dg_profile_enable(True, 200 * S)
    run(S)
    torch.cuda.synchronize()
    prof = L.dg_profile_report()
    L.dg_profile_enable(False)
    model.close()
    steps_per_s = args.steps / dt
    lm = prof.get("lm_head", {"avg_us": float("nan")})
    lm_flops = 2 * C * d.d_model * V
    out = {
        "metric": "canvas denoise steps/s (tiny fp32 configuration)",
        "value": steps_per_s, "unit": "steps/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": dt * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"tiny fp32: 1 layer d_model {d.d_model}, 4x64 heads over {w.prompt} prompt KV + "
                               f"the canvas, 16 experts top-2 (plain GeLU {d.d_expert}) + shared {d.d_shared}, "
                               f"vocab {V}, self-conditioning {d.d_selfcond}, {S}-step canvases over the prompt; "
                               "committed tokens/s from one canvas plus its commit; random-init weights",
                   "canvas_tokens_per_s": steps_per_s * C,
                   "committed_tokens_per_s": C / dt_canvas,
                   "kernels_us": {k: v["avg_us"] for k, v in sorted(prof.items())}},
        "roofline": {"kernel": "lm_head", "bound": "mfma", "achieved": lm_flops / (lm["avg_us"] * 1e-6) / 1e12,
                     "peak": 157.3, "unit": "TFLOP/s",
                     "frac": lm_flops / (lm["avg_us"] * 1e-6) / 1e12 / 157.3, "traffic": None,
                     "algorithmic_flops_per_launch": lm_flops, "avg_us": lm["avg_us"],
                     "note": "fp32 MFMA peak; the configuration is launch-bound (about 1.7 GFLOP a step)"},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_tiny(d, w.prompt, S)
    return out


def cpu_baseline_tiny(d, prompt, S):
    """The oracle's whole step of the tiny configuration (all 256 rows): self-conditioning, the layer, LM head
    and sampler, with the seeded synthetic weights."""
    sys.path.insert(0, ROOT)
    import numpy as np
    import synthetic
    from canvas_denoising_amd import configs
    from oracle import model as OM
    from oracle.sampler import Schedule, sample_step, tempered_probs

    shape = OM.ModelShape(n_layers=d.n_layers, d_model=d.d_model, n_q_heads=d.n_q_heads, n_kv_heads=d.n_kv_heads,
                          head_dim=d.head_dim, n_experts=d.n_experts, top_k=d.top_k, d_expert=d.d_expert,
                          d_shared=d.d_shared, gated=bool(d.gated), vocab=d.vocab, d_selfcond=d.d_selfcond,
                          canvas=d.canvas)
    W = synthetic.SyntheticWeights(configs.shape_dict(d), seed=0, dtype="f32", sigma=0.02)
    cache = OM.KVCache.empty(shape, prompt + d.canvas)
    OM.encode(W, cache, synthetic.uniform_ids(1, 10, prompt, d.vocab), shape)
    canvas = synthetic.uniform_ids(2, 10, d.canvas, d.vocab)
    sched = Schedule(max_steps=S, seed=0)
    prev, n, t = None, 0, 0.0
    while n < S and t < 15.0:
        t0 = time.perf_counter()
        sc = None if prev is None else OM.self_condition(W, tempered_probs(prev, 0.8))
        lg = OM.denoise_step(W, cache.copy(), canvas, sc, shape)
        sample_step(lg, n, 0, sched, None, 0)
        t += time.perf_counter() - t0
        prev, n = lg, n + 1
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas = 1
    cores = len(os.sched_getaffinity(0))
    return {"value": n / t, "unit": "steps/s", "cores": min(cores, blas), "kind": "oracle",
            "sample": f"oracle (NumPy fp64) whole steps of the tiny configuration, all {d.canvas} rows: "
                      f"self-conditioning, the layer, LM head and sampler; {n} steps in {t:.1f} s; host cores "
                      f"{cores}, BLAS threads {blas}"}


def bench_stream(args):
    """Calibration: libdg's plain streaming-read kernel over 4 GiB (nontemporal 16-byte loads, grid-stride),
    at several grid sizes; the value is the best read bandwidth. A ceiling for the bandwidth-bound kernels."""
    import torch
    from canvas_denoising_amd import _lib as L
    n = 4 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    L.dg_synth_uniform_ids(7, 11, n // 4, 1 << 30, src)
    sink = torch.empty(1 << 16, dtype=torch.int32, device="cuda")
    res = {}
    for blocks in (1024, 2048, 4096, 8192, 16384):
        for _ in range(args.warmup):
            L.dg_stream_read(src, n, sink, blocks)
        torch.cuda.synchronize()
        L.dg_profile_enable(True, args.steps + 4)
        for _ in range(args.steps):
            L.dg_stream_read(src, n, sink, blocks)
        prof = L.dg_profile_report()["stream_read"]
        L.dg_profile_enable(False)
        res[blocks] = n / (prof["avg_us"] * 1e-6) / 1e9
    best = max(res, key=res.get)
    return {"metric": "streaming read bandwidth (calibration kernel, 4 GiB)", "value": res[best], "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": n / res[best] / 1e6,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
            "config": {"workload": "plain streaming read of 4 GiB, nontemporal 16-byte loads, grid-stride",
                       "gbs_by_workgroups": res, "best_workgroups": best},
            "roofline": {"kernel": "stream_read", "bound": "hbm", "achieved": res[best], "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": res[best] / HBM_PEAK_GBS, "traffic": None,
                         "algorithmic_bytes_per_launch": n}}


def bench_copy(args):
    """Plain device-to-device copy of a known size: the calibration run for HBM byte counters
    (FETCH_SIZE / WRITE_SIZE per launch divided by the bytes copied)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    return {"metric": "device copy bandwidth (read + write)", "value": 2 * n * args.steps / dt / 1e9,
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": dt * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "u8", "data": "synthetic",
            "config": {"workload": f"calibration copy of {n} bytes per launch"}}


WORKLOADS = {"sampler": bench_sampler, "full": bench_full, "blockar": bench_blockar, "prefill": bench_prefill,
             "tiny": bench_tiny, "stream": bench_stream, "copy": bench_copy}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="full")
    ap.add_argument("--layers", type=int, default=30, help="layers of the full workload (30 = the benchmark)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sampler-mode", type=int, default=0,
                    help="sampler workload: dg_sched.mode flags (1 either-stop, 2 group acceptance, 4 categorical)")
    ap.add_argument("--experts", choices=["bf16", "fp8"], default="bf16",
                    help="full / prefill workloads: routed-expert weights in the model dtype or as FP8 E4M3 "
                         "(opt-in mode)")
    ap.add_argument("--prefill-rows", type=int, default=2048,
                    help="rows per prefill chunk (0 = the canvas); chunks above 256 rows run the experts as "
                         "token-tiled GEMMs")
    ap.add_argument("--placement-tries", type=int, default=4,
                    help="full workload: allocations of the weights timed at load time (the fastest is kept); "
                         "1 keeps the first")
    ap.add_argument("--sampler-records", choices=["lm_head", "pass"], default="pass",
                    help="full / blockar workloads: the sampler's split-row records made by the LM head as it "
                         "writes the logits (dg_ctx_fuse_sampler_stats), or by the sampler's own pass over them")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: libdg has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    if args.steps is None:
        args.steps = {"sampler": 480, "copy": 20, "prefill": 3, "tiny": 400, "stream": 10}.get(args.workload, 96)
    if args.warmup is None:
        args.warmup = {"sampler": 48, "copy": 2, "prefill": 1, "tiny": 16, "stream": 2}.get(args.workload, 4)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (libdg runs only on MI355X).", file=sys.stderr)
        sys.exit(1)
    out = WORKLOADS[args.workload](args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
