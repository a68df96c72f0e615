"""Benchmark: denoising steps/s and generated tokens/s of the early-skip decode
of a 32-layer 8B-class masked-diffusion model (d 4096, 32x128 heads, FFN
11008, vocab 126464, random-init bf16 weights) on one MI355X: batch 1,
256 uniform prompt tokens + 256 masked, blocks of 32, 256 steps x 1 token,
skip at layer 4 with keep = 25% (128 of 512 rows recomputed in layers 4..31).

A step is one dl_denoise_step (embed, 4 full-row layers, score + top-k,
28 partial layers on the kept rows, LM head + confidence, unmask; every 32nd
step is a full refresh).  Inputs are resident in HBM before the timed region.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-variants]

Prints one JSON line.  After the timed headline steps it also times, on the
same model, the nested two-level skip, the response-only schedule and the key
score on the same prompt, and the long-context shape (4096 + 512) with the
plain skip and with DyLLM's per-layer re-selection ("variants"; their own
steps/s, not part of `value`).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
# full8b step rooflines: the sum over a step's stages of max(algorithmic bytes /
# 8 TB/s, FLOPs / 2.5 PFLOP/s).  A skip step moves ~15.1 GB (28 kept-row layers,
# 4 full prefix layers, the LM head on the kept rows): 1.98 ms; a refresh step
# ~16.6 GB and 7.3 TFLOP (every layer and the LM head on all 512 rows): 2.92 ms.
ROOFLINE_SKIP_MS = 1.98
ROOFLINE_REFRESH_MS = 2.92


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--weights", choices=("blocked", "row_major"), default="blocked",
                    help="storage order of the product weights on the device (same results bit for bit)")
    ap.add_argument("--workload", default="full8b")
    ap.add_argument("--timing-stride", type=int, default=8,
                    help="time about one launch in this many of each kernel class (1: every launch)")
    ap.add_argument("--no-variants", action="store_true",
                    help="only the headline decode: skip the per-step, one-layer and variant timings")
    ap.add_argument("--no-sample", action="store_true",
                    help="skip the sampled kernel-timing pass that follows the headline steps")
    return ap.parse_args()


def variant_schedules(sched):
    """Schedules of the method's variants timed beside the headline step on the
    same model and prompt: a second skip level at layer 8 (keep 50% at layer 4,
    25% at layer 8; ES-dLLM section 2B), DyLLM's response-only steps with a
    full-context step every 4 steps (section 2B, strategy 3), eq. I on
    layer 4's rotated keys instead of its input (ES-dLLM section 2A), and the
    more frequent full refresh of ES-dLLM* (every 16 or every 8 steps inside a
    block, besides each block's first step; ES-dLLM section 2B and its results)."""
    import dataclasses
    return {
        "nested_s4_keep0.5_s8_keep0.25": dataclasses.replace(sched, keep=0.5, skip_layer2=8, keep2=0.25),
        "response_only_full_every4": dataclasses.replace(sched, response_interval=4),
        "key_rows_scored": dataclasses.replace(sched, score_tensor="key"),
        "refresh_every16": dataclasses.replace(sched, refresh_interval=16),
        "refresh_every8": dataclasses.replace(sched, refresh_interval=8),
    }


def long_context_schedules():
    """The long-context shape (4096 prompt + 512 masked tokens, blocks of 64,
    keep 1/8: 576 of 4608 rows) with the plain early skip and with DyLLM's
    per-layer re-selection at keep 1/8 (section 2B)."""
    import dataclasses
    import workloads
    wl = workloads.workload("long8b")
    return wl, {
        "long_context_skip": wl.sched,
        "long_context_per_layer": dataclasses.replace(wl.sched, per_layer=True, keep_layer=wl.sched.keep),
    }


def time_variant(torch, Decoder, dev_model, prompts, sched, steps: int, warmup: int, timed_classes=()):
    """steps/s of one variant schedule (fresh caches; warm-up, then `steps`
    steps from the decode's first step, refresh steps included).  The kernel
    classes in timed_classes are timed (one launch in 8) and reported."""
    from dynamic_token_skipping_amd import dl_timing_enable, dl_timing_read, dl_timing_reset
    dec = Decoder(dev_model, prompts, sched)
    for t in range(warmup):
        dec.step(t % sched.steps)
    dec.reset()
    dl_timing_reset()
    for kc in timed_classes:
        dl_timing_enable(kc, 8)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        t = i % sched.steps
        if t == 0 and i > 0:
            dec.reset()
        dec.step(t)
    end.record()
    torch.cuda.synchronize()
    for kc in timed_classes:
        dl_timing_enable(kc, 0)
    ms = start.elapsed_time(end)
    kinds = {"refresh": 0, "response_only": 0, "full_context": 0}
    for i in range(steps):
        t = i % sched.steps
        p = dec.params(t)
        kinds["refresh" if p.full_refresh else ("response_only" if p.response_only else "full_context")] += 1
    out = {"steps_per_s": round(steps / (ms / 1e3), 3), "ms_per_step": round(ms / steps, 4),
           "gen_tokens_per_s": round(steps / (ms / 1e3) * dec.per_step * dec.B, 3), "steps": steps,
           "step_kinds": kinds, "keep": sched.keep, "skip_layer": sched.skip_layer,
           "skip_layer2": sched.skip_layer2, "keep2": sched.keep2, "response_interval": sched.response_interval,
           "refresh_interval": sched.refresh_interval,
           "score_tensor": sched.score_tensor, "per_layer": sched.per_layer, "keep_layer": sched.keep_layer,
           "rows": dec.S, "batch": dec.B}
    for kc in timed_classes:
        tm = dl_timing_read(kc)
        out[f"kernel_class_{kc}"] = {"launches_timed": tm["launches"],
                                     "avg_launch_us": round(tm["ms"] * 1e3 / max(tm["launches"], 1), 2),
                                     "TFLOP/s": round(tm["flops"] / max(tm["ms"], 1e-9) / 1e9, 1),
                                     "GB/s": round(tm["bytes"] / max(tm["ms"], 1e-9) / 1e6, 1)}
    del dec
    torch.cuda.empty_cache()
    return out


def keep_rows(keep: float, n: int) -> int:
    """Rows a top-k step keeps of n: ceil(keep * n) with keep read as float32,
    clamped to [1, n] (the count the library computes)."""
    import math

    import numpy as np
    return max(1, min(n, math.ceil(float(np.float32(keep)) * n))) if n > 0 else 0


def decode_step_flops(dims, lens, sched, refresh: bool) -> float:
    """Algorithmic FLOPs of one step: every layer's products on its rows
    (2 * layer params * rows), attention (4 * d * rows * keys per sequence)
    and the LM head (2 * vocab * d * rows) on the rows that reach it."""
    P, d, L, s = dims.layer_params(), dims.d, dims.n_layers, sched.skip_layer
    ks = lens if refresh else [keep_rows(sched.keep, n) for n in lens]
    full = s * (2.0 * P * sum(lens) + 4.0 * d * sum(n * n for n in lens))
    part = (L - s) * (2.0 * P * sum(ks) + 4.0 * d * sum(k * n for k, n in zip(ks, lens)))
    return full + part + 2.0 * dims.vocab * d * sum(ks)


def time_batched(torch, Decoder, dev_model, steps: int = 32, warmup: int = 4):
    """The batched workload (16 sequences, prompts ~U{128..1024} right-padded,
    256 generated each, blocks of 32, 128 steps x 2 tokens, keep 1/4 per
    sequence) on the loaded weights: steps/s and tokens/s over the decode's
    first `steps` steps (refresh steps included), and the algorithmic FLOP rate
    against the bf16 matrix-core peak (the step is matrix-core bound: about
    3.3k kept rows)."""
    import workloads
    wl = workloads.workload("batch8b")
    prompts, lens = workloads.make_prompt(wl)
    dec = Decoder(dev_model, prompts, wl.sched)
    for t in range(warmup):
        dec.step(t)
    dec.reset()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for t in range(steps):
        dec.step(t)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    flops = sum(decode_step_flops(wl.dims, dec.seq_lens, wl.sched, bool(dec.params(t).full_refresh))
                for t in range(steps))
    n_ref = sum(bool(dec.params(t).full_refresh) for t in range(steps))
    tflops = flops / (ms / 1e3) / 1e12
    out = {"workload": ("batch8b: 16 sequences, prompts ~U{128..1024} right-padded + 256 masked each, blocks of 32, "
                        "128 steps x 2 tokens, skip layer 4, keep 1/4 per sequence, full8b weights"),
           "steps": steps, "refresh_steps": n_ref, "steps_per_s": round(steps / (ms / 1e3), 3),
           "ms_per_step": round(ms / steps, 3),
           "gen_tokens_per_s": round(steps / (ms / 1e3) * dec.per_step * dec.B, 1),
           "rows": sum(dec.seq_lens), "kept_rows_per_skip_step": sum(keep_rows(wl.sched.keep, n) for n in dec.seq_lens),
           "TFLOP/s": round(tflops, 1), "frac_mfma": round(tflops / PEAK_BF16_TFLOPS, 4)}
    del dec
    torch.cuda.empty_cache()
    return out


def time_tiny(torch, reps: int = 40):
    """The tiny workload (2 layers, d 64, fp32, 16 prompt + 48 masked, 8 steps
    x 6 tokens): steps/s over `reps` whole decodes.  Launch-bound; no roofline
    claim."""
    import workloads
    from dynamic_token_skipping_amd import Decoder, DeviceModel
    wl = workloads.workload("tiny")
    m = workloads.make_model(wl.dims, wl.seed, wl.dtype, "cuda")
    prompts, _ = workloads.make_prompt(wl)
    dec = Decoder(DeviceModel(m, wl.dims.n_heads, wl.dims.head_dim, wl.dtype), prompts, wl.sched)
    dec.run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dec.reset()
        dec.run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    n = reps * wl.sched.steps
    return {"workload": "tiny: 2 layers, d 64, fp32, 16 prompt + 48 masked, 8 steps x 6 tokens, keep 16 of 64",
            "steps": n, "steps_per_s": round(n / (ms / 1e3), 1), "ms_per_step": round(ms / n, 4),
            "decodes_per_s": round(reps / (ms / 1e3), 2)}


def time_step_kinds(torch, dec, sched, n_steps: int):
    """Median time of the skip steps and of the refresh steps among the
    decode's first n_steps steps, each step bracketed by its own pair of HIP
    events on the decode stream."""
    dec.reset()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_steps)]
    for t in range(n_steps):
        ev[t][0].record()
        dec.step(t)
        ev[t][1].record()
    torch.cuda.synchronize()
    times = {"refresh": [], "skip": []}
    for t in range(n_steps):
        times["refresh" if dec.params(t).full_refresh else "skip"].append(ev[t][0].elapsed_time(ev[t][1]))

    def med(v):
        v = sorted(v)
        return round(v[len(v) // 2], 4) if v else None
    out = {"sample": f"steps 0..{n_steps - 1} of the decode, one event pair per step",
           "skip_steps": len(times["skip"]), "refresh_steps": len(times["refresh"]),
           "skip_ms_median": med(times["skip"]), "refresh_ms_median": med(times["refresh"]),
           "roofline_skip_ms": ROOFLINE_SKIP_MS, "roofline_refresh_ms": ROOFLINE_REFRESH_MS}
    if out["skip_ms_median"]:
        out["skip_frac_of_roofline"] = round(ROOFLINE_SKIP_MS / out["skip_ms_median"], 4)
    if out["refresh_ms_median"]:
        out["refresh_frac_of_roofline"] = round(ROOFLINE_REFRESH_MS / out["refresh_ms_median"], 4)
    dec.reset()
    return out


def time_layer_steps(torch, model, weight_layout: str, n_steps: int = 30, warmup: int = 3):
    """One layer step of the 8B-class layer per keep ratio, on the layer8b
    inputs (cached and current hidden states, K/V caches, confidences):
    score + top-k over the 512 rows (the selection's row map built with
    row_off, for the row entry points to reuse), gather of the kept fp32 rows,
    the partial attention sub-block and the FFN on them.  Consecutive steps take layers 4,
    5 and 6 of the loaded model in turn (1.2 GB of distinct weights), so the
    weights stream from HBM.  Algorithmic bytes: the layer's weights, its K/V
    cache and the two score inputs read once, and the kept fp32 rows read and
    written; FLOPs: 2 * params * k + 4 * k * S * d."""
    import workloads
    from dynamic_token_skipping_amd import (DL_F32, DL_SEL_TOPK, SelectionTensors, dl_ffn_rows, dl_gather,
                                            dl_partial_attn, dl_score_select, make_dims, workspace)
    wl = workloads.workload("layer8b")
    dims, S = wl.dims, wl.prompt_len
    d = dims.d
    st = workloads.make_layer_state(wl, "cuda")
    dl = make_dims(1, S, d, dims.n_heads, dims.head_dim, dims.d_ffn, dims.vocab, 1, "bf16",
                   weight_layout=weight_layout)
    ws = workspace(dl, S)
    seq = torch.tensor([S], dtype=torch.int32, device="cuda")
    x_s = st["h_cur"].float()                      # the fp32 layer input the kept rows are gathered from
    kc, vc = st["k"].clone(), st["v"].clone()
    layers = [model["layers"][i] for i in (4, 5, 6)]
    params = dims.layer_params()
    sel = SelectionTensors(1, S, row_map=True)
    x_rows = torch.empty((S, d), dtype=torch.float32, device="cuda")
    out = {"sample": f"{n_steps} layer steps per keep after {warmup} warm-up steps, one event pair around them"}
    for keep in (1.0, 0.5, 0.25, 0.125):
        k = max(1, min(S, int(keep * S + 0.999999)))

        def one(i):
            lw = layers[i % len(layers)]
            dl_score_select(dl, st["h_cur"], st["h_prev"], st["conf"], seq, "esdllm", 0.5, DL_SEL_TOPK, keep, 0.0,
                            sel, ws=ws)
            dl_gather(dl, x_s, d, DL_F32, sel, k, x_rows)
            dl_partial_attn(dl, lw, x_rows, sel, seq, k, kc, vc, ws)
            dl_ffn_rows(dl, lw, x_rows, sel, k, ws)
        for i in range(warmup):
            one(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        h0 = time.perf_counter()
        for i in range(n_steps):
            one(i)
        host_us = (time.perf_counter() - h0) * 1e6 / n_steps   # enqueue time: below us, the GPU never waits
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / n_steps
        alg = 2 * params + 2 * (2 * S * d * 2) + k * d * 8
        flops = 2 * params * k + 4 * k * S * d
        out[f"keep_{keep}"] = {"rows": k, "us": round(us, 2), "host_enqueue_us": round(host_us, 1),
                               "alg_MB": round(alg / 1e6, 1),
                               "GB/s": round(alg / us / 1e3, 1), "frac_hbm": round(alg / us / 1e3 / PEAK_HBM_GBS, 4),
                               "TFLOP/s": round(flops / us / 1e6, 1),
                               "frac_mfma": round(flops / us / 1e6 / PEAK_BF16_TFLOPS, 4)}
    return out


def blas_threads() -> int:
    """Threads numpy's BLAS runs the oracle's products on."""
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(wl, model_gpu, prompts, skip_steps: int = 4):
    """The fp64 oracle's own decode loop on the host cores, on a bounded
    sample of the same workload: from the initial state of the first
    sequence, its refresh step (step 0) and the next ``skip_steps`` skip steps,
    each timed.  Every layer uses its own weights (converted to float64 once,
    before the timed steps).  The per-step rate of a whole decode follows from
    the schedule: each block has one refresh step and steps_per_block - 1
    skip steps."""
    import numpy as np
    import torch

    from oracle import esdllm as E

    dims, sched = wl.dims, wl.sched
    t0 = time.perf_counter()
    m_np = {"embed": model_gpu["embed"].to(torch.float64).cpu().numpy(),
            "final_norm": model_gpu["final_norm"].to(torch.float64).cpu().numpy(),
            "lm_head": model_gpu["lm_head"].to(torch.float64).cpu().numpy(),
            "layers": [{k: v.to(torch.float64).cpu().numpy() for k, v in lw.items()} for lw in model_gpu["layers"]]}
    t_convert = time.perf_counter() - t0
    st = E.init_state(prompts[0].numpy(), sched.gen_len, dims)
    times = []
    for t in range(1 + skip_steps):
        t0 = time.perf_counter()
        info = E.denoise_step(m_np, dims, st, t, sched)
        times.append(time.perf_counter() - t0)
        assert info.refresh == (t == 0)
    del m_np
    t_ref, t_skip = times[0], sum(times[1:]) / skip_steps
    spb = sched.steps_per_block
    per_step = (t_ref + (spb - 1) * t_skip) / spb
    return {"value": round(1.0 / per_step, 4), "unit": "denoise steps/s", "cores": blas_threads(), "kind": "oracle",
            "sample": (f"the oracle's decode loop (oracle.esdllm.denoise_step, fp64 numpy) on the first sequence "
                       f"of the same workload with every layer's own weights: step 0 (refresh, "
                       f"{t_ref:.2f} s) and steps 1..{skip_steps} (skip, mean {t_skip:.2f} s); a decode step "
                       f"= (1 refresh + {spb - 1} skip) / {spb}; weights converted to float64 beforehand "
                       f"({t_convert:.1f} s, not timed)"),
            "refresh_step_s": round(t_ref, 3), "skip_step_s": round(t_skip, 3),
            "seconds_measured": round(sum(times), 2)}


def recorded_traffic():
    """HBM bytes per dispatch of the dominant kernel, from the rocprofv3
    FETCH_SIZE / WRITE_SIZE runs recorded under profiles/ (scaled by the copy
    calibration).  None when the kernel's source changed after the counters
    were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "kept_row_products_full8b_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        with open(os.path.join(ROOT, rec["source"]), "rb") as f:
            sha = hashlib.sha1(f.read()).hexdigest()
    except (OSError, KeyError, ValueError):
        return None
    return rec["hbm_bytes_per_dispatch"] if sha == rec["source_sha1"] else None


def copy_probe(torch, n_bytes: int = 1 << 30, reps: int = 5):
    """Device-to-device copy of n_bytes, reps times, timed with events: the
    HBM bandwidth a plain streaming kernel reaches (read + write bytes / s).
    Its dispatches also calibrate the FETCH_SIZE / WRITE_SIZE counters."""
    src = torch.empty(n_bytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    gbs = 2.0 * n_bytes * reps / (a.elapsed_time(b) / 1e3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_per_copy": n_bytes, "GB/s": round(gbs, 1)}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; multi-GPU runs are not part of it",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import workloads
    from dynamic_token_skipping_amd import (DL_KC_APPROX, DL_KC_ATTN, DL_KC_GEMM, DL_KC_GEMM_TILED, DL_KC_LMHEAD,
                                            Decoder, DeviceModel, dl_timing_enable, dl_timing_read, dl_timing_reset,
                                            pack_model)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wl = workloads.workload(args.workload)
    dims, sched = wl.dims, wl.sched
    t0 = time.time()
    model = workloads.make_model(dims, wl.seed, wl.dtype, "cuda")
    # the decode's weights: the product weights copied into the blocked order
    # (the row-major model stays for the host baseline's fp64 copy)
    dev_weights = pack_model(model) if args.weights == "blocked" else model
    prompts, lens = workloads.make_prompt(wl)
    dec = Decoder(DeviceModel(dev_weights, dims.n_heads, dims.head_dim, wl.dtype, weight_layout=args.weights),
                  prompts, sched)
    torch.cuda.synchronize()
    print(f"# setup {time.time() - t0:.1f} s: {dims.model_params() / 1e9:.2f} B params", file=sys.stderr, flush=True)

    copy = copy_probe(torch)
    # warm-up (untimed), then restart the decode from its first step
    for t in range(args.warmup):
        dec.step(t % sched.steps)
    dec.reset()
    torch.cuda.synchronize()

    # the headline: K steps of the decode, no instrumentation
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        t = i % sched.steps
        if t == 0 and i > 0:
            dec.reset()
        dec.step(t)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = start.elapsed_time(end)
    steps_per_s = args.steps / (ms / 1e3)
    tok_per_s = steps_per_s * dec.per_step * dec.B

    # a separate pass samples kernel durations: about one launch in
    # timing_stride of each product class (every LM-head launch), each timed by
    # HIP events bound to its own dispatch packets on the decode stream
    classes = (DL_KC_GEMM, DL_KC_ATTN, DL_KC_LMHEAD, DL_KC_GEMM_TILED)
    sample_steps = min(args.steps, 2 * dec.steps_per_block)
    dl_timing_reset()
    if not args.no_sample:
        for kc in classes:
            dl_timing_enable(kc, 1 if kc == DL_KC_LMHEAD else max(1, args.timing_stride))
        dec.reset()
        for t in range(sample_steps):
            dec.step(t)
        torch.cuda.synchronize()
        for kc in classes:
            dl_timing_enable(kc, 0)
        dec.reset()
    g = dl_timing_read(DL_KC_GEMM)
    a = dl_timing_read(DL_KC_ATTN)
    lmh = dl_timing_read(DL_KC_LMHEAD)
    gt = dl_timing_read(DL_KC_GEMM_TILED)
    gemm_gbs = g["bytes"] / (g["ms"] / 1e3) / 1e9 if g["ms"] > 0 else None
    roofline = {"bound": "hbm", "achieved": round(gemm_gbs, 1) if gemm_gbs else None, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(gemm_gbs / PEAK_HBM_GBS, 4) if gemm_gbs else None,
                "traffic": recorded_traffic(),
                "kernel": ("layer products on the 128 kept rows (128-row tiles, 8 waves): k_gemm_mfma BN 64 with 4 K "
                           "splits (O, down), BN 96 with 2 K splits + k_epi_qkv_rows4 (QKV), BN 96 on 256 "
                           f"ragged tiles (gate|up); weights {args.weights.replace('_', '-')}, loaded non-temporal"),
                "sample": (f"a separate pass of {sample_steps} decode steps after the headline steps, about one "
                           f"launch in {max(1, args.timing_stride)} timed"),
                "launches_timed": g["launches"], "launches_total": g["launches"] + g["dropped"],
                "avg_launch_us": round(g["ms"] * 1e3 / max(g["launches"], 1), 2),
                "alg_bytes_per_launch": round(g["bytes"] / max(g["launches"], 1))}
    out = {
        "metric": "denoise steps/sec & gen tokens/sec at keep=25% (8B-class); HBM GB/s vs peak",
        "value": round(steps_per_s, 3), "unit": "denoise steps/s",
        "gen_tokens_per_s": round(tok_per_s, 3),
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{wl.name}: 32-layer 8B-class random-init bf16 model, batch 1, 256 prompt + 256 "
                               f"masked, blocks of 32, 256 steps x 1 token, skip layer 4, keep 0.25",
                   "global_batch": dec.B, "seq_len": dec.S, "keep": sched.keep, "skip_layer": sched.skip_layer,
                   "weight_layout": args.weights},
        "roofline": roofline,
        "kernels": {
            "gemm": {"ms_timed": round(g["ms"], 3), "launches_timed": g["launches"],
                     "GB/s": round(gemm_gbs, 1) if gemm_gbs else None,
                     "TFLOP/s": round(g["flops"] / max(g["ms"], 1e-9) / 1e9, 1)},
            "gemm_tiled": {"ms_timed": round(gt["ms"], 3), "launches_timed": gt["launches"],
                           "GB/s": round(gt["bytes"] / max(gt["ms"], 1e-9) / 1e6, 1),
                           "TFLOP/s": round(gt["flops"] / max(gt["ms"], 1e-9) / 1e9, 1)},
            "attention": {"ms_timed": round(a["ms"], 3), "launches_timed": a["launches"],
                          "avg_launch_us": round(a["ms"] * 1e3 / max(a["launches"], 1), 2),
                          "TFLOP/s": round(a["flops"] / max(a["ms"], 1e-9) / 1e9, 2)},
            "lm_head": {"ms_timed": round(lmh["ms"], 3), "launches_timed": lmh["launches"],
                        "GB/s": round(lmh["bytes"] / max(lmh["ms"], 1e-9) / 1e6, 1)},
        },
        "copy_probe": copy,
        "wall_s": round(wall, 3),
    }
    if wl.name == "full8b" and not args.no_variants:
        out["step_times"] = time_step_kinds(torch, dec, sched, 2 * sched.steps_per_block)
        out["layer_steps"] = time_layer_steps(torch, dev_weights, args.weights)
    if not args.no_variants and wl.name == "full8b":
        dev_model = dec.m
        del dec
        torch.cuda.empty_cache()
        out["variants"] = {name: time_variant(torch, Decoder, dev_model, prompts, vs, min(args.steps, 128), 8)
                           for name, vs in variant_schedules(sched).items()}
        # long context on the same weights: one block of 64 steps (its refresh included)
        lwl, lscheds = long_context_schedules()
        lprompts, _ = workloads.make_prompt(lwl)
        for name, vs in lscheds.items():
            out["variants"][name] = time_variant(torch, Decoder, dev_model, lprompts, vs, 64, 4,
                                                 (DL_KC_ATTN, DL_KC_APPROX) if vs.per_layer else (DL_KC_ATTN,))
        out["variants"]["kernel_classes"] = {str(DL_KC_ATTN): "attention", str(DL_KC_APPROX): "approximate context"}
        out["variants"]["batched"] = time_batched(torch, Decoder, dev_model)
        out["variants"]["tiny"] = time_tiny(torch)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, model, prompts)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
