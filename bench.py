#!/usr/bin/env python3
"""Benchmark of the Whisper-large-v3 encoder attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload window|chunked|batched|small|verify|encoder|decoder|decoder_q8]

A step is one pass of the hot path over one batch of synthetic input. The
default workload is one 30 s window (1500 frames x 1280, 20 heads of 64) through
32 attention sublayers with independently seeded weights, each sublayer being
packed QKV GEMM -> flash attention -> output projection (edda_qkv_pack +
edda_encoder_attn through the C ABI, serial on one stream). Inputs and weights
are resident in HBM before the timed region starts.

Prints ONE JSON line: TFLOP/s (algorithmic FLOPs: 2MNK per GEMM, 4*64 per
admitted (query, key) pair per head), ms per window, the fraction of MI355X
dense fp16 MFMA peak, a roofline entry for the dominant kernel (its duration
measured here with HIP events around back-to-back launches), and the fp64 CPU
oracle timed on a bounded sample of the same workload as a baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2516.6    # MI355X dense fp16 MFMA: 256 CUs x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
COPY_BYTES = 256 << 20       # reference copy: reads and writes this many bytes
D, H, DH, QKV = 1280, 20, 64, 3840


def gemm_flops(m, n, k):
    return 2.0 * m * n * k


def attn_flops(pairs):
    return 4.0 * DH * H * pairs


def source_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "whisper_asr_encoder_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profile_entry(kernel_key, digest):
    """The committed rocprofv3 summary of a kernel (profiles/traffic.json: HBM bytes per launch
    from the PMC runs, the kernel trace's mean duration), or None when the kernel source
    changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        ent = json.load(open(path)).get(kernel_key)
        if ent and ent.get("source_digest") == digest:
            return ent
    except (OSError, ValueError):
        return None
    return None


def measured_traffic(kernel_key, digest):
    """HBM bytes per launch from the committed counters, or None (see profile_entry)."""
    ent = profile_entry(kernel_key, digest)
    return ent.get("bytes_per_launch") if ent else None


def profile_roofline(kernel_key, digest, work, peak, unit_scale):
    """The roofline fraction from the committed profile's timing source (rocprofv3 kernel-trace
    mean duration, another run and possibly another box), beside the live HIP-event figure."""
    ent = profile_entry(kernel_key, digest)
    if not ent or not ent.get("trace_mean_us"):
        return None
    achieved = work / (ent["trace_mean_us"] * 1e-6) / unit_scale
    return {"source": f"profiles/ rocprofv3 kernel-trace mean duration of {kernel_key}",
            "us_per_launch": ent["trace_mean_us"], "achieved": round(achieved, 2),
            "frac": round(achieved / peak, 4)}


class Timer:
    """HIP events on the stream the kernels are launched on (torch's current stream)."""

    def __init__(self, torch):
        self.torch = torch

    def __call__(self, fn, reps):
        t = self.torch
        start, end = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        t.cuda.synchronize()
        start.record()
        for _ in range(reps):
            fn()
        end.record()
        t.cuda.synchronize()
        return start.elapsed_time(end) / reps  # ms


# ---------------------------------------------------------------------------
# Encoder workloads.
# ---------------------------------------------------------------------------

def encoder_bench(args, torch, cfg):
    from whisper_asr_encoder_amd import _lib, inputs as I
    from whisper_asr_encoder_amd.encoder import EncoderAttention
    import oracle  # noqa: F401  (imported lazily for the CPU baseline only)

    wl = I.encoder_workload(cfg)
    layers = wl.layers
    weights = [wl.weights(l) for l in range(layers)]
    enc = EncoderAttention(weights, wl.batch, wl.seq_len, wl.chunk_len,
                           None if cfg in (0, 1) else wl.valid_len)
    x = torch.from_numpy(wl.x).cuda()
    rows = wl.rows
    ys = [torch.empty((rows, D), dtype=torch.float16, device="cuda") for _ in range(layers)]
    o = torch.empty((rows, D), dtype=torch.float16, device="cuda")

    # Algorithmic work per sublayer.
    if cfg == 2:
        valid_rows = int(wl.valid_len[0])
        pairs = 0
        for lo in range(0, valid_rows, wl.chunk_len):
            n = min(lo + wl.chunk_len, valid_rows) - lo
            pairs += n * n
        f_qkv, f_out = gemm_flops(valid_rows, QKV, D), gemm_flops(valid_rows, D, D)
    else:
        pairs = int(sum(wl.seq_len * int(v) for v in wl.valid_len))
        f_qkv, f_out = gemm_flops(rows, QKV, D), gemm_flops(rows, D, D)
    f_attn = attn_flops(pairs)
    flops_layer = f_qkv + f_attn + f_out

    def step():
        for l in range(layers):
            enc.sublayer(x, l, ys[l])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    eager_ms = start.elapsed_time(end) / args.steps
    # The same step captured once in a HIP graph and replayed (as a serving loop would issue
    # it): no host work between launches.
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.warmup):
        graph.replay()
    graph_ms = Timer(torch)(graph.replay, args.steps)
    ms = min(eager_ms, graph_ms)
    tflops = flops_layer * layers / (ms * 1e-3) / 1e12

    # Per-kernel durations: back-to-back launches of one kernel cycling through the layers.
    timer = Timer(torch)
    reps = max(2, args.steps)
    vl = None if cfg in (0, 1) else wl.valid_len

    def run_qkv():
        for l in range(layers):
            _lib.edda_qkv_pack(x, enc.w_qkv[l], enc.b_qkv[l], enc.qkv)

    def run_flash():
        for l in range(layers):
            _lib.edda_flash_attn(enc.qkv, wl.batch, wl.seq_len, wl.chunk_len, vl, o)

    def run_out():  # the output projection's GEMM as edda_encoder_attn launches it (same kernel)
        for l in range(layers):
            _lib.edda_linear(o, enc.w_o[l], enc.b_o[l], ys[l])

    t_qkv = timer(run_qkv, reps) / layers
    t_flash = timer(run_flash, reps) / layers
    t_out = timer(run_out, reps) / layers
    kernels = {
        "qkv_gemm": {"ms": t_qkv, "tflops": f_qkv / (t_qkv * 1e-3) / 1e12},
        "flash_attn": {"ms": t_flash, "tflops": f_attn / (t_flash * 1e-3) / 1e12},
        "out_gemm": {"ms": t_out, "tflops": f_out / (t_out * 1e-3) / 1e12},
    }
    dom = max(("qkv_gemm", "flash_attn"), key=lambda k: kernels[k]["ms"])
    dom_flops = f_qkv if dom == "qkv_gemm" else f_attn
    dom_src = ["gemm.hip"] if dom == "qkv_gemm" else ["flash_attn.hip"]
    achieved = dom_flops / (kernels[dom]["ms"] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP16_TFLOPS, 4),
                "flops_per_launch": dom_flops, "ms_per_launch": round(kernels[dom]["ms"], 5),
                "timing": "HIP events around back-to-back launches of the kernel, this run",
                "traffic": measured_traffic(dom, source_digest(dom_src)),
                "profile": profile_roofline(dom, source_digest(dom_src), dom_flops, PEAK_FP16_TFLOPS, 1e12)}

    names = {0: "one 4 s chunk (200 frames), 1 attention sublayer",
             1: "one 30 s Whisper-large-v3 window (1500 frames), 32 attention sublayers",
             2: "45 s of audio in 4 s chunks (2400 rows, 2250 valid), 32 attention sublayers",
             3: "16 batched 30 s windows with padded key tails, 32 attention sublayers"}
    result = {
        "metric": "encoder attention TFLOP/s + ms per 30 s window (32 layers) on 1 MI355X; % fp16 peak",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_window": round(ms / wl.batch, 4) if cfg != 2 else None,
        "frac_of_fp16_peak": round(tflops / PEAK_FP16_TFLOPS, 4),
        "wall_ms_per_step": round(wall_ms, 4),
        "eager_ms_per_step": round(eager_ms, 4),
        "graph_ms_per_step": round(graph_ms, 4),
        "launch": "hip graph of the step" if graph_ms <= eager_ms else "eager launches",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic (seeded N(0,1) inputs, N(0,1/1280) weights; no trained weights or audio)",
        "config": {"workload": names[cfg], "batch": wl.batch, "seq_len": wl.seq_len,
                   "chunk_len": wl.chunk_len, "d_model": D, "heads": H, "head_dim": DH, "layers": layers,
                   "gflop_per_step": round(flops_layer * layers / 1e9, 3), "parallelism": "single GPU"},
        "kernels": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "roofline": roofline,
        "context": "the pages' only figure for this path is ~430 -> ~285 ms per 30 s window for the "
                   "whole encoder on a Radeon 8060S (gfx1151); not comparable, hence vs_baseline null",
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_encoder(wl, weights, flops_layer, args.cpu_seconds)
    return result


def cpu_baseline_encoder(wl, weights, flops_layer, budget_s):
    """The oracle as it stands, timed on the host on a bounded sample of the same workload:
    whole sublayers (one window) until the time budget is used."""
    import oracle
    threads = blas_threads()
    done, t0 = 0, time.perf_counter()
    windows = wl.batch if wl.cfg != 2 else 1
    per_window_flops = flops_layer / windows
    while done < wl.layers and (done == 0 or time.perf_counter() - t0 < budget_s):
        w = weights[done]
        x = wl.x[:wl.seq_len]
        oracle.encoder_attention(x, w.w_qkv, w.b_qkv, w.w_o, w.b_o, 1, wl.seq_len, wl.chunk_len,
                                 int(wl.valid_len[0]), H)
        done += 1
    el = time.perf_counter() - t0
    return {"value": round(per_window_flops * done / el / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} of {wl.layers} sublayers of window 0 ({wl.seq_len} rows), fp64 NumPy, "
                      f"{el:.1f} s",
            "ms_per_window_extrapolated": round(el / done * wl.layers * 1e3, 1),
            "cpu": cpu_model()}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(n[0])
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


# ---------------------------------------------------------------------------
# Whole encoder: convolutional stem + 32 pre-norm layers + final LayerNorm, one window.
# ---------------------------------------------------------------------------

PAGES_ENCODER_MS = 285.0  # the pages' whole-encoder time per 30 s window (Radeon 8060S)


def full_encoder_bench(args, torch):
    from whisper_asr_encoder_amd import _lib, inputs as I
    from whisper_asr_encoder_amd.encoder import FullEncoder

    seq, layers = I.FRAMES_PER_WINDOW, I.ENCODER_LAYERS
    weights = [I.full_layer_weights(1, l) for l in range(layers)]
    sw = I.stem_weights()
    enc = FullEncoder(weights, stem=sw, batch=1, seq_len=seq)
    mel = torch.from_numpy(I.mel_input(1)).cuda()
    out = torch.empty((seq, D), dtype=torch.float16, device="cuda")

    # Algorithmic work: stem convolutions as GEMMs, per layer QKV + attention + output
    # projection + the two MLP GEMMs (LayerNorm, GELU and residual adds are not counted).
    f_stem = gemm_flops(2 * seq, D, 3 * I.N_MELS) + gemm_flops(seq, D, 3 * D)
    f_qkv, f_out = gemm_flops(seq, QKV, D), gemm_flops(seq, D, D)
    f_attn = attn_flops(seq * seq)
    f_fc = gemm_flops(seq, I.D_FF, D)
    f_layer = f_qkv + f_attn + f_out + 2 * f_fc
    f_total = f_stem + layers * f_layer

    def step():
        enc.forward(mel, out)

    for _ in range(args.warmup):
        step()
    timer = Timer(torch)
    ms = timer(step, args.steps)

    # Components: back-to-back launches of one step, cycling through the layers.
    reps = max(2, args.steps // 2)
    kw = enc._keep
    h = torch.empty((seq, D), dtype=torch.float16, device="cuda")
    x1 = torch.empty((seq, D), dtype=torch.float16, device="cuda")
    qkv = torch.empty((seq, QKV), dtype=torch.float16, device="cuda")
    f = torch.empty((seq, I.D_FF), dtype=torch.float16, device="cuda")
    xw = torch.empty((seq, D), dtype=torch.float16, device="cuda")
    enc.stem(mel, xw)

    def run(fn):
        return timer(lambda: [fn(l) for l in range(layers)], reps) / layers

    t = {
        "stem": timer(lambda: enc.stem(mel, xw), reps),
        "layer": run(lambda l: enc.layer(xw, l, x1)),
        "layer_norm": run(lambda l: _lib.edda_layer_norm(xw, kw[l]["ln1_gamma"], kw[l]["ln1_beta"], h)),
        "qkv_gemm": run(lambda l: _lib.edda_qkv_pack(h, kw[l]["w_qkv"], kw[l]["b_qkv"], qkv)),
        "flash_attn": run(lambda l: _lib.edda_flash_attn(qkv, 1, seq, 0, None, h)),
        "out_gemm": run(lambda l: _lib.edda_linear(h, kw[l]["w_o"], kw[l]["b_o"], x1, residual=xw)),
        "fc1_gemm": run(lambda l: _lib.edda_linear(h, kw[l]["w_fc1"], kw[l]["b_fc1"], f, activation=_lib.ACT_GELU)),
        "fc2_gemm": run(lambda l: _lib.edda_linear(f, kw[l]["w_fc2"], kw[l]["b_fc2"], x1, residual=xw)),
    }
    flops = {"qkv_gemm": f_qkv, "flash_attn": f_attn, "out_gemm": f_out, "fc1_gemm": f_fc, "fc2_gemm": f_fc,
             "layer": f_layer, "stem": f_stem}
    kernels = {k: {"ms": round(v, 5), **({"tflops": round(flops[k] / (v * 1e-3) / 1e12, 2)} if k in flops else {})}
               for k, v in t.items()}
    dom = max(("qkv_gemm", "flash_attn", "out_gemm", "fc1_gemm", "fc2_gemm"), key=lambda k: t[k])
    src = ["flash_attn.hip"] if dom == "flash_attn" else ["gemm.hip"]
    achieved = flops[dom] / (t[dom] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": PEAK_FP16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP16_TFLOPS, 4), "flops_per_launch": flops[dom],
                "ms_per_launch": round(t[dom], 5), "timing": "HIP events around back-to-back launches, this run",
                "traffic": measured_traffic(dom, source_digest(src)),
                "profile": profile_roofline(dom, source_digest(src), flops[dom], PEAK_FP16_TFLOPS, 1e12)}
    result = {
        "metric": "whole-encoder ms per 30 s window (stem + 32 layers + final LayerNorm) on 1 MI355X",
        "value": round(ms, 4), "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "tflops": round(f_total / (ms * 1e-3) / 1e12, 3),
        "frac_of_fp16_peak": round(f_total / (ms * 1e-3) / 1e12 / PEAK_FP16_TFLOPS, 4),
        "higher_is_better": False, "scaling": "weak",
        "vs_baseline": round(ms / PAGES_ENCODER_MS, 6),
        "vs_baseline_note": "value / the pages' ~285 ms per 30 s window for the whole encoder, measured on a "
                            "Radeon 8060S (gfx1151) with trained weights: context, another machine",
        "dtype": "fp16", "data": "synthetic (seeded weights and log-mel input; no trained weights or audio)",
        "config": {"workload": "Whisper-large-v3 encoder, one 30 s window: 128 x 3000 log-mel in, conv stem, "
                               "32 pre-norm layers (1500 x 1280, 20 heads, MLP 5120), final LayerNorm",
                   "gflop_per_step": round(f_total / 1e9, 3), "parallelism": "single GPU"},
        "kernels": kernels, "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_full_encoder(weights, f_layer, layers, args.cpu_seconds)
    return result


def cpu_baseline_full_encoder(weights, f_layer, layers, budget_s):
    """The oracle's whole layers on one window until the time budget is used."""
    import oracle.encoder_layer as OL
    from whisper_asr_encoder_amd import inputs as I
    threads = blas_threads()
    x = I.encoder_workload(1, layers=1).x
    done, t0 = 0, time.perf_counter()
    while done < layers and (done == 0 or time.perf_counter() - t0 < budget_s):
        OL.encoder_layer(x, weights[done], 1, I.FRAMES_PER_WINDOW, 0, I.FRAMES_PER_WINDOW, H)
        done += 1
    el = time.perf_counter() - t0
    return {"value": round(f_layer * done / el / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {layers} encoder layers of one window (1500 rows), fp64 NumPy, {el:.1f} s",
            "ms_per_layer": round(el / done * 1e3, 1), "cpu": cpu_model()}


# ---------------------------------------------------------------------------
# Decoder verification pass: 32 whole decoder layers for one block of 16 tokens.
# ---------------------------------------------------------------------------

def decoder_bench(args, torch):
    from whisper_asr_encoder_amd import _lib, inputs as I
    from whisper_asr_encoder_amd.encoder import DecoderVerifier

    layers, n_q, trial = I.ENCODER_LAYERS, I.VERIFY_BLOCK, 0
    L = I.cache_length(trial)
    weights = [I.decoder_layer_weights(l) for l in range(layers)]
    q8 = args.workload == "decoder_q8"
    dv = DecoderVerifier(weights, max_kv=L, q8=q8)
    enc = torch.from_numpy(I.encoder_workload(1, layers=1).x).cuda()
    dv.set_encoder_output(enc)
    caches = []
    for l in range(layers):
        c = I.verify_self_case(trial, l)
        caches.append((torch.from_numpy(c.k).cuda(), torch.from_numpy(c.v).cuda()))
    mask = torch.from_numpy(_lib.pack_mask_rows(I.causal_block_mask(n_q, L)).view(np.int32)).cuda()
    slots = list(range(L - n_q, L))
    x = torch.from_numpy(I.decoder_block_input(trial)).cuda()
    y = torch.empty_like(x)

    def layer_by_layer():
        for l in range(layers):
            dv.layer(x if l == 0 else y, l, slots, caches[l][0], caches[l][1], L, mask, y)

    def stacked():  # edda_decoder_verify_stack (or _q8): launches of 8 layers
        dv.stack(x, slots, caches, L, mask, y)

    timer = Timer(torch)

    def graph_ms(step):
        for _ in range(args.warmup):
            step()
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()
        return timer(graph.replay, args.steps), graph

    forms = {"stack": stacked, "layer_by_layer": layer_by_layer}
    if args.decoder_form == "stack":
        forms = {"stack": stacked}
    elif args.decoder_form == "layer":
        forms = {"layer_by_layer": layer_by_layer}
    timed = {name: graph_ms(fn) for name, fn in forms.items()}
    best = min(timed, key=lambda k: timed[k][0])
    ms = timed[best][0]
    eager_ms = timer(forms[best], args.steps)

    # Algorithmic bytes per layer: every weight once, the self and cross K/V read, the block's
    # K/V rows written, activations and the mask (small).
    # Matrices: W_qkv (3 D^2), self output, cross query and output (3 D^2), fc1 and fc2;
    # biases: qkv, self output, cross query and output, fc1, fc2; three LayerNorms.
    # Q8_0 matrices: one code byte per weight plus an fp16 scale per 32 (1.0625 bytes).
    mat_bytes = (6 * D * D + 2 * D * I.D_FF) * (1.0625 if q8 else 2)
    w_bytes = int(mat_bytes) + 2 * (3 * D + 3 * D + I.D_FF + D) + 2 * 6 * D
    kv_bytes = 2 * 2 * D * (L + I.FRAMES_PER_WINDOW) + 2 * 2 * D * n_q
    act_bytes = 2 * n_q * D * 4 + n_q * ((L + 31) // 32) * 4
    per_layer = w_bytes + kv_bytes + act_bytes
    gbs = per_layer * layers / (ms * 1e-3) / 1e9
    flops = layers * (gemm_flops(n_q, QKV, D) + 2 * gemm_flops(n_q, D, D) + gemm_flops(n_q, D, D)
                      + 2 * gemm_flops(n_q, I.D_FF, D) + attn_flops(n_q * L) + attn_flops(n_q * I.FRAMES_PER_WINDOW))
    res = {
        "metric": ("decoder verification pass (32 decoder layers, 16-token block"
                   + (", Q8_0 projection weights" if q8 else "") + ") on 1 MI355X"),
        "value": round(ms * 1e3, 2), "unit": "us per pass", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp16 activations, q8_0 weights" if q8 else "fp16",
        "data": "synthetic (seeded weights, caches and block rows)",
        "launch": (f"hip graph of the pass ({'edda_decoder_verify_stack' if best == 'stack' else 'edda_decoder_verify_layer'}"
                   f"{'_q8' if q8 else ''}{'' if best == 'stack' else ' per layer'})"),
        "eager_ms_per_step": round(eager_ms, 4),
        "us_per_pass_by_form": {k: round(v[0] * 1e3, 2) for k, v in timed.items()},
        "us_per_layer": round(ms * 1e3 / layers, 3), "tflops": round(flops / (ms * 1e-3) / 1e12, 3),
        "config": {"workload": f"Whisper-large-v3 decoder verification layers: 16 block tokens, causal self-attention "
                               f"over a {L}-slot cache (block appended), cross-attention over 1500 frames, "
                               "GELU MLP 5120; 32 layers", "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_layer": per_layer, "traffic": None},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decoder(weights, trial, L, n_q, slots, q8, dv, args.cpu_seconds)
    return res


def cpu_baseline_decoder(weights, trial, L, n_q, slots, q8, dv, budget_s):
    """The oracle's decoder layers (fp64) on the same block, caches and cross K/V until the time
    budget is used; microseconds per 32-layer pass, extrapolated."""
    import oracle.decoder_layer as DL
    import oracle.quant as Q
    from whisper_asr_encoder_amd import inputs as I
    threads = blas_threads()
    x = I.decoder_block_input(trial)
    enc = I.encoder_workload(1, layers=1).x
    mask = I.causal_block_mask(n_q, L)
    done, el = 0, 0.0
    while done < len(weights) and (done == 0 or el < budget_s):
        w = weights[done]
        if q8:  # quantized once at load time on both sides: not timed
            w = Q.DequantizedDecoderWeights(w, Q.quantize_decoder_weights(w))
        c = I.verify_self_case(trial, done)
        # Cross K/V are projected once per utterance on both sides: not timed.
        ck, cv = DL.cross_kv(enc, weights[done].w_ck, weights[done].w_cv, weights[done].b_cv)
        t0 = time.perf_counter()
        DL.decoder_verify_layer(x, w, slots, c.k, c.v, L, mask, ck, cv)
        el += time.perf_counter() - t0
        done += 1
    return {"value": round(el / done * len(weights) * 1e6, 1), "unit": "us per pass", "cores": threads,
            "kind": "oracle", "sample": f"{done} of {len(weights)} decoder layers (cross K/V and Q8_0 weights "
                                        f"prepared untimed, as on the GPU), fp64 NumPy, {el:.1f} s",
            "cpu": cpu_model()}


# ---------------------------------------------------------------------------
# Verification workload: 32 decoder layers x (causal self-attention + cross-attention).
# ---------------------------------------------------------------------------

def verify_bench(args, torch):
    """All 8 drawn cache lengths of the verification workload: per trial, 32 layers of causal
    self-attention (16 queries over L_t slots) and cross-attention (16 queries over 1500 encoder
    frames), and the beam variant (5 queries on the token tree of L_t slots)."""
    from whisper_asr_encoder_amd import inputs as I
    from whisper_asr_encoder_amd.encoder import VerifyAttention

    layers, trials = 32, 8
    va = VerifyAttention(1500)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    # Cross K/V: one set per layer (the encoder output of one utterance; drawn as trial 0's),
    # reused by every trial. Two copies of every layer's K/V are used in turn (2 x 32 x 7.7 MB of
    # cross K/V alone, more than the 256 MB Infinity Cache), so every pass reads HBM.
    copies = 2
    cross = [[] for _ in range(copies)]
    cross_cases = []
    for l in range(layers):
        c = I.verify_cross_case(0, l)
        cross_cases.append(c)
        for cp in cross:
            cp.append((d(c.k), d(c.v)))
    per_trial = []
    tot = {"bytes": 0.0, "us": 0.0, "beam_bytes": 0.0, "beam_us": 0.0, "flops": 0.0}
    timer = Timer(torch)
    o = torch.empty((16, H, DH), dtype=torch.float16, device="cuda")
    ob = torch.empty((I.BEAMS, H, DH), dtype=torch.float16, device="cuda")

    def capture(step):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(g):
            step()
        for _ in range(max(1, args.warmup)):
            g.replay()
        return g

    for t in range(trials):
        L = I.cache_length(t)
        sets = [[] for _ in range(copies)]
        beams = [[] for _ in range(copies)]
        b_self = b_cross = b_beam = 0
        f = 0.0
        for l in range(layers):
            sc = I.verify_self_case(t, l)
            tc = I.verify_tree_case(t, l)
            cc = cross_cases[l]
            for i in range(copies):
                q = d(sc.q)  # the block's queries serve the self and the cross call
                sets[i].append((q, d(sc.k), d(sc.v), va.mask_rows(sc.mask), q))
                beams[i].append((d(tc.q), d(tc.k), d(tc.v), va.mask_rows(tc.mask)))
            words = (L + 31) // 32
            b_self += sc.k.nbytes + sc.v.nbytes + 2 * sc.q.nbytes + 16 * words * 4
            b_cross += cc.k.nbytes + cc.v.nbytes + 2 * sc.q.nbytes
            # Beam: K/V rows of the union of the five ancestor sets (the algorithmic bytes),
            # queries, outputs and mask words.
            used = int(tc.mask.any(axis=0).sum())
            b_beam += used * H * DH * 2 * 2 + 2 * tc.q.nbytes + I.BEAMS * words * 4
            f += attn_flops(int(sc.mask.sum())) + attn_flops(16 * 1500)

        def step():
            for i in range(copies):
                for (q, k, v, m, qx), (ck, cv) in zip(sets[i], cross[i]):
                    va(q, k, v, m, o)
                    va(qx, ck, cv, None, o)

        def beam_step():
            for i in range(copies):
                for q, k, v, m in beams[i]:
                    va(q, k, v, m, ob)

        g, gb = capture(step), capture(beam_step)
        ms = timer(g.replay, args.steps) / copies
        ms_b = timer(gb.replay, args.steps) / copies
        per_trial.append({"L": L, "us_per_pass": round(ms * 1e3, 2), "us_per_call": round(ms * 1e3 / (2 * layers), 3),
                          "gbs": round((b_self + b_cross) / (ms * 1e-3) / 1e9, 1),
                          "beam_us_per_call": round(ms_b * 1e3 / layers, 3),
                          "beam_gbs": round(b_beam / (ms_b * 1e-3) / 1e9, 1)})
        tot["bytes"] += b_self + b_cross
        tot["us"] += ms * 1e3
        tot["beam_bytes"] += b_beam
        tot["beam_us"] += ms_b * 1e3
        tot["flops"] += f
        del g, gb, sets, beams
    gbs = tot["bytes"] / (tot["us"] * 1e-6) / 1e9
    dig = source_digest(["verify_attn.hip", "verify_core.hpp"])
    t_causal, t_cross = measured_traffic("verify_causal", dig), measured_traffic("verify_cross", dig)
    traffic = round((t_causal + t_cross) / 2) if t_causal and t_cross else None
    p_causal, p_cross = profile_entry("verify_causal", dig), profile_entry("verify_cross", dig)
    bytes_per_launch = round(tot["bytes"] / (trials * 2 * layers))
    profile = None
    if p_causal and p_cross and p_causal.get("trace_mean_us") and p_cross.get("trace_mean_us"):
        # As many causal as cross launches per pass: the mean of the two traced means.
        us = (p_causal["trace_mean_us"] + p_cross["trace_mean_us"]) / 2
        ach = bytes_per_launch / (us * 1e-6) / 1e9
        profile = {"source": "profiles/ rocprofv3 kernel-trace mean durations of verify_causal and verify_cross",
                   "us_per_launch": round(us, 3), "achieved": round(ach, 2), "frac": round(ach / PEAK_HBM_GBS, 4)}
    res = {
        "metric": "verification attention (8 drawn cache lengths x 32 layers x causal self + cross attention) "
                  "on 1 MI355X, HBM GB/s of algorithmic bytes",
        "value": round(gbs, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(tot["us"] / 1e3 / trials, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
        "data": "synthetic", "us_per_call": round(tot["us"] / (trials * 2 * layers), 3),
        "launch": "hip graph of each trial's pass (64 launches per copy of the K/V)",
        "tflops": round(tot["flops"] / (tot["us"] * 1e-6) / 1e12, 3),
        "per_trial": per_trial,
        "beam": {"value": round(tot["beam_bytes"] / (tot["beam_us"] * 1e-6) / 1e9, 2), "unit": "GB/s",
                 "us_per_call": round(tot["beam_us"] / (trials * layers), 3),
                 "bytes": "K/V rows of the union of the 5 ancestor sets + queries, outputs, mask words"},
        "config": {"workload": "speculative block verification: 16 queries, self caches L in "
                               f"{sorted(p['L'] for p in per_trial)}, cross 1500 encoder frames, 32 layers; "
                               "beam variant 5 queries on a token tree", "parallelism": "single GPU"},
        # Per launch on average (32 causal + 32 cross launches per pass); traffic is the
        # mean of the two kernels' measured HBM bytes per launch.
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "bytes_per_launch": bytes_per_launch, "timing": "HIP events around each trial's graph replay, this run",
                     "traffic": traffic, "profile": profile},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_verify(cross_cases, args.cpu_seconds)
    return res


def cpu_baseline_verify(cross_cases, budget_s):
    """The oracle on trial 0's layers (causal self-attention + cross-attention per layer) until
    the time budget is used; GB/s of the same algorithmic bytes."""
    import oracle
    from whisper_asr_encoder_amd import inputs as I
    threads = blas_threads()
    layers = len(cross_cases)
    done, nbytes, el = 0, 0, 0.0
    while done < 8 * layers and (done == 0 or el < budget_s):
        trial, layer = divmod(done, layers)
        sc = I.verify_self_case(trial, layer)
        cc = cross_cases[layer]
        t0 = time.perf_counter()
        oracle.verify_attention(sc.q, sc.k, sc.v, sc.mask)
        oracle.verify_attention(sc.q, cc.k, cc.v, None)
        el += time.perf_counter() - t0
        nbytes += sc.k.nbytes + sc.v.nbytes + cc.k.nbytes + cc.v.nbytes + 4 * sc.q.nbytes
        done += 1
    return {"value": round(nbytes / el / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {8 * layers} (trial, layer) pairs in trial order (causal self-attention over the "
                      f"trial's cache + cross-attention over 1500 frames), fp64 NumPy, {el:.1f} s",
            "us_per_call": round(el / (2 * done) * 1e6, 1), "cpu": cpu_model()}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="window", choices=["small", "window", "chunked", "batched", "verify", "encoder", "decoder",
                                                             "decoder_q8"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decoder-form", default="both", choices=["both", "stack", "layer"],
                    help="decoder workloads: time edda_decoder_verify_stack, per-layer calls, or both")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 256 MiB device-to-device copy (reference dispatch for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "edda runs on one GPU: --gpus must be 1 (sharding across GPUs is "
                                   "described in the design notes, not implemented)", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    from whisper_asr_encoder_amd import _lib
    _lib.load()
    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.workload == "verify":
        res = verify_bench(args, torch)
    elif args.workload == "encoder":
        res = full_encoder_bench(args, torch)
    elif args.workload in ("decoder", "decoder_q8"):
        res = decoder_bench(args, torch)
    else:
        cfg = {"small": 0, "window": 1, "chunked": 2, "batched": 3}[args.workload]
        res = encoder_bench(args, torch, cfg)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
