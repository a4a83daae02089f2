"""Summaries of rocprofv3 output for the encoder kernels (host-side text processing).

Reads the CSV files that `rocprofv3 --kernel-trace --stats` and two `rocprofv3 --pmc`
passes (FETCH_SIZE, then WRITE_SIZE) write, and produces

* per-kernel launch statistics (calls, mean / min / max duration),
* HBM traffic per launch: the median counter value per dispatch (KiB) scaled by the
  factor that makes the same counter read the true byte count of a plain device copy
  of known size in the same run (bench.py --calibrate-copy issues that copy).

    python -m whisper_asr_encoder_amd.profiling TRACE_DIR FETCH_DIR WRITE_DIR OUT_DIR \
        --workload window|verify --command "<the rocprofv3 command lines>"

writes OUT_DIR/<kernel>_<workload>.md for each kernel of the workload and updates
OUT_DIR/traffic.json, keyed by the names bench.py reports (qkv_gemm, flash_attn, out_gemm;
verify_causal, verify_cross), each with the digest of the kernel sources the counters were
taken on.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 256 << 20  # the calibration copy reads and writes this many bytes

# Per workload: kernel symbol fragment -> (report key, source files).  The window workload
# launches the 128x192 GEMM variant for the QKV projection (N = 3840) and the 128x64
# variant for the output projection (N = 1280); the verification pass launches the masked
# kernel for causal self-attention and the unmasked one for cross-attention.
WORKLOADS = {
    "window": ("one 30 s window (1500 frames), 32 attention sublayers", {
        "gemm_bias_kernelILi128ELi192E": ("qkv_gemm", ["gemm.hip"]),
        "flash_attn_kernel": ("flash_attn", ["flash_attn.hip"]),
        "gemm_bias_kernelILi128ELi64E": ("out_gemm", ["gemm.hip"]),
    }),
    "verify": ("block verification, 16 queries, 32 layers (causal self-attention over a "
               "360-slot cache, cross-attention over 1500 frames)", {
        # Mask mode 0 (mask rows: the causal self-attention), mode 1 (none: cross-attention).
        "verify_kernelILi0E": ("verify_causal", ["verify_attn.hip"]),
        "verify_kernelILi1E": ("verify_cross", ["verify_attn.hip"]),
    }),
    # The whole encoder: fc1 is the only 128x256-tile GEMM (N = 5120, GELU, no residual).
    # The decoder verification pass: block-sized GEMMs by fused variant (LayerNorm inside the
    # GEMM, cache append in the QKV epilogue, split K for the 1280-wide residual outputs).
    "decoder": ("decoder verification pass, 32 layers, 16-token block, 360-slot cache, 1500 frames", {
        # skinny_gemm_kernel<act, residual, LayerNorm, append, split K, Q8_0 weights>
        "skinny_gemm_kernelILi0ELb0ELb1ELb1ELb0ELb0E": ("ln_qkv_append", ["skinny.hip", "layer_norm_row.hpp"]),
        "skinny_gemm_kernelILi0ELb0ELb1ELb0ELb0ELb0E": ("ln_cross_query", ["skinny.hip", "layer_norm_row.hpp"]),
        "skinny_gemm_kernelILi1ELb0ELb1ELb0ELb0ELb0E": ("ln_fc1_gelu", ["skinny.hip", "layer_norm_row.hpp"]),
        "skinny_gemm_kernelILi0ELb1ELb0ELb0ELb1ELb0E": ("split_k_residual", ["skinny.hip"]),
        "verify_kernelILi0E": ("verify_self", ["verify_attn.hip"]),
        "verify_kernelILi1E": ("verify_cross", ["verify_attn.hip"]),
    }),
    # The same pass with Q8_0 projection weights (last template flag of the block GEMMs).
    "decoder_q8": ("decoder verification pass with Q8_0 projection weights, 32 layers, 16-token block, "
                   "360-slot cache, 1500 frames", {
        "skinny_gemm_kernelILi0ELb0ELb1ELb1ELb0ELb1E": ("q8_ln_qkv_append", ["skinny.hip", "layer_norm_row.hpp"]),
        "skinny_gemm_kernelILi0ELb0ELb1ELb0ELb0ELb1E": ("q8_ln_cross_query", ["skinny.hip", "layer_norm_row.hpp"]),
        "skinny_gemm_kernelILi1ELb0ELb1ELb0ELb0ELb1E": ("q8_ln_fc1_gelu", ["skinny.hip", "layer_norm_row.hpp"]),
        "skinny_gemm_kernelILi0ELb1ELb0ELb0ELb1ELb1E": ("q8_split_k_residual", ["skinny.hip"]),
        "quantize_q8_0_kernel": ("quantize_q8_0 (setup, once per matrix)", ["skinny.hip"]),
        "verify_kernelILi0E": ("verify_self", ["verify_attn.hip"]),
        "verify_kernelILi1E": ("verify_cross", ["verify_attn.hip"]),
    }),
    "encoder": ("whole encoder of one 30 s window (stem, 32 pre-norm layers, final LayerNorm)", {
        "gemm_bias_kernelILi128ELi256E": ("fc1_gemm", ["gemm.hip"]),
        "layer_norm_kernelILi5E": ("layer_norm", ["norm_im2col.hip", "layer_norm_row.hpp"]),
        "im2col3_kernel": ("im2col3", ["norm_im2col.hip"]),
    }),
}

# Optional extra counter pass (one rocprofv3 --pmc run): median per dispatch.
EXTRA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_F16",
                  "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_VALU_TRANS_F32")
COPY_KERNEL = "copyBuffer"


def source_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(HERE, "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _one(pattern):
    files = sorted(glob.glob(pattern))
    if not files:
        raise FileNotFoundError(pattern)
    return files[0]


def kernel_stats(trace_dir):
    out = {}
    with open(_one(os.path.join(trace_dir, "*kernel_stats.csv"))) as f:
        for row in csv.DictReader(f):
            out[row["Name"]] = {"calls": int(row["Calls"]), "avg_ns": float(row["AverageNs"]),
                                "min_ns": float(row["MinNs"]), "max_ns": float(row["MaxNs"])}
    return out


def counter_values(pmc_dir, counter):
    vals = {}
    with open(_one(os.path.join(pmc_dir, "*counter_collection.csv"))) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter:
                vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return vals


def _match(values, fragment):
    hits = [v for k, v in values.items() if fragment in k]
    return [x for h in hits for x in h]


def summarize(trace_dir, fetch_dir, write_dir, out_dir, command, workload="window", extra_dir=None):
    title, kernels = WORKLOADS[workload]
    extra = {c: counter_values(extra_dir, c) for c in EXTRA_COUNTERS} if extra_dir else {}
    stats = kernel_stats(trace_dir)
    if fetch_dir is None:  # kernel trace only
        return trace_only(stats, kernels, title, out_dir, command, workload)
    fetch = counter_values(fetch_dir, "FETCH_SIZE")
    write = counter_values(write_dir, "WRITE_SIZE")
    copy_f, copy_w = _match(fetch, COPY_KERNEL), _match(write, COPY_KERNEL)
    if not copy_f or not copy_w:
        raise RuntimeError("no calibration copy dispatch in the counter runs (run bench.py --calibrate-copy)")
    f_scale = COPY_BYTES / (max(copy_f) * 1024.0)
    w_scale = COPY_BYTES / (max(copy_w) * 1024.0)
    os.makedirs(out_dir, exist_ok=True)
    tpath = os.path.join(out_dir, "traffic.json")
    traffic = {}
    if os.path.exists(tpath):
        with open(tpath) as f:
            traffic = json.load(f)
    traffic["_method"] = (f"median per-dispatch FETCH_SIZE x {f_scale:.3f} + WRITE_SIZE x {w_scale:.3f} "
                           f"(KiB -> bytes; factors make a {COPY_BYTES >> 20} MiB device copy read its "
                           "true size)")
    for frag, (key, srcs) in kernels.items():
        st = [v for k, v in stats.items() if frag in k]
        fv, wv = _match(fetch, frag), _match(write, frag)
        if not st or not fv or not wv:
            continue
        s = st[0]
        fb = statistics.median(fv) * 1024.0 * f_scale
        wb = statistics.median(wv) * 1024.0 * w_scale
        digest = source_digest(srcs)
        traffic[key] = {"bytes_per_launch": round(fb + wb), "fetch_bytes": round(fb), "write_bytes": round(wb),
                        "source_digest": digest}
        name = [k for k in stats if frag in k][0]
        with open(os.path.join(out_dir, f"{key}_{workload}.md"), "w") as f:
            f.write(f"# {key}: {title}\n\n")
            f.write(f"Kernel symbol: `{name}`\n\n")
            f.write("Commands (run from the repository root on one MI355X):\n\n```\n" + command.strip() + "\n```\n\n")
            f.write("| figure | value |\n|---|---|\n")
            f.write(f"| dispatches in the trace run | {s['calls']} |\n")
            f.write(f"| mean duration | {s['avg_ns'] / 1e3:.2f} us |\n")
            f.write(f"| min / max duration | {s['min_ns'] / 1e3:.2f} / {s['max_ns'] / 1e3:.2f} us |\n")
            f.write(f"| FETCH_SIZE median per dispatch | {statistics.median(fv):.0f} KiB (x {f_scale:.3f}) |\n")
            f.write(f"| WRITE_SIZE median per dispatch | {statistics.median(wv):.0f} KiB (x {w_scale:.3f}) |\n")
            f.write(f"| HBM bytes per launch (scaled) | {(fb + wb) / 1e6:.2f} MB "
                    f"(read {fb / 1e6:.2f}, write {wb / 1e6:.2f}) |\n")
            f.write(f"| kernel sources digest | {digest} |\n")
            for c, vals in extra.items():
                v = _match(vals, frag)
                if v:
                    f.write(f"| {c} median per dispatch | {statistics.median(v):.0f} |\n")
    with open(tpath, "w") as f:
        json.dump(traffic, f, indent=1)
        f.write("\n")
    return traffic


def trace_only(stats, kernels, title, out_dir, command, workload):
    """One summary file for a workload profiled with the kernel trace alone."""
    os.makedirs(out_dir, exist_ok=True)
    out = {}
    with open(os.path.join(out_dir, f"{workload}_kernels.md"), "w") as f:
        f.write(f"# kernels of the {title}\n\n")
        f.write("Commands (run from the repository root on one MI355X):\n\n```\n" + command.strip() + "\n```\n\n")
        f.write("| kernel | symbol fragment | dispatches | mean | min / max |\n|---|---|---|---|---|\n")
        for frag, (key, _) in kernels.items():
            st = [v for k, v in stats.items() if frag in k]
            if not st:
                continue
            calls = sum(v["calls"] for v in st)
            mean = sum(v["avg_ns"] * v["calls"] for v in st) / calls
            lo, hi = min(v["min_ns"] for v in st), max(v["max_ns"] for v in st)
            out[key] = {"calls": calls, "mean_us": round(mean / 1e3, 2)}
            f.write(f"| {key} | `{frag}` | {calls} | {mean / 1e3:.2f} us | {lo / 1e3:.2f} / {hi / 1e3:.2f} us |\n")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("trace_dir")
    ap.add_argument("fetch_dir", help="FETCH_SIZE run, or - for a kernel-trace-only summary")
    ap.add_argument("write_dir", help="WRITE_SIZE run, or -")
    ap.add_argument("out_dir")
    ap.add_argument("--command", required=True)
    ap.add_argument("--workload", default="window", choices=sorted(WORKLOADS))
    ap.add_argument("--extra-pmc", default=None, help="directory of a rocprofv3 --pmc run of EXTRA_COUNTERS")
    a = ap.parse_args()
    fetch = None if a.fetch_dir == "-" else a.fetch_dir
    write = None if a.write_dir == "-" else a.write_dir
    print(json.dumps(summarize(a.trace_dir, fetch, write, a.out_dir, a.command, a.workload, a.extra_pmc),
                     indent=1))


if __name__ == "__main__":
    main()
