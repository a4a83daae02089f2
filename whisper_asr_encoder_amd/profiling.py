"""Summaries of rocprofv3 output for the encoder kernels (host-side text processing).

Reads the CSV files that `rocprofv3 --kernel-trace --stats` and two `rocprofv3 --pmc`
passes (FETCH_SIZE, then WRITE_SIZE) write, and produces

* per-kernel launch statistics (calls, mean / min / max duration),
* HBM traffic per launch: the median counter value per dispatch (KiB) scaled by the
  factor that makes the same counter read the true byte count of a plain device copy
  of known size in the same run (bench.py --calibrate-copy issues that copy),
* the median per dispatch of every counter in further --pmc runs, with derived figures:
  MFMA utilisation (SQ_VALU_MFMA_BUSY_CYCLES is the busy cycles of the 1024 SIMDs summed,
  one busy cycle per 1024 dense fp16 FLOP) against the nominal 2.4 GHz clock over the
  trace's mean duration, and rocprof's own MfmaUtil formula; the share of L2 read / write
  requests that go to DRAM (TCC_EA0_RDREQ_DRAM / TCC_EA0_RDREQ and the write pair) and the
  DRAM bytes they imply,
* beside the trace's mean, the per-launch time bench.py measured with HIP events on the same
  box (--bench-json: the JSON line of an untraced run, since under the tracer the eager
  launches become host-bound).

    python -m whisper_asr_encoder_amd.profiling TRACE_DIR FETCH_DIR WRITE_DIR OUT_DIR \
        --workload window|verify --command "<the rocprofv3 command lines>"

writes OUT_DIR/<kernel>_<workload>.md for each kernel of the workload and updates
OUT_DIR/traffic.json, keyed by the names bench.py reports (qkv_gemm, flash_attn, out_gemm;
verify_causal, verify_cross), each with the trace's mean duration and the digest of the kernel
sources the counters were taken on.
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
    "verify": ("block verification over the 8 drawn cache lengths (44-360 slots), 32 layers each: "
               "16-query causal blocks and 5-beam token trees (mask rows), cross-attention over 1500 "
               "frames (no mask)", {
        # Mask mode 0 (mask rows: causal blocks and beam trees), mode 1 (none: cross-attention).
        "verify_kernelILi0E|verify_kernel<0,": ("verify_causal", ["verify_attn.hip", "verify_core.hpp"]),
        "verify_kernelILi1E|verify_kernel<1,": ("verify_cross", ["verify_attn.hip", "verify_core.hpp"]),
    }),
    # The decoder verification pass: the single-launch layer kernel
    # (decoder_layer_kernel<self-attention chunks per wave, mask mode, Q8_0 weights>), launched
    # by edda_decoder_verify_stack for 8 layers at a time (bench --decoder-form stack), or once per
    # layer by edda_decoder_verify_layer (--decoder-form layer; the Q8_0 pass).
    "decoder": ("decoder verification pass, 32 layers, 16-token block, 360-slot cache, 1500 frames "
                "(edda_decoder_verify_stack: 4 launches of 8 layers)", {
        "decoder_layer_kernelILi2ELi0ELb0E|decoder_layer_kernel<2, 0, false>": ("decoder_layers_x8", ["decoder_fused.hip", "verify_core.hpp",
                                                                    "layer_norm_row.hpp"]),
    }),
    "decoder_q8": ("decoder verification pass with Q8_0 projection weights, 32 layers, 16-token block, "
                   "360-slot cache, 1500 frames (one launch per layer)", {
        "decoder_layer_kernelILi2ELi0ELb1E|decoder_layer_kernel<2, 0, true>": ("q8_decoder_layer", ["decoder_fused.hip", "verify_core.hpp",
                                                                   "layer_norm_row.hpp"]),
        "quantize_q8_0_kernel": ("quantize_q8_0 (setup, once per matrix)", ["skinny.hip"]),
    }),
    # The whole encoder: fc1 is the only 128x256-tile GEMM (N = 5120, GELU, no residual).
    "encoder": ("whole encoder of one 30 s window (stem, 32 pre-norm layers, final LayerNorm)", {
        "gemm_bias_kernelILi128ELi256E": ("fc1_gemm", ["gemm.hip"]),
        "layer_norm_kernelILi5E": ("layer_norm", ["norm_im2col.hip", "layer_norm_row.hpp"]),
        "im2col3_kernel": ("im2col3", ["norm_im2col.hip"]),
    }),
}

# Optional extra counter passes (rocprofv3 --pmc runs): every counter they hold is reported as
# its median per dispatch, and these combinations are derived when their counters are present.
COPY_KERNEL = "copyBuffer"
SIMDS = 1024            # 256 CUs x 4 SIMDs
FLOP_PER_BUSY = 1024    # fp16 dense MFMA FLOP per busy cycle of one SIMD
NOMINAL_GHZ = 2.4
XCDS = 8


def derived_lines(med, mean_ns):
    """Figures derived from the median counter values `med` of one kernel (see module doc)."""
    out = []
    busy = med.get("SQ_VALU_MFMA_BUSY_CYCLES")
    if busy is not None and mean_ns:
        util = busy / (SIMDS * NOMINAL_GHZ * mean_ns)
        out.append(("MFMA work executed (busy cycles x 1024 FLOP)", f"{busy * FLOP_PER_BUSY / 1e9:.3f} GFLOP"))
        out.append(("MfmaUtil at the nominal 2.4 GHz over the trace's mean duration "
                    "(busy / (1024 SIMDs x 2.4 GHz x duration))", f"{100 * util:.1f} %"))
        cu_cycles, wgs = med.get("SQ_BUSY_CU_CYCLES"), med.get("_workgroups")
        if cu_cycles and wgs:
            cus = min(wgs, SIMDS // 4)  # one workgroup per CU at most for these kernels
            per_cu = cu_cycles / cus
            out.append(("shader clock under this load (SQ_BUSY_CU_CYCLES / busy CUs / duration)",
                        f"{per_cu / mean_ns:.2f} GHz ({per_cu:.0f} cycles per busy CU)"))
            out.append(("MfmaUtil at that clock over the busy CUs' SIMDs (busy / (4 x busy CUs x cycles))",
                        f"{100 * busy / (4 * cus * per_cu):.1f} %"))
        gui = med.get("GRBM_GUI_ACTIVE")
        if gui:
            out.append(("rocprof's MfmaUtil formula, busy / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs) "
                        "(its counting window also holds the profiler's per-dispatch overhead)",
                        f"{100 * busy / (gui / XCDS * SIMDS):.1f} %"))
    rd, rq = med.get("TCC_EA0_RDREQ_DRAM"), med.get("TCC_EA0_RDREQ")
    if rd is not None and rq:
        n32, n128 = med.get("TCC_EA0_RDREQ_32B", 0.0), med.get("TCC_EA0_RDREQ_128B", 0.0)
        n64 = max(rq - n32 - n128, 0.0)
        avg = (32 * n32 + 64 * n64 + 128 * n128) / rq
        out.append(("L2 read requests to DRAM / all L2-to-fabric read requests", f"{rd:.0f} / {rq:.0f} "
                    f"({100 * rd / rq:.1f} %)"))
        out.append(("DRAM read bytes (DRAM requests x mean request size)", f"{rd * avg / 1e6:.2f} MB "
                    f"(mean request {avg:.0f} B)"))
    wd, wq = med.get("TCC_EA0_WRREQ_DRAM"), med.get("TCC_EA0_WRREQ")
    if wd is not None and wq:
        n64 = med.get("TCC_EA0_WRREQ_64B", 0.0)
        avg = (64 * n64 + 32 * max(wq - n64, 0.0)) / wq
        out.append(("L2 write requests to DRAM / all", f"{wd:.0f} / {wq:.0f} ({100 * wd / wq:.1f} %)"))
        out.append(("DRAM write bytes (DRAM requests x mean request size)", f"{wd * avg / 1e6:.2f} MB"))
    return out


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


def all_counters(pmc_dirs):
    """{counter: {kernel: [values per dispatch]}} over every counter in the given runs."""
    out = {}
    for d in pmc_dirs or []:
        with open(_one(os.path.join(d, "*counter_collection.csv"))) as f:
            for row in csv.DictReader(f):
                name = row["Counter_Name"].removesuffix("_sum")
                out.setdefault(name, {}).setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
                wgs = int(row["Grid_Size"]) // max(int(row["Workgroup_Size"]), 1)
                out.setdefault("_workgroups", {}).setdefault(row["Kernel_Name"], []).append(float(wgs))
    return out


def _has(name, fragment):
    """fragment: one or more '|'-separated pieces of a kernel's name as the trace records it
    (mangled, or demangled where the profiler could demangle it)."""
    return any(f in name for f in fragment.split("|"))


def _match(values, fragment):
    hits = [v for k, v in values.items() if _has(k, fragment)]
    return [x for h in hits for x in h]


def summarize(trace_dir, fetch_dir, write_dir, out_dir, command, workload="window", extra_dirs=None,
              bench_json=None):
    title, kernels = WORKLOADS[workload]
    extra = all_counters(extra_dirs)
    bench = None
    if bench_json:
        with open(bench_json) as f:
            lines = [ln for ln in f.read().splitlines() if ln.startswith("{")]
        bench = json.loads(lines[-1]) if lines else None
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
        st = [v for k, v in stats.items() if _has(k, frag)]
        fv, wv = _match(fetch, frag), _match(write, frag)
        if not st or not fv or not wv:
            continue
        # Every instantiation matching the fragment (e.g. the verification kernel's chunk and
        # wave counts, chosen by cache length) counts: calls-weighted mean over them.
        calls = sum(v["calls"] for v in st)
        s = {"calls": calls, "avg_ns": sum(v["avg_ns"] * v["calls"] for v in st) / calls,
             "min_ns": min(v["min_ns"] for v in st), "max_ns": max(v["max_ns"] for v in st)}
        fb = statistics.median(fv) * 1024.0 * f_scale
        wb = statistics.median(wv) * 1024.0 * w_scale
        digest = source_digest(srcs)
        traffic[key] = {"bytes_per_launch": round(fb + wb), "fetch_bytes": round(fb), "write_bytes": round(wb),
                        "trace_mean_us": round(s["avg_ns"] / 1e3, 3), "source_digest": digest}
        names = [k for k in stats if _has(k, frag)]
        with open(os.path.join(out_dir, f"{key}_{workload}.md"), "w") as f:
            f.write(f"# {key}: {title}\n\n")
            f.write("Kernel symbol" + ("s" if len(names) > 1 else "") + ": " +
                    ", ".join(f"`{n}` ({stats[n]['calls']} calls, {stats[n]['avg_ns'] / 1e3:.2f} us)" for n in names)
                    + "\n\n")
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
            med = {}
            for c, vals in sorted(extra.items()):
                v = _match(vals, frag)
                if v:
                    med[c] = statistics.median(v)
                    if not c.startswith("_"):
                        f.write(f"| {c} median per dispatch | {med[c]:.0f} |\n")
            for label, value in derived_lines(med, s["avg_ns"]):
                f.write(f"| {label} | {value} |\n")
            k = (bench or {}).get("kernels", {}).get(key) or {}
            if k.get("ms"):
                f.write(f"| bench.py on the same box (--bench-json), HIP events around back-to-back launches | "
                        f"{k['ms'] * 1e3:.2f} us per launch ({100 * (s['avg_ns'] / 1e3 / (k['ms'] * 1e3) - 1):+.1f} % "
                        f"trace vs events) |\n")
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
            st = [v for k, v in stats.items() if _has(k, frag)]
            if not st:
                continue
            calls = sum(v["calls"] for v in st)
            mean = sum(v["avg_ns"] * v["calls"] for v in st) / calls
            lo, hi = min(v["min_ns"] for v in st), max(v["max_ns"] for v in st)
            out[key] = {"calls": calls, "mean_us": round(mean / 1e3, 2)}
            shown = " or ".join(f"`{x}`" for x in frag.split("|"))
            f.write(f"| {key} | {shown} | {calls} | {mean / 1e3:.2f} us | {lo / 1e3:.2f} / {hi / 1e3:.2f} us |\n")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("trace_dir")
    ap.add_argument("fetch_dir", help="FETCH_SIZE run, or - for a kernel-trace-only summary")
    ap.add_argument("write_dir", help="WRITE_SIZE run, or -")
    ap.add_argument("out_dir")
    ap.add_argument("--command", required=True)
    ap.add_argument("--workload", default="window", choices=sorted(WORKLOADS))
    ap.add_argument("--extra-pmc", action="append", default=[],
                    help="directory of a further rocprofv3 --pmc run (repeatable)")
    ap.add_argument("--bench-json", default=None,
                    help="stdout of an untraced bench.py run of the same workload on the same box (its JSON line)")
    a = ap.parse_args()
    fetch = None if a.fetch_dir == "-" else a.fetch_dir
    write = None if a.write_dir == "-" else a.write_dir
    print(json.dumps(summarize(a.trace_dir, fetch, write, a.out_dir, a.command, a.workload, a.extra_pmc,
                               a.bench_json), indent=1))


if __name__ == "__main__":
    main()
