"""Summarise rocprofv3 output for the attention kernel into short text/JSON
files under ``profiles/``.

    python -m exact_tiled_attention_04_amd.profiling \\
        --workload causal_8k --trace DIR [--fetch DIR --write DIR --copy-mib 1024] \\
        [--pmc DIR ...] --command "..." [--last N]

--trace   a ``rocprofv3 --kernel-trace --stats`` output directory
--fetch / --write
          ``rocprofv3 --pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` output
          directories of a run that also copied ``--copy-mib`` MiB device to
          device; the copy's own counter value (bytes known) calibrates the
          counter: bytes = counter_KiB * 1024 * (copy bytes / copy counter bytes)
--pmc     further counter-collection directories (SQ_*/GRBM_* counters), summed
          per dispatch of the attention kernel
--last    use only the last N dispatches of the kernel (the timed steps)
--kernel  substring selecting the kernel (default: the forward, "fwd_";
          "fwd_fp8" with --fp8 for the FP8 forward)
--peak    TFLOP/s the algorithmic FLOPs are priced against (default 2516.6)
--bytes   algorithmic bytes per launch, for HBM-bound kernels (priced
          against 8000 GB/s)
--name    output base name (default: fwd_<workload>; the traffic JSON that
          bench.py reads is written only for the forward)
--note    a paragraph appended to the summary (repeatable)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_KEY = "fwd_"


# sources each forward kernel is compiled from (its launch, host code aside)
FWD_SOURCES = ("fa_fwd_mfma.hip", "fa_mfma_common.h", "fa_internal.h")
FP8_SOURCES = ("fa_fwd_fp8.hip", "fa_mfma_common.h", "fa_internal.h")
F32_SOURCES = ("fa_fwd_f32.hip", "fa_internal.h")
BWD_SOURCES = ("fa_bwd_mfma.hip", "fa_mfma_common.h", "fa_internal.h")
DECODE_SOURCES = ("fa_decode.hip", "fa_decode.h", "fa_mfma_common.h", "fa_internal.h")


def sources_of(kernel_key: str, fp8: bool = False):
    """The source files of the kernel a --kernel substring selects."""
    if fp8 or "fp8" in kernel_key:
        return FP8_SOURCES
    if "bwd" in kernel_key:
        return BWD_SOURCES
    if "decode" in kernel_key:
        return DECODE_SOURCES
    if "f32" in kernel_key:
        return F32_SOURCES
    return FWD_SOURCES


def kernel_source_hash(sources=FWD_SOURCES) -> str:
    """sha256 over a kernel's sources (sorted by name): a stored traffic
    measurement stays valid while these are unchanged."""
    csrc = os.path.join(ROOT, "exact_tiled_attention_04_amd", "csrc")
    h = hashlib.sha256()
    for fn in sorted(sources):
        h.update(fn.encode())
        h.update(open(os.path.join(csrc, fn), "rb").read())
    return h.hexdigest()


def _csv(d, suffix):
    files = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return list(csv.DictReader(open(files[0])))


def _is_attn(name):
    return KERNEL_KEY in name and "fa::" in name


def trace_summary(d, last=None):
    rows = [r for r in _csv(d, "kernel_trace.csv") if _is_attn(r["Kernel_Name"])]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) for r in rows]
    if last:
        durs = durs[-last:]
    return {"kernel": rows[0]["Kernel_Name"] if rows else None, "dispatches": len(durs),
            "avg_us": statistics.mean(durs) / 1e3 if durs else None,
            "min_us": min(durs) / 1e3 if durs else None, "max_us": max(durs) / 1e3 if durs else None,
            "grid": rows[0].get("Grid_Size_X") if rows else None,
            "workgroup": rows[0].get("Workgroup_Size_X") if rows else None,
            "lds_bytes": rows[0].get("LDS_Block_Size") if rows else None,
            "vgpr": rows[0].get("VGPR_Count") if rows else None,
            "agpr": rows[0].get("Accum_VGPR_Count") if rows else None}


def stats_summary(d):
    """The kernel's row of rocprofv3's --stats table (every dispatch, warm-up
    included), or None when the run wrote none."""
    try:
        rows = _csv(d, "kernel_stats.csv")
    except FileNotFoundError:
        return None
    for r in rows:
        if _is_attn(r["Name"]):
            return {"calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
                    "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3}
    return None


def counter_per_dispatch(d, last=None):
    """{counter: [value per dispatch]} for the attention kernel, plus the copy
    kernel: only the calibration copy's dispatches (those with the largest
    grid among the copies; a run may hold other, small copies, whose counts
    would dilute the factor)."""
    rows = _csv(d, "counter_collection.csv")
    copy_grids = [int(r.get("Grid_Size") or 0) for r in rows if "copyBuffer" in r["Kernel_Name"]]
    big = max(copy_grids, default=0)
    attn, copy = {}, {}
    for r in rows:
        name = r["Kernel_Name"]
        is_cal = "copyBuffer" in name and int(r.get("Grid_Size") or 0) == big
        target = attn if _is_attn(name) else copy if is_cal else None
        if target is None:
            continue
        key = (r["Dispatch_Id"], r["Counter_Name"])
        target[key] = target.get(key, 0.0) + float(r["Counter_Value"])
    def regroup(m):
        out = {}
        for (disp, cname), val in sorted(m.items(), key=lambda kv: int(kv[0][0])):
            out.setdefault(cname, []).append(val)
        return out
    a = regroup(attn)
    if last:
        a = {k: v[-last:] for k, v in a.items()}
    return a, regroup(copy)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-mib", type=int, default=0)
    ap.add_argument("--pmc", nargs="*", default=[])
    ap.add_argument("--command", action="append", default=[])
    ap.add_argument("--last", type=int, default=None)
    ap.add_argument("--kernel", default="fwd_")
    ap.add_argument("--name", default=None)
    ap.add_argument("--flops", type=float, default=None, help="algorithmic FLOPs per launch")
    ap.add_argument("--peak", type=float, default=2516.6, help="peak TFLOP/s the FLOPs are priced against")
    ap.add_argument("--bytes", type=float, default=None,
                    help="algorithmic bytes per launch (HBM-bound kernels), priced against 8000 GB/s")
    ap.add_argument("--fp8", action="store_true", help="the FP8 forward kernel (its sources for the hash)")
    ap.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--note", action="append", default=[], help="a paragraph appended to the summary")
    args = ap.parse_args()
    global KERNEL_KEY
    KERNEL_KEY = args.kernel
    forward = args.kernel in ("fwd_", "fwd_fp8", "fwd_f32")
    sources = sources_of(args.kernel, args.fp8)
    name = args.name or f"fwd_{args.workload}"

    tr = trace_summary(args.trace, args.last)
    title = "attention forward kernel" if forward else f"attention kernel matching '{args.kernel}'"
    lines = [f"# {title}, workload {args.workload}", "",
             "Commands (run from the repository root on one MI355X):", ""]
    lines += [f"    {c}" for c in args.command]
    lines += ["", f"kernel: `{tr['kernel']}`",
              f"grid {tr['grid']} work-items, workgroup {tr['workgroup']}, LDS {tr['lds_bytes']} B, "
              f"trace fields VGPR_Count {tr['vgpr']}, Accum_VGPR_Count {tr['agpr']} (the compiler's resource report is the authority on register use)", "",
              f"kernel trace, last {tr['dispatches']} dispatches: avg {tr['avg_us']:.1f} us, "
              f"min {tr['min_us']:.1f} us, max {tr['max_us']:.1f} us"]
    st = stats_summary(args.trace)
    if st:
        lines.append(f"rocprofv3 --stats, all {st['calls']} dispatches (warm-up included): avg {st['avg_us']:.1f} us, "
                     f"min {st['min_us']:.1f} us, max {st['max_us']:.1f} us")
    if args.flops:
        lines.append(f"algorithmic FLOPs per launch {args.flops:.4e} -> {args.flops / (tr['avg_us'] * 1e-6) / 1e12:.1f} "
                     f"TFLOP/s at the average duration ({100 * args.flops / (tr['avg_us'] * 1e-6) / (args.peak * 1e12):.1f}% "
                     f"of {args.peak} TFLOP/s)")
    if args.bytes:
        gbs = args.bytes / (tr['avg_us'] * 1e-6) / 1e9
        lines.append(f"algorithmic bytes per launch {args.bytes:.4e} -> {gbs:.1f} GB/s at the average duration "
                     f"({100 * gbs / 8000:.1f}% of 8000 GB/s)")
    traffic = None
    if args.fetch and args.write and args.copy_mib:
        copy_bytes = args.copy_mib * 2 ** 20
        fa_f, cp_f = counter_per_dispatch(args.fetch, args.last)
        fa_w, cp_w = counter_per_dispatch(args.write, args.last)
        f_scale = copy_bytes / (statistics.mean(cp_f["FETCH_SIZE"]) * 1024)
        w_scale = copy_bytes / (statistics.mean(cp_w["WRITE_SIZE"]) * 1024)
        fetch_b = statistics.mean(fa_f["FETCH_SIZE"]) * 1024 * f_scale
        write_b = statistics.mean(fa_w["WRITE_SIZE"]) * 1024 * w_scale
        traffic = fetch_b + write_b
        lines += ["", "HBM traffic per launch (counters in KiB per dispatch, scaled by a device copy of "
                  f"{args.copy_mib} MiB measured in the same run):",
                  f"  FETCH_SIZE: copy reads {statistics.mean(cp_f['FETCH_SIZE']):.0f} KiB for "
                  f"{copy_bytes // 1024} KiB -> factor {f_scale:.4f}; kernel {statistics.mean(fa_f['FETCH_SIZE']):.0f} KiB "
                  f"-> {fetch_b / 2**20:.1f} MiB read",
                  f"  WRITE_SIZE: copy writes {statistics.mean(cp_w['WRITE_SIZE']):.0f} KiB for "
                  f"{copy_bytes // 1024} KiB -> factor {w_scale:.4f}; kernel {statistics.mean(fa_w['WRITE_SIZE']):.0f} KiB "
                  f"-> {write_b / 2**20:.1f} MiB written",
                  f"  total {traffic / 2**20:.1f} MiB per launch"]
        if forward:
            json.dump({"workload": args.workload, "kernel_source_sha256": kernel_source_hash(sources),
                       "hbm_bytes_per_launch": round(traffic), "fetch_bytes": round(fetch_b),
                       "write_bytes": round(write_b), "fetch_scale": f_scale, "write_scale": w_scale,
                       "commands": args.command},
                      open(os.path.join(args.out_dir, f"traffic_{args.workload}.json"), "w"), indent=1)
    for d in args.pmc:
        a, _ = counter_per_dispatch(d, args.last)
        lines += ["", f"counters ({os.path.basename(os.path.normpath(d))}), mean per dispatch:"]
        for k, v in sorted(a.items()):
            lines.append(f"  {k:34s} {statistics.mean(v):.6g}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in a and "GRBM_GUI_ACTIVE" in a:
            # GRBM_GUI_ACTIVE comes back summed over the 8 XCDs: one XCD's
            # count is the kernel's duration in GPU clocks
            simd = 256 * 4
            gui = statistics.mean(a["GRBM_GUI_ACTIVE"]) / 8
            util = statistics.mean(a["SQ_VALU_MFMA_BUSY_CYCLES"]) / (gui * simd)
            lines.append(f"  MFMA busy cycles / (GPU-active cycles per XCD x 1024 SIMDs) = {100 * util:.1f}%")
        for mops in ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU_MFMA_MOPS_F8"):
            if mops in a:
                # the counter is in units of 512 FLOPs of MFMA work
                mf = statistics.mean(a[mops]) * 512
                util = mf / (tr["avg_us"] * 1e-6) / (args.peak * 1e12)
                lines.append(f"  MFMA FLOPs from {mops} x 512 = {mf:.4e} per launch -> {100 * util:.1f}% of "
                             f"{args.peak} TFLOP/s over the trace's average duration")
        if "TCC_HIT_sum" in a and "TCC_MISS_sum" in a:
            hit, miss = statistics.mean(a["TCC_HIT_sum"]), statistics.mean(a["TCC_MISS_sum"])
            lines.append(f"  L2 hit rate TCC_HIT / (TCC_HIT + TCC_MISS) = {100 * hit / max(1.0, hit + miss):.1f}%")
        if "SQ_LDS_BANK_CONFLICT" in a and "SQ_LDS_IDX_ACTIVE" in a:
            bc = statistics.mean(a["SQ_LDS_BANK_CONFLICT"]) / max(1.0, statistics.mean(a["SQ_LDS_IDX_ACTIVE"]))
            lines.append(f"  LDS bank-conflict cycles / LDS active cycles = {100 * bc:.2f}%")
    for note in args.note:
        lines += ["", note]
    lines.append(f"\nkernel sources sha256 {kernel_source_hash(sources)}")
    out = os.path.join(args.out_dir, f"{name}.md")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
