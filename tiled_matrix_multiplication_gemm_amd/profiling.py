"""Summaries of rocprofv3 output for the GEMM kernels.

  python -m tiled_matrix_multiplication_gemm_amd.profiling trace  <kernel_stats.csv> <out.txt> --cmd "..." [--last N]
  python -m tiled_matrix_multiplication_gemm_amd.profiling traffic <fetch_dir> <write_dir> <out.txt> --cmd "..."
  python -m tiled_matrix_multiplication_gemm_amd.profiling counters <out.txt> <dir>... --cmd "..."

`trace` condenses a `--kernel-trace --stats` run (per-kernel calls and mean
duration).  `traffic` turns two `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs
of `bench.py --pmc-probe` into HBM bytes per GEMM dispatch: the probe runs a
plain elementwise copy of a known size in the same process, and the counter
readings of the GEMM are scaled by (known bytes / counter reading) of that
copy.  The summary records a hash of the kernel sources; bench.py reports the
traffic only while that hash matches the current sources.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import time

PKG = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 256 * 1024 * 1024  # bytes read and bytes written by the probe's copy kernel
SIMDS = 256 * 4                 # MI355X: 256 CUs of 4 SIMDs
SHADER_ENGINES = 32             # 8 XCDs of 4 shader engines


def source_hash() -> str:
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(PKG, "csrc", "*.h")) + glob.glob(os.path.join(PKG, "csrc", "*.hip"))):
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_summary(path: str) -> dict:
    out = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                out[k.strip()] = v.strip()
    return out


def _counter_rows(d: str):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError("no counter_collection.csv under %s" % d)
    rows = []
    for fn in files:
        with open(fn) as f:
            rows += list(csv.DictReader(f))
    return rows


def _per_dispatch(rows, counter: str):
    """{dispatch id: (kernel name, summed counter value)}"""
    acc = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        k = int(r["Dispatch_Id"])
        name, v = acc.get(k, (r["Kernel_Name"], 0.0))
        acc[k] = (name, v + float(r["Counter_Value"]))
    return acc


def traffic(fetch_dir: str, write_dir: str, kernel_key: str = "gemm_") -> dict:
    res = {}
    for label, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        disp = _per_dispatch(_counter_rows(d), counter)
        gemm = [(k, v) for k, v in sorted(disp.items()) if kernel_key in v[0]]
        copies = [(k, v) for k, v in sorted(disp.items()) if kernel_key not in v[0]]
        if not gemm or not copies:
            raise RuntimeError("need both a GEMM and a copy dispatch in %s" % d)
        g_name, g_kib = gemm[-1][1]
        c_name, c_kib = max((v for _, v in copies), key=lambda t: t[1])
        factor = COPY_BYTES / (c_kib * 1024.0)
        res[label] = dict(kernel=g_name, kib=g_kib, copy_kernel=c_name, copy_kib=c_kib, factor=factor,
                          bytes=g_kib * 1024.0 * factor)
    return res


def write_traffic(fetch_dir, write_dir, out, cmd):
    t = traffic(fetch_dir, write_dir)
    total = t["fetch"]["bytes"] + t["write"]["bytes"]
    with open(out, "w") as f:
        f.write("# HBM traffic of one GEMM dispatch (rocprofv3 FETCH_SIZE / WRITE_SIZE, copy-calibrated)\n")
        f.write("# commands:\n")
        for c in cmd:
            f.write("#   %s\n" % c)
        f.write("kernel = %s\n" % t["fetch"]["kernel"])
        for lab in ("fetch", "write"):
            f.write("%s_kib_raw = %.1f\n" % (lab, t[lab]["kib"]))
            f.write("%s_copy_kib_raw = %.1f   (copy of %d bytes: %s)\n" % (lab, t[lab]["copy_kib"], COPY_BYTES,
                                                                     t[lab]["copy_kernel"][:60]))
            f.write("%s_scale = %.4f\n" % (lab, t[lab]["factor"]))
            f.write("%s_bytes = %.0f\n" % (lab, t[lab]["bytes"]))
        f.write("traffic_bytes = %.0f\n" % total)
        f.write("source_hash = %s\n" % source_hash())
    return total


def write_counters(dirs, out, cmd, kernel_key: str = "gemm_"):
    """Counter values of the last GEMM dispatch of each run, plus the derived
    MFMA-busy and LDS bank-conflict ratios and the L2 hit rate."""
    vals = {}
    for d in dirs:
        rows = _counter_rows(d)
        ids = sorted({int(r["Dispatch_Id"]) for r in rows if kernel_key in r["Kernel_Name"]})
        for r in rows:
            if int(r["Dispatch_Id"]) == ids[-1]:
                vals[r["Counter_Name"]] = vals.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    with open(out, "w") as f:
        f.write("# rocprofv3 --pmc counters of one GEMM dispatch (summed over all instances)\n")
        f.write("# commands:\n")
        for c in cmd:
            f.write("#   %s\n" % c)
        f.write("# source_hash = %s\n" % source_hash())
        for k in sorted(vals):
            f.write("%s = %.6g\n" % (k, vals[k]))
        if "SQ_INSTS_MFMA" in vals and "SQ_VALU_MFMA_BUSY_CYCLES" in vals:
            f.write("mfma_busy_cycles_per_instruction = %.2f\n" % (vals["SQ_VALU_MFMA_BUSY_CYCLES"] / vals["SQ_INSTS_MFMA"]))
        if "SQ_VALU_MFMA_BUSY_CYCLES" in vals and "SQ_BUSY_CYCLES" in vals:
            # MFMA busy cycles are summed over the 1024 SIMDs, SQ busy cycles
            # over the 32 shader engines: the ratio of the per-unit means is
            # the fraction of the kernel's cycles the matrix cores were busy
            f.write("mfma_busy_fraction = %.4f\n" % ((vals["SQ_VALU_MFMA_BUSY_CYCLES"] / SIMDS) /
                                                     (vals["SQ_BUSY_CYCLES"] / SHADER_ENGINES)))
        if "SQ_LDS_BANK_CONFLICT" in vals and "SQ_LDS_IDX_ACTIVE" in vals:
            f.write("lds_bank_conflict_ratio = %.4f\n" % (vals["SQ_LDS_BANK_CONFLICT"] / max(vals["SQ_LDS_IDX_ACTIVE"], 1)))
        if "TCC_HIT_sum" in vals and "TCC_MISS_sum" in vals:
            f.write("l2_hit_rate = %.4f\n" % (vals["TCC_HIT_sum"] / (vals["TCC_HIT_sum"] + vals["TCC_MISS_sum"])))
    return vals


def write_trace(stats_csv, out, cmd, last=0):
    """Per-kernel calls and mean duration from the --stats summary; with
    `last`, also the mean over the last `last` dispatches of each kernel from
    the kernel trace beside it (the timed calls, without the warm-up ones,
    whose first call includes loading the code object)."""
    with open(stats_csv) as f:
        rows = list(csv.DictReader(f))
    timed = {}
    trace_csv = stats_csv.replace("kernel_stats.csv", "kernel_trace.csv")
    if last > 0 and os.path.exists(trace_csv):
        per = {}
        with open(trace_csv) as f:
            for r in csv.DictReader(f):
                per.setdefault(r["Kernel_Name"], []).append(
                    (int(r["Dispatch_Id"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
        for name, v in per.items():
            d = [ns for _, ns in sorted(v)][-last:]
            timed[name] = (len(d), sum(d) / len(d))
    with open(out, "w") as f:
        f.write("# rocprofv3 --kernel-trace --stats summary\n")
        f.write("# command: %s\n" % cmd)
        f.write("# source_hash = %s\n" % source_hash())
        f.write("%-100s %6s %14s %12s %18s\n" % ("kernel", "calls", "mean_ns", "pct", "mean_ns_timed"))
        for r in rows:
            t = timed.get(r["Name"])
            tt = "%.1f (last %d)" % (t[1], t[0]) if t else "-"
            f.write("%-100s %6s %14.1f %12s %18s\n" % (r["Name"][:100], r["Calls"], float(r["AverageNs"]),
                                                        r["Percentage"], tt))


def soak_telemetry(fn, seconds: float = 1.6, with_rate: bool = False):
    """Graphics and memory clocks, socket power and hotspot temperature while
    `fn` runs back to back.

    Sampled through amdsmi on a background thread during a soak that follows
    the timed region (never inside it).  The driver's metrics table trails
    the hardware by up to about a second, so only samples from the second
    half of the soak are kept.  Returns None where amdsmi is unavailable."""
    import statistics
    import threading

    import torch

    try:
        import amdsmi

        amdsmi.amdsmi_init()
    except Exception:
        return None
    try:
        handles = amdsmi.amdsmi_get_processor_handles()
        if len(handles) != 1:
            return None
        h = handles[0]
        limit_w = None
        try:
            limit_w = float(amdsmi.amdsmi_get_power_info(h)["power_limit"]) / 1e6  # reported in microwatts
        except Exception:
            pass
        samples = []
        stop = threading.Event()

        def sample():
            while not stop.is_set():
                try:
                    m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                    clks = [v for v in (m.get("current_gfxclks") or [m.get("current_gfxclk")])
                            if isinstance(v, (int, float)) and 0 < v < 65535]
                    pw = m.get("current_socket_power")
                    uclk = m.get("current_uclk")
                    hot = m.get("temperature_hotspot")
                    samples.append((time.perf_counter(), sum(clks) / len(clks) if clks else None,
                                    float(pw) if isinstance(pw, (int, float)) and pw < 65535 else None,
                                    float(uclk) if isinstance(uclk, (int, float)) and 0 < uclk < 65535 else None,
                                    float(hot) if isinstance(hot, (int, float)) and 0 < hot < 65535 else None))
                except Exception:
                    pass
                time.sleep(0.02)

        th = threading.Thread(target=sample, daemon=True)
        th.start()
        t0 = time.perf_counter()
        calls = 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(16):
                fn()
            calls += 16
            torch.cuda.synchronize()
        t1 = time.perf_counter()
        stop.set()
        th.join()
        keep = [x for x in samples if x[0] >= t0 + (t1 - t0) / 2]
        clk = [x[1] for x in keep if x[1] is not None]
        pw = [x[2] for x in keep if x[2] is not None]
        uclk = [x[3] for x in keep if x[3] is not None]
        hot = [x[4] for x in keep if x[4] is not None]
        res = {"gfx_clock_mhz": round(statistics.median(clk), 1) if clk else None,
               "mem_clock_mhz": round(statistics.median(uclk), 1) if uclk else None,
               "socket_power_w": round(statistics.median(pw), 1) if pw else None,
               "hotspot_c": round(statistics.median(hot), 1) if hot else None,
               "power_limit_w": limit_w, "samples": len(keep), "soak_s": round(t1 - t0, 2)}
        if with_rate:
            res["ms_per_call"] = (t1 - t0) * 1e3 / calls
        return res
    except Exception:
        return None
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("trace")
    a.add_argument("stats_csv")
    a.add_argument("out")
    a.add_argument("--cmd", required=True)
    a.add_argument("--last", type=int, default=0, help="also average the last N dispatches (the timed calls)")
    b = sub.add_parser("traffic")
    b.add_argument("fetch_dir")
    b.add_argument("write_dir")
    b.add_argument("out")
    b.add_argument("--cmd", action="append", required=True)
    c = sub.add_parser("counters")
    c.add_argument("out")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--cmd", action="append", required=True)
    args = ap.parse_args()
    if args.what == "counters":
        write_counters(args.dirs, args.out, args.cmd)
    elif args.what == "trace":
        write_trace(args.stats_csv, args.out, args.cmd, args.last)
    else:
        print(write_traffic(args.fetch_dir, args.write_dir, args.out, args.cmd))


if __name__ == "__main__":
    main()
