"""Summaries of rocprofv3 output for the profiles/ folder.

    python -m exact_scaled_dot_sdpa_amd.profiling stats KERNEL_STATS_CSV --cmd "..." --out FILE.md \
        [--trace KERNEL_TRACE_CSV --last N]
    python -m exact_scaled_dot_sdpa_amd.profiling traffic --fetch FETCH_CSV --write WRITE_CSV \
        --calib-mib 512 --cmd-fetch "..." --cmd-write "..." --json profiles/traffic.json --out FILE.md

`stats` condenses a `rocprofv3 --kernel-trace --stats -f csv` kernel_stats file
into a short table.  `traffic` turns two `rocprofv3 --pmc FETCH_SIZE` /
`--pmc WRITE_SIZE` counter files (KiB per dispatch) into HBM bytes per launch:
each counter is scaled by the factor that makes the plain device copy of
--calib-mib MiB (launched by `bench.py --calib-copy-mib`) read and write
exactly that many bytes.  The JSON records each kernel's source digest;
bench.py reports a kernel's bytes only while its sources are unchanged.
"""
import argparse
import csv
import json
import os
import re
import statistics
import sys

KERNELS = {
    # logical kernel -> substrings of the dispatched kernel names that make one launch
    "prefill": ["prefill_bf16_kernel"],
    "decode": ["decode_chunk_kernel", "decode_merge_kernel"],
    "bwd": ["bwd_pre_kernel", "bwd_dq_kernel", "bwd_dkdv_kernel"],
    "fp8": ["prefill_fp8_kernel"],
}
COPY_KERNEL = "copyBuffer"


def _short(name):
    """The kernel's own identifier: the length-prefixed name after the
    namespaces of an Itanium-mangled symbol, or the function name of a
    demangled one."""
    m = re.match(r"_ZN(?:\d+attn)?(?:12_GLOBAL__N_1)?(\d+)", name)
    if m:
        n = int(m.group(1))
        return name[m.end():m.end() + n]
    m = re.search(r"(\w+)<", name)
    if m:
        return m.group(1)
    return name[:60]


def _targs(name):
    """The integer / bool template arguments of an Itanium-mangled kernel
    name, as "<64,true,8>", or "" when it has none."""
    short = _short(name)
    i = name.find(short)
    if not name.startswith("_Z") or i < 0 or name[i + len(short):i + len(short) + 1] != "I":
        return ""
    args = re.findall(r"L([ib])(n?\d+)E", name[i + len(short):].split("EE", 1)[0] + "E")
    return "<%s>" % ",".join(("true" if v == "1" else "false") if t == "b" else v.replace("n", "-")
                              for t, v in args)


def _labels(names):
    """Short names; where several kernels share one, each with its template
    arguments."""
    shorts = [_short(n) for n in names]
    return {n: s + (_targs(n) if shorts.count(s) > 1 else "") for n, s in zip(names, shorts)}


def _last_n(trace_csv, n):
    """(dispatches, median us, mean us) of the last n dispatches of each
    kernel in a rocprofv3 kernel_trace csv (the timed steps, after the
    warm-up ones)."""
    per = {}
    for r in csv.DictReader(open(trace_csv)):
        per.setdefault(r["Kernel_Name"], []).append(
            (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    res = {}
    for name, v in per.items():
        v.sort()
        last = [d for _, d in v[-n:]]
        res[name] = (len(last), statistics.median(last) / 1e3, sum(last) / len(last) / 1e3)
    return res


def stats(path, cmd, out, trace=None, last=0):
    rows = list(csv.DictReader(open(path)))
    label = _labels([r["Name"] for r in rows])
    lines = ["# rocprofv3 kernel statistics", "", "Command:", "", "```", cmd, "```", "",
             "| kernel | calls | avg (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append("| %s | %s | %.2f | %.2f | %.2f | %.2f%% |" % (
            label[r["Name"]], r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    if trace and last > 0:
        timed = _last_n(trace, last)
        lines += ["", "The last %d dispatches of each kernel (the timed steps; the table above also counts the "
                      "warm-up dispatches), from the kernel trace: the median is the primary figure, the mean "
                      "the one the bench line's HIP events compare with:" % last, "",
                  "| kernel | dispatches | median (us) | mean (us) |", "|---|---|---|---|"]
        tl = _labels(list(timed))
        for name, (cnt, med, avg) in sorted(timed.items(), key=lambda kv: -kv[1][2]):
            lines.append("| %s | %d | %.2f | %.2f |" % (tl[name], cnt, med, avg))
    lines += ["", "Full kernel names:", ""] + ["- `%s`" % r["Name"] for r in rows]
    text = "\n".join(lines) + "\n"
    with open(out, "w") as f:
        f.write(text)
    return text


def _per_dispatch(path, counter):
    res = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        res.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return res


def _calib(values, calib_kib):
    # the copy of calib_kib KiB is the largest copyBuffer dispatch
    cands = [v for name, vs in values.items() if COPY_KERNEL in name for v in vs]
    if not cands:
        raise SystemExit("no %s dispatch found for calibration" % COPY_KERNEL)
    return calib_kib / max(cands), max(cands)


def traffic(fetch_csv, write_csv, calib_mib, cmd_fetch, cmd_write, json_out, out):
    from exact_scaled_dot_sdpa_amd.build import source_digest

    calib_kib = calib_mib * 1024.0
    fetch = _per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(write_csv, "WRITE_SIZE")
    f_fac, f_raw = _calib(fetch, calib_kib)
    w_fac, w_raw = _calib(write, calib_kib)
    kernels = {}
    for logical, parts in KERNELS.items():
        fk = wk = 0.0
        found = True
        detail = {}
        for part in parts:
            fv = [v for n, vs in fetch.items() if part in n for v in vs]
            wv = [v for n, vs in write.items() if part in n for v in vs]
            if not fv or not wv:
                found = False
                break
            detail[part] = {"fetch_kib_raw": statistics.median(fv), "write_kib_raw": statistics.median(wv),
                            "dispatches": len(fv)}
            fk += statistics.median(fv)
            wk += statistics.median(wv)
        if not found:
            continue
        read_b = fk * f_fac * 1024.0
        write_b = wk * w_fac * 1024.0
        kernels[logical] = {"bytes_per_launch": int(round(read_b + write_b)), "read_bytes": int(round(read_b)),
                            "write_bytes": int(round(write_b)), "source_digest": source_digest(logical),
                            "parts": detail}
    doc = {
        "kernel_source_digest": source_digest(),
        "calibration": {"copy_mib": calib_mib, "fetch_kib_raw": f_raw, "write_kib_raw": w_raw,
                        "fetch_factor": f_fac, "write_factor": w_fac},
        "commands": {"fetch": cmd_fetch, "write": cmd_write},
        "kernels": kernels,
    }
    with open(json_out, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    lines = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
             "Commands:", "", "```", cmd_fetch, cmd_write, "```", "",
             "Calibration: one plain device copy of %d MiB reads %.1f KiB by FETCH_SIZE and writes %.1f KiB by "
             "WRITE_SIZE, so FETCH_SIZE is scaled by %.4f and WRITE_SIZE by %.4f." % (
                 calib_mib, f_raw, w_raw, f_fac, w_fac), "",
             "| kernel | read (MB) | write (MB) | total (MB) | source digest |", "|---|---|---|---|---|"]
    for k, e in kernels.items():
        lines.append("| %s | %.2f | %.2f | %.2f | `%s` |" % (k, e["read_bytes"] / 1e6, e["write_bytes"] / 1e6,
                                                             e["bytes_per_launch"] / 1e6, e["source_digest"]))
    text = "\n".join(lines) + "\n"
    with open(out, "w") as f:
        f.write(text)
    return text


# Normalisations of the SQ counters on MI355X: SQ_CYCLES sums the cycles of
# every shader engine (8 XCDs x 4), SQ_VALU_MFMA_BUSY_CYCLES the busy cycles of
# every SIMD (256 CUs x 4), the SQ_WAVE/WAIT/BUSY counters count in units of
# four cycles per wave, and one MFMA MOP is 512 FLOPs.
N_SE, N_SIMD, MOP_FLOPS = 32, 1024, 512
# MI355X dense MFMA peaks (TFLOP/s) and the engine clock they assume
PEAK_BF16_TFLOPS, PEAK_FP8_TFLOPS, PEAK_CLOCK_GHZ = 2500.0, 5000.0, 2.4


def counters(csv_path, cmd, out, algorithmic=None, json_out=None):
    """Per-kernel medians over the dispatches of a --pmc run, with the derived
    figures: executed MFMA FLOPs against the algorithmic ones, the clock
    (cycles over duration), the share of SIMD cycles with the MFMA unit busy,
    and the shares of wave time spent waiting.  With json_out, each logical
    kernel's clock (its parts' cycles over their summed durations) and MFMA
    busy share are stored with its source digest, for bench.py to report."""
    per = {}
    for r in csv.DictReader(open(csv_path)):
        k = _short(r["Kernel_Name"])
        d = per.setdefault(k, {}).setdefault(r["Dispatch_Id"], {"dur": int(r["End_Timestamp"]) -
                                                               int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    lines = ["# rocprofv3 SQ counters", "", "Command:", "", "```", cmd, "```", "",
             "Medians over the dispatches of each kernel. The derived columns assume MI355X's 32 shader "
             "engines (SQ_CYCLES sums them) and 1024 SIMDs (SQ_VALU_MFMA_BUSY_CYCLES sums them); wave "
             "counters tick every 4 cycles; one MFMA MOP is 512 FLOPs.", ""]
    names = sorted({c for k in per.values() for d in k.values() for c in d if c != "dur"})
    lines.append("| kernel | dispatches | " + " | ".join(names) + " |")
    lines.append("|---|---|" + "---|" * len(names))
    derived = ["", "| kernel | duration (us) | clock (GHz) | MFMA busy | executed MFMA TFLOP | algorithmic TFLOP |"
               " algorithmic rate vs peak at this clock | wait share | wait-issue share |",
               "|---|---|---|---|---|---|---|---|---|"]
    parts = {}  # short kernel name -> (cycles per engine, duration ns, MFMA busy cycles per SIMD)
    for k, ds in per.items():
        if k.startswith("__amd"):
            continue
        med = {c: statistics.median(d[c] for d in ds.values() if c in d) for c in names if
               any(c in d for d in ds.values())}
        dur = statistics.median(d["dur"] for d in ds.values())
        lines.append("| %s | %d | " % (k, len(ds)) + " | ".join("%.4g" % med[c] if c in med else "" for c in names)
                     + " |")
        cyc = med.get("SQ_CYCLES", 0.0) / N_SE
        clock = cyc / dur if dur > 0 else 0.0  # cycles per ns = GHz
        parts[k] = (cyc, dur, med.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / N_SIMD)
        busy = med.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (N_SIMD * cyc) if cyc > 0 else 0.0
        mops = sum(v for c, v in med.items() if c.startswith("SQ_INSTS_VALU_MFMA_MOPS"))
        wc = med.get("SQ_WAVE_CYCLES", 0.0)
        alg = (algorithmic or {}).get(k)
        # dense peak scaled to the measured clock; a kernel mixing fp8 and
        # bf16 MFMAs gets the rate of its executed mix
        vs_clock = ""
        if alg and mops and clock > 0 and dur >= 100e3:  # the clock is only meaningful for long kernels
            f8 = med.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0) / mops
            peak = 1.0 / (f8 / PEAK_FP8_TFLOPS + (1.0 - f8) / PEAK_BF16_TFLOPS) * clock / PEAK_CLOCK_GHZ
            vs_clock = "%.1f%% of %.0f TFLOP/s" % (100 * (alg / (dur * 1e-9) / 1e12) / peak, peak)
        derived.append("| %s | %.1f | %.2f | %s | %s | %s | %s | %s | %s |" % (
            k, dur / 1e3, clock, "%.1f%%" % (100 * busy) if busy else "",
            "%.4g" % (mops * MOP_FLOPS / 1e12) if mops else "", "%.4g" % (alg / 1e12) if alg else "", vs_clock,
            "%.1f%%" % (100 * med["SQ_WAIT_ANY"] / wc) if wc and "SQ_WAIT_ANY" in med else "",
            "%.1f%%" % (100 * med["SQ_WAIT_INST_ANY"] / wc) if wc and "SQ_WAIT_INST_ANY" in med else ""))
    text = "\n".join(lines + derived) + "\n"
    with open(out, "w") as f:
        f.write(text)
    if json_out:
        from exact_scaled_dot_sdpa_amd.build import source_digest

        kernels = {}
        for logical, names in KERNELS.items():
            found = [parts[k] for k in parts if any(n in k for n in names)]
            if len(found) != len(names) or not all(c > 0 and d > 0 for c, d, _ in found):
                continue
            cyc, dur, busy = (sum(x[i] for x in found) for i in range(3))
            # the cycle counters' window exceeds a short kernel's duration, so
            # the clock is only recorded for long ones (as in the table above)
            kernels[logical] = {"clock_ghz": round(cyc / dur, 3) if dur >= 100e3 else None,
                                "mfma_busy": round(busy / cyc, 4),
                                "duration_us": round(dur / 1e3, 2), "source_digest": source_digest(logical)}
        with open(json_out, "w") as f:
            json.dump({"command": cmd, "kernels": kernels}, f, indent=1)
            f.write("\n")
    return text


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--cmd", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--trace", default=None, help="kernel_trace csv of the same run")
    s.add_argument("--last", type=int, default=0,
                   help="also give the median and mean of the last N dispatches per kernel")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--calib-mib", type=int, required=True)
    t.add_argument("--cmd-fetch", required=True)
    t.add_argument("--cmd-write", required=True)
    t.add_argument("--json", required=True)
    t.add_argument("--out", required=True)
    c = sub.add_parser("counters", help="summarise an SQ counter run")
    c.add_argument("csv")
    c.add_argument("--cmd", required=True)
    c.add_argument("--out", required=True)
    c.add_argument("--algorithmic", default=None,
                   help="kernel=FLOPs[,kernel=FLOPs...]: algorithmic FLOPs per launch to compare with")
    c.add_argument("--json", default=None, help="also store each logical kernel's clock here")
    a = ap.parse_args(argv)
    if a.what == "stats":
        print(stats(a.csv, a.cmd, a.out, a.trace, a.last))
    elif a.what == "counters":
        alg = {}
        for item in (a.algorithmic.split(",") if a.algorithmic else []):
            k, v = item.split("=")
            alg[k] = float(v)
        print(counters(a.csv, a.cmd, a.out, alg, a.json))
    else:
        print(traffic(a.fetch, a.write, a.calib_mib, a.cmd_fetch, a.cmd_write, a.json, a.out))


if __name__ == "__main__":
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    main()
