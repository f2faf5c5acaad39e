"""rocprofv3 runs behind the committed profile summaries.

    python quantized_paged_kv_mixed_amd/profiling.py --out prof_out --summary profiles

1. a kernel trace with --stats of the default benchmark command
   (`python bench.py`), which gives every kernel's average duration;
2. two counter passes over a short benchmark (2 layers): FETCH_SIZE, then
   WRITE_SIZE. The same runs include the benchmark's 1 GiB device copy,
   whose counters calibrate both (bytes the copy must move / KiB reported);
3. two SQ counter passes over the same short benchmark (instruction counts,
   wave cycles and busy cycles: eight SQ counters a pass), summarized per
   kernel as means over its dispatches.

It writes a Markdown summary per workload into --summary (one of the SQ
counters, decode_<workload>_sq_counters.md, and one of the encoder and
promotion kernels, encode_<workload>.md) and a small JSON
record (decode_<workload>_traffic.json) that bench.py reads to report the
measured HBM traffic per decode call, only while the decode source still has
the hash recorded here. Runs nothing on the GPU itself: each profiler run is
a child process.
"""
from __future__ import annotations

import argparse
import csv
import re
import glob
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DECODE_SRC = os.path.join(ROOT, "quantized_paged_kv_mixed_amd", "csrc", "decode.hip")
COPY_BYTES = 1 << 30          # bench.py's reference copy moves 1 GiB each way


def source_hash() -> str:
    """Hash of the decode kernels and the work-split header (the counters
    hold only while both are unchanged)."""
    h = hashlib.sha256()
    for path in (DECODE_SRC, os.path.join(os.path.dirname(DECODE_SRC), "kvq_internal.h")):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _run(cmd, log, timeout):
    print(f"[profile] {' '.join(cmd)}", flush=True)
    t0 = time.time()
    with open(log, "w") as f:
        r = subprocess.run(cmd, stdout=f, stderr=subprocess.STDOUT, timeout=timeout, cwd=ROOT)
    print(f"[profile] rc {r.returncode} in {time.time() - t0:.1f} s", flush=True)
    if r.returncode != 0:
        with open(log) as f:
            print(f.read()[-2000:], file=sys.stderr)
        raise SystemExit(r.returncode)


def _one(pattern):
    hits = glob.glob(pattern, recursive=True)
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


# kernels whose traffic and duration are recorded (template arguments kept)
KERNEL_RE = (r"(decode_kernel<\d+(?:, (?:true|false))+>|merge_kernel<\d+(?:, (?:true|false))+>|"
             r"plan_kernel|items_kernel|encode_tq\w*<\d+, \d+(?:, (?:true|false))?>|"
             r"encode_tqk_tiles_kernel<(?:true|false)>|encode_fp8\w*<\d+, (?:true|false)>|promote_\w*<\d+, \d+>|"
             r"prefill_kernel<\d+, \d+>)")


# SQ counters, two passes of at most eight SQ counters (plus one GRBM)
SQ_PASSES = {
    "A": ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_MFMA",
          "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_WAIT_INST_ANY", "GRBM_GUI_ACTIVE"],
    "B": ["SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_ACTIVE_INST_ANY", "SQ_WAIT_ANY", "SQ_INSTS_SMEM",
          "SQ_LDS_BANK_CONFLICT", "SQ_THREAD_CYCLES_VALU", "SQ_CYCLES"],
}


def sq_summary(absout, summary, workload, sq_cmds, short):
    """Means per dispatch of every SQ counter for the recorded kernels, with
    instructions per wave (VALU, MFMA, SALU, LDS)."""
    per = {}
    for name in sq_cmds:
        with open(_one(f"{absout}/sq_{name}/**/*counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                m = re.search(KERNEL_RE, r["Kernel_Name"])
                if m:
                    per.setdefault(m.group(1), {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    kernels = sorted(per)
    counters = sorted({c for k in kernels for c in per[k]})
    mean = {k: {c: sum(v) / len(v) for c, v in per[k].items()} for k in kernels}
    lines = [f"# SQ counters per kernel, {workload} workload", "",
             "Two `--pmc` passes over the short benchmark; means over every dispatch of each kernel in the run.", ""]
    for name, cmd in sq_cmds.items():
        lines += ["```", " ".join(cmd[:-len(short)] + ["python"] + short[1:]), "```"]
    lines += ["", "| counter | " + " | ".join(f"`{k}`" for k in kernels) + " |",
              "|---|" + "---|" * len(kernels)]
    for c in counters:
        lines.append(f"| {c} | " + " | ".join(f"{mean[k].get(c, float('nan')):,.0f}" for k in kernels) + " |")
    lines += ["", "Per wave (counter / SQ_WAVES):", "", "| kernel | waves | VALU | MFMA | SALU | LDS | VALU busy of "
              "wave cycles |", "|---|---|---|---|---|---|---|"]
    for k in kernels:
        mk = mean[k]
        w = mk.get("SQ_WAVES", 0.0)
        if w <= 0:
            continue
        busy = mk.get("SQ_ACTIVE_INST_VALU", 0.0) / mk["SQ_WAVE_CYCLES"] if mk.get("SQ_WAVE_CYCLES") else float("nan")
        lines.append(f"| `{k}` | {w:,.0f} | {mk.get('SQ_INSTS_VALU', 0) / w:,.0f} | {mk.get('SQ_INSTS_MFMA', 0) / w:,.1f} "
                     f"| {mk.get('SQ_INSTS_SALU', 0) / w:,.0f} | {mk.get('SQ_INSTS_LDS', 0) / w:,.1f} | {busy:.2f} |")
    lines.append("")
    with open(os.path.join(summary, f"decode_{workload}_sq_counters.md"), "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines), flush=True)
    return mean


ENCODE_RE = r"^(encode_|promote_)"


def encode_summary(summary, workload, rec, sq_mean, commands):
    """The encoders' and promotion's rows of the kernel trace, the traffic
    counters and the SQ counters, side by side."""
    names = sorted({n for n in list(rec["kernels"]) + list(rec["trace_us"]) if re.match(ENCODE_RE, n)})
    lines = [f"# Encoders and promotion, {workload} workload (rocprofv3)", "",
             "Kernel durations from the kernel trace of the default benchmark (every layer's cache is "
             "encoded by the library during set-up: FP8 append, then demotion of the Stale pages from "
             "FP8 pages; promotion is timed on up to 4,096 pages of each compressed pool); HBM bytes "
             "from the FETCH_SIZE / WRITE_SIZE passes, scaled by the 1 GiB copy; instruction counts "
             "from the two SQ passes. All three are means per dispatch.", ""]
    for key in ("trace", "FETCH_SIZE", "WRITE_SIZE"):
        lines += ["```", commands[key], "```"]
    for cmd in commands.get("sq", []):
        lines += ["```", cmd, "```"]
    lines += ["", "| kernel | dispatches (trace) | average (us) | read bytes | written bytes | counter GB/s | "
              "of 8 TB/s | VALU / wave | VALU busy of wave cycles |", "|---|---|---|---|---|---|---|---|---|"]
    for n in names:
        t = rec["kernels"].get(n, {})
        tr = rec["trace_us"].get(n, {})
        rd = t.get("FETCH_SIZE", {}).get("bytes")
        wr = t.get("WRITE_SIZE", {}).get("bytes")
        gbps = t.get("counter_GBps")
        mk = sq_mean.get(n, {}) if sq_mean else {}
        w = mk.get("SQ_WAVES", 0.0)
        valu = f"{mk.get('SQ_INSTS_VALU', 0) / w:,.0f}" if w else "-"
        busy = (f"{mk['SQ_ACTIVE_INST_VALU'] / mk['SQ_WAVE_CYCLES']:.2f}"
                if mk.get("SQ_WAVE_CYCLES") and "SQ_ACTIVE_INST_VALU" in mk else "-")
        fmt = lambda x, spec: "-" if x is None else format(x, spec)
        lines.append(f"| `{n}` | {tr.get('calls', '-')} | {fmt(tr.get('average_us'), '.2f')} | {fmt(rd, ',.0f')} | "
                     f"{fmt(wr, ',.0f')} | {fmt(gbps, ',.0f')} | {fmt(None if gbps is None else gbps / 8000, '.3f')} | "
                     f"{valu} | {busy} |")
    lines += ["", "Algorithmic bytes per token-head (both roles): FP8 append reads 8d (fp32 rows) and writes "
              "2d + 8; demotion from FP8 pages reads 2(d + 4) and writes 2(b d / 8 + 2) for b-bit codes "
              "(grouped keys: 48 + 6 + 48 + 2 at d = 128); promotion reads the compressed page and writes "
              "the FP8 page. The counter GB/s above are what the kernels moved, not these figures.", ""]
    with open(os.path.join(summary, f"encode_{workload}.md"), "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines), flush=True)


def counter_per_kernel(csv_path, counter):
    """{kernel name: [value per dispatch]} for one counter."""
    out = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default="prof_out")
    ap.add_argument("--summary", default="profiles")
    ap.add_argument("--workload", default="canary")
    ap.add_argument("--skip-trace", action="store_true")
    ap.add_argument("--parse-only", action="store_true", help="summarize existing profiler output in --out")
    ap.add_argument("--no-sq", action="store_true", help="skip the two SQ counter passes")
    args = ap.parse_args()
    out = os.path.relpath(os.path.abspath(args.out), ROOT)     # profiler runs start in the repository root
    os.makedirs(os.path.join(ROOT, out), exist_ok=True)
    bench = [sys.executable, "bench.py", "--workload", args.workload]
    # counter passes: a short benchmark (2 layers); its entry-point timings
    # also run promotion, and the scored / prefill / appending variants are
    # separate kernels (their own template arguments)
    short = bench + ["--layers", "2", "--steps", "3", "--warmup", "1", "--no-cpu-baseline"]
    trace_cmd = ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d", f"{out}/trace",
                 "-o", "run", "--"] + bench
    pmc_cmds = {c: ["rocprofv3", "--pmc", c, "--output-format", "csv", "-d", f"{out}/{c.lower()}", "-o", "run",
                    "--"] + short for c in ("FETCH_SIZE", "WRITE_SIZE")}
    sq_cmds = {name: ["rocprofv3", "--pmc", *ctrs, "--output-format", "csv", "-d", f"{out}/sq_{name}", "-o", "run",
                      "--"] + short for name, ctrs in SQ_PASSES.items()}
    absout = os.path.join(ROOT, out)
    if not args.parse_only:
        if not args.skip_trace:
            _run(trace_cmd, f"{absout}/trace.log", 900)
        for c, cmd in pmc_cmds.items():
            _run(cmd, f"{absout}/{c.lower()}.log", 300)
        if not args.no_sq:
            for name, cmd in sq_cmds.items():
                _run(cmd, f"{absout}/sq_{name}.log", 300)

    # kernel statistics
    stats_rows = []
    if not args.skip_trace:
        with open(_one(f"{absout}/trace/**/*kernel_stats.csv")) as f:
            stats_rows = list(csv.DictReader(f))
    # counters
    per = {}
    for c in pmc_cmds:
        per[c] = counter_per_kernel(_one(f"{absout}/{c.lower()}/**/*counter_collection.csv"), c)
    copy_name = next(k for k in per["WRITE_SIZE"] if "copyBuffer" in k)
    fetch_copy = max(per["FETCH_SIZE"][copy_name])
    write_copy = max(per["WRITE_SIZE"][copy_name])
    f_scale = COPY_BYTES / (fetch_copy * 1024.0)
    w_scale = COPY_BYTES / (write_copy * 1024.0)
    traffic = {}
    for c, scale in (("FETCH_SIZE", f_scale), ("WRITE_SIZE", w_scale)):
        for k, v in per[c].items():
            m = re.search(KERNEL_RE, k)
            if m:
                short_name = m.group(1)
                traffic.setdefault(short_name, {})[c] = {"kib_reported": sum(v) / len(v),
                                                         "bytes": sum(v) / len(v) * 1024.0 * scale,
                                                         "dispatches": len(v)}
    # one plain decode call = the plain scan and merge kernels (the scored,
    # appending and prefill variants the benchmark also times are listed but
    # not counted)
    call_bytes = sum(t[c]["bytes"] for n, t in traffic.items()
                     if re.fullmatch(r"(decode|merge)_kernel<\d+, false, false>", n) for c in t)
    # average durations of the same kernels in the kernel trace (microseconds)
    trace_us = {}
    for r in stats_rows:
        m = re.search(KERNEL_RE, r["Name"])
        if m:
            trace_us[m.group(1)] = {"average_us": float(r["AverageNs"]) / 1e3, "calls": int(r["Calls"])}
    for n, t in traffic.items():
        if n in trace_us:
            t["trace_average_us"] = trace_us[n]["average_us"]
            moved = sum(t[c]["bytes"] for c in ("FETCH_SIZE", "WRITE_SIZE") if c in t)
            t["counter_GBps"] = moved / (trace_us[n]["average_us"] * 1e-6) / 1e9
    rec = {"workload": args.workload, "decode_source_sha256_16": source_hash(), "trace_us": trace_us,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "copy_fetch_kib": fetch_copy, "copy_write_kib": write_copy,
           "kernels": traffic, "decode_call_hbm_bytes": call_bytes,
           "commands": {"trace": " ".join(trace_cmd[:-len(bench)] + ["python", "bench.py", "--workload",
                                                                      args.workload]),
                        **{c: " ".join(cmd[:-len(short)] + ["python"] + short[1:]) for c, cmd in pmc_cmds.items()}}}
    summary = os.path.join(ROOT, args.summary) if not os.path.isabs(args.summary) else args.summary
    os.makedirs(summary, exist_ok=True)
    with open(os.path.join(summary, f"decode_{args.workload}_traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    lines = [f"# rocprofv3: mixed-format paged decode, {args.workload} workload", "",
             f"decode.hip + kvq_internal.h sha256[:16] = `{rec['decode_source_sha256_16']}`", ""]
    if stats_rows:
        lines += ["## Kernel trace (`--kernel-trace --stats`)", "", "```", rec["commands"]["trace"], "```", "",
                  "| kernel | calls | average (us) | total (ms) | % |", "|---|---|---|---|---|"]
        for r in stats_rows[:14]:
            name = r["Name"].replace("|", "/")
            if len(name) > 90:
                name = name[:87] + "..."
            lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                         f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f} |")
        lines.append("")
    lines += ["## HBM traffic (`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`)", ""]
    for c, cmd in pmc_cmds.items():
        lines += ["```", rec["commands"][c], "```"]
    lines += ["", f"Calibration: the benchmark's 1 GiB device copy reads FETCH_SIZE = {fetch_copy:.1f} KiB and "
              f"WRITE_SIZE = {write_copy:.1f} KiB per dispatch, so reported KiB are scaled by "
              f"{f_scale:.4f} (fetch) and {w_scale:.4f} (write).", "",
              "| kernel | FETCH_SIZE (KiB, reported) | read bytes (scaled) | WRITE_SIZE (KiB, reported) | "
              "written bytes (scaled) |", "|---|---|---|---|---|"]
    for n, t in sorted(traffic.items()):
        fz, wz = t.get("FETCH_SIZE", {}), t.get("WRITE_SIZE", {})
        lines.append(f"| `{n}` | {fz.get('kib_reported', 0):.1f} | {fz.get('bytes', 0):.0f} | "
                     f"{wz.get('kib_reported', 0):.1f} | {wz.get('bytes', 0):.0f} |")
    lines += ["", f"One plain decode call (scan + merge kernels) moves {call_bytes:.0f} bytes of HBM traffic.", ""]
    rated = [(n, t) for n, t in sorted(traffic.items()) if "counter_GBps" in t]
    if rated:
        lines += ["Counter traffic over the kernel-trace average duration:", "",
                  "| kernel | bytes per dispatch (read + write) | trace average (us) | GB/s | of 8 TB/s |",
                  "|---|---|---|---|---|"]
        for n, t in rated:
            moved = sum(t[c]["bytes"] for c in ("FETCH_SIZE", "WRITE_SIZE") if c in t)
            lines.append(f"| `{n}` | {moved:.0f} | {t['trace_average_us']:.3f} | {t['counter_GBps']:.0f} | "
                         f"{t['counter_GBps'] / 8000:.3f} |")
        lines.append("")
    with open(os.path.join(summary, f"decode_{args.workload}.md"), "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines), flush=True)
    sq_mean = sq_summary(absout, summary, args.workload, sq_cmds, short) if not args.no_sq else {}
    commands = dict(rec["commands"])
    commands["sq"] = [" ".join(cmd[:-len(short)] + ["python"] + short[1:]) for cmd in sq_cmds.values()] \
        if not args.no_sq else []
    encode_summary(summary, args.workload, rec, sq_mean, commands)


if __name__ == "__main__":
    main()
