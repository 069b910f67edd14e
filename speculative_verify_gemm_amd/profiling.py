"""Short text summaries of rocprofv3 runs of bench.py, for profiles/.

    python -m speculative_verify_gemm_amd.profiling trace <trace dir> --cmd "<command>" --out <file.md>
    python -m speculative_verify_gemm_amd.profiling mfma <pmc dir>=<bench out> ... --cmd "<commands>" --out <file.md>
    python -m speculative_verify_gemm_amd.profiling calib <program output> <counter dir> <MfmaUtil dir> --cmd ... --out ...
    python -m speculative_verify_gemm_amd.profiling traffic <fetch dir> <write dir> --calib-mib 256 \\
        --workload stack_w4g64 --m 16 --fetch-json <bench out> --write-json <bench out> \\
        --cmd "<commands>" --out <file.md>

`trace` reads the kernel trace (`--kernel-trace`, csv) and lists every kernel's
dispatch count and mean / median / min duration, with the W4A8 and W8A8 linear
kernels also pooled over the launch mix of a pass.

`mfma` reads counter runs of the MFMA passes (`--pmc MfmaUtil
SQ_INSTS_VALU_MFMA_MOPS_I8 SQ_INSTS_VALU_MFMA_I8`, one run per workload and
M), each paired with the bench.py line of a plain run (no profiler: counter
collection serializes the dispatches) of the same workload and M, and lists
per linear kernel the share of SIMD cycles the matrix unit was busy, the int8
operations it executed per launch against the algorithmic 2*M*N*K, and the
executed rate over the plain run's mean launch duration.

`calib` summarizes the int8 MFMA calibration program (calib/mfma_peak.hip):
its throughput, and the busy cycles and operations the counters charge per
MFMA instruction.

`hbm` summarizes the HBM read calibration program (calib/hbm_read.hip): per
size, the time per launch and the dispatch spans of a kernel trace.

`traffic` reads two counter runs (`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`):
each counter is scaled by what it reads for the device-to-device copy of
`--calib-mib` MiB that bench.py makes first (`--calib-copy-mib`), whose true
size is known, and the linear kernels' HBM bytes per launch are pooled the same
way.  The summary records the digest of the kernel sources the runs were taken
on (which bench.py prints in its JSON line); bench.py reports the figure only
while that digest still matches the sources.
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _rows(d, suffix):
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    out = []
    for f in files:
        with open(f, newline="") as fh:
            out.extend(csv.DictReader(fh))
    return out


def _short(name):
    """Kernel name without the argument list and anonymous-namespace noise."""
    n = name.replace("(anonymous namespace)::", "")
    if n.startswith("void "):
        n = n[5:]
    depth = 0
    for i, c in enumerate(n):
        depth += c == "<"
        depth -= c == ">"
        if c == "(" and depth == 0:
            return n[:i]
    return n


def _is_linear(name):
    return name.startswith(("k_linear<", "k_linear_fused<"))


def _policy(name):
    """'k_linear<MfmaW4<1, 64, false, false>, 8, 4, 4>' -> 'k_linear<MfmaW4<1, 64, false, false>>'."""
    head, inner = name.split("<", 1)
    return f"{head}<{_first_arg(inner)}>"


def _first_arg(inner):
    depth = 0
    for i, c in enumerate(inner):
        depth += c == "<"
        depth -= c == ">"
        if c == "," and depth == 0:
            return inner[:i]
    return inner.rstrip(">")


def trace_summary(d, cmd, only=None, bench_json=None):
    """Per-kernel span statistics of a kernel trace; `only`: keep the kernels
    whose name starts with it (the others are counted as other kernels).
    With the traced run's bench.py output, the kernel digest it printed and
    the figures of its JSON line that the trace cross-checks."""
    rows = _rows(d, "kernel_trace.csv")
    by, other = {}, []
    for r in rows:
        n = _short(r["Kernel_Name"])
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if not n.startswith(only or "k_"):
            other.append(dur)
            continue
        wgs, wg = 1, 1
        for ax in ("X", "Y", "Z"):  # grid sizes are in threads, per dimension
            g, w = int(r.get(f"Grid_Size_{ax}") or 1), max(1, int(r.get(f"Workgroup_Size_{ax}") or 1))
            wgs *= max(1, g // w)
            wg *= w
        by.setdefault((n, wgs, wg), []).append(dur)
    head = []
    if bench_json:
        b = _bench_line(bench_json)
        head = [f"digest: {b['kernel_digest']}", ""]
        if "roofline" in b:
            r = b["roofline"]
            head[-1:] = [f"bench line of the traced run (timed under the profiler, which stretches the "
                         f"event spans; the trace's own spans are below): {b['ms_per_step']} ms per pass "
                         f"(M = {b['config'].get('M')}), mean linear launch {r.get('mean_launch_us')} us "
                         f"({r.get('kernel')})", ""]
    lines = ["# rocprofv3 kernel trace", "", "Command:", "", "```", cmd, "```", ""] + head + [
             "Durations are kernel-trace spans (start to end of each dispatch).", "",
             "| kernel | workgroups x threads | dispatches | mean us | median us | min us |",
             "|---|---|---|---|---|---|"]
    for (n, wgs, wg), v in sorted(by.items()):
        lines.append(f"| `{n}` | {wgs} x {wg} | {len(v)} | {statistics.mean(v):.2f} | "
                     f"{statistics.median(v):.2f} | {min(v):.2f} |")
    pooled = {}
    for (n, _w, _g), v in by.items():
        if _is_linear(n):
            pooled.setdefault(_policy(n), []).extend(v)
    if pooled:
        lines += ["", "Linear kernels pooled per policy over all launch shapes of a pass:", ""]
        for pol, v in sorted(pooled.items()):
            lines.append(f"- `{pol}`: {len(v)} dispatches, mean {statistics.mean(v):.3f} us, "
                         f"median {statistics.median(v):.3f} us")
    if other:
        what = "every other kernel of the run" if only else "torch weight generation and fills at set-up"
        lines += ["", f"Other kernels ({what}): {len(other)} dispatches, {sum(other) / 1e3:.1f} ms in total."]
    return "\n".join(lines) + "\n"


def _counter(rows, counter):
    """{dispatch id: (kernel, value)} for one counter (KiB per dispatch)."""
    out = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        did = r["Dispatch_Id"]
        k, v = out.get(did, (r["Kernel_Name"], 0.0))
        out[did] = (k, v + float(r["Counter_Value"]))
    return out


def _scale(vals, calib_kib):
    """Factor that maps the counter onto true KiB, from the calibration copy:
    the copy dispatches whose reading lies between a quarter and 1.5 times
    its size (FETCH_SIZE reads half of it, WRITE_SIZE all of it; copies of
    other sizes in the same run fall outside)."""
    copies = [v for k, v in vals.values() if COPY_KERNEL in k and 0.25 * calib_kib <= v <= 1.5 * calib_kib]
    if not copies:
        raise SystemExit("no calibration copy found in the counter run")
    return calib_kib / statistics.median(copies), len(copies)


def _run_digest(bench_json):
    """The kernel digest bench.py printed in a profiled run."""
    import json
    with open(bench_json) as f:
        lines = [ln for ln in f if ln.startswith("{")]
    if not lines:
        raise SystemExit(f"no bench JSON line in {bench_json}")
    return json.loads(lines[-1])["kernel_digest"]


def traffic_summary(fetch_dir, write_dir, calib_mib, workload, M, cmd, fetch_json, write_json):
    digest = _run_digest(fetch_json)
    if _run_digest(write_json) != digest:
        raise SystemExit("the two counter runs were taken on different kernels")
    calib_kib = calib_mib * 1024.0
    fetch = _counter(_rows(fetch_dir, "counter_collection.csv"), "FETCH_SIZE")
    write = _counter(_rows(write_dir, "counter_collection.csv"), "WRITE_SIZE")
    ff, nf = _scale(fetch, calib_kib)
    fw, nw = _scale(write, calib_kib)
    lf = [v for k, v in fetch.values() if _is_linear(_short(k))]
    lw = [v for k, v in write.values() if _is_linear(_short(k))]
    if not lf or not lw:
        raise SystemExit("no linear kernel dispatch in the counter runs")
    fetch_b = statistics.mean(lf) * ff * 1024.0
    write_b = statistics.mean(lw) * fw * 1024.0
    lines = ["# rocprofv3 HBM traffic of the linear kernels", "", "Commands (two counter runs):", "", "```",
             cmd, "```", "",
             f"workload: {workload} M={M}",
             f"digest: {digest}",
             f"calibration: device-to-device copy of {calib_mib} MiB; FETCH_SIZE scale {ff:.4f} "
             f"({nf} copies), WRITE_SIZE scale {fw:.4f} ({nw} copies)",
             f"linear dispatches counted: {len(lf)} (fetch run), {len(lw)} (write run)",
             f"fetch_bytes_per_launch: {fetch_b:.6g}",
             f"write_bytes_per_launch: {write_b:.6g}",
             f"traffic_bytes_per_launch: {fetch_b + write_b:.6g}", ""]
    return "\n".join(lines)


PEAK_I8_TOPS = 5000.0  # MI355X dense int8 MFMA, TOP/s


def _bench_line(path):
    import json
    with open(path) as f:
        lines = [ln for ln in f if ln.startswith("{")]
    if not lines:
        raise SystemExit(f"no bench JSON line in {path}")
    return json.loads(lines[-1])


def mfma_summary(runs, cmd):
    """runs: [(counter dir, bench.py output of a plain run)], one per workload
    and M."""
    lines = ["# rocprofv3 MFMA counters of the linear kernels", "", "Commands (one counter run per row group):", "",
             "```", cmd, "```", "",
             "Per linear kernel of each run: `busy` = MfmaUtil, the matrix unit's busy cycles over all SIMDs "
             "divided by (GPU-active cycles x SIMDs) during the dispatch, so launch ramp and tail count as idle "
             "(the counter charges 16 busy cycles per v_mfma_i32_16x16x64_i8, profiles/mfma_i8_calibration.md, "
             "so `busy` reading about half of `% of peak` is the time base: a serialized dispatch of the counter "
             "run stays active about twice as long as the plain run's launch; `% of peak` is the figure quoted); "
             "`executed` = SQ_INSTS_VALU_MFMA_MOPS_I8 x 512 int8 operations per launch; `algorithmic` = "
             "2*M*N*K per launch (the MFMA form executes more: rows padded to 16 tokens, the zero-point "
             "MFMA of W4); `rate` = executed operations over the mean linear launch duration of a plain "
             f"32-layer run (bench.py, HIP events), against the {PEAK_I8_TOPS:.0f} TOP/s dense int8 peak.", "",
             "| workload | M | kernel | dispatches | busy % | MFMA instr / launch | executed Gop / launch | "
             "algorithmic Gop / launch | executed / algorithmic | mean launch us | rate TOP/s | % of peak |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    digests = set()
    for d, js in runs:
        out = _bench_line(js)
        digests.add(out["kernel_digest"])
        rows = _rows(d, "counter_collection.csv")
        util = _counter(rows, "MfmaUtil")
        mops = _counter(rows, "SQ_INSTS_VALU_MFMA_MOPS_I8")
        inst = _counter(rows, "SQ_INSTS_VALU_MFMA_I8")
        rf = out["roofline"]
        launch_us = rf["mean_launch_us"]
        alg = rf["mean_algorithmic_int8_ops_per_launch"]
        by = {}
        for did, (k, v) in util.items():
            n = _short(k)
            if not _is_linear(n):
                continue
            b = by.setdefault(_policy(n), [[], [], []])
            b[0].append(v)
            b[1].append(mops.get(did, (k, 0.0))[1] * 512.0)
            b[2].append(inst.get(did, (k, 0.0))[1])
        cfg = out["config"]
        for pol, (u, o, ni) in sorted(by.items()):
            ex = statistics.mean(o)
            rate = ex / (launch_us * 1e-6) / 1e12
            lines.append(f"| {cfg['workload']} | {cfg['M']} | `{pol}` | {len(u)} | {statistics.mean(u):.2f} | "
                         f"{statistics.mean(ni):.0f} | {ex / 1e9:.3f} | {alg / 1e9:.3f} | {ex / alg:.2f} | "
                         f"{launch_us:.2f} | {rate:.1f} | {100 * rate / PEAK_I8_TOPS:.2f} |")
    lines += ["", "digest: " + ", ".join(sorted(digests)), ""]
    return "\n".join(lines)


def calib_summary(plain_txt, counter_dir, util_dir, cmd):
    """The int8 MFMA calibration program (calib/mfma_peak.hip): its printed
    throughput per occupancy, and per timed dispatch the busy cycles and int8
    operations the counters charge per MFMA instruction."""
    with open(plain_txt) as f:
        printed = [ln.strip() for ln in f if ln.startswith("waves per SIMD")]
    rows = _rows(counter_dir, "counter_collection.csv")
    by = {}
    for r in rows:
        d = by.setdefault(r["Dispatch_Id"], {"kernel": _short(r["Kernel_Name"])})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    util = {did: v for did, (_k, v) in _counter(_rows(util_dir, "counter_collection.csv"), "MfmaUtil").items()}
    lines = ["# Calibration of the int8 MFMA pipe (v_mfma_i32_16x16x64_i8)", "", "Commands:", "", "```", cmd, "```",
             "", "Throughput (plain run, HIP events; 256 workgroups, four independent accumulator chains per "
             "wave):", ""]
    lines += [f"- {ln}" for ln in printed]
    lines += ["", "Counters of the timed dispatches (the larger of each kernel's two):", "",
              "| kernel | MFMA instructions | busy cycles / instruction | int8 ops / instruction | MfmaUtil % |",
              "|---|---|---|---|---|"]
    best = {}
    for did, d in by.items():
        n = d.get("SQ_INSTS_VALU_MFMA_I8", 0.0)
        if n and n > best.get(d["kernel"], (0, None))[0]:
            best[d["kernel"]] = (n, did)
    for k, (n, did) in sorted(best.items()):
        d = by[did]
        u = util.get(did)
        lines.append(f"| `{k}` | {n:.0f} | {d['SQ_VALU_MFMA_BUSY_CYCLES'] / n:.2f} | "
                     f"{d['SQ_INSTS_VALU_MFMA_MOPS_I8'] * 512 / n:.0f} | {'' if u is None else f'{u:.1f}'} |")
    lines.append("")
    return "\n".join(lines)


def hbm_summary(plain_txt, trace_dir, cmd, reps=50):
    """The HBM read calibration program (calib/hbm_read.hip): its printed
    per-launch times (events around back-to-back launches) and, from a kernel
    trace of the same program, the dispatch spans of the timed launches of
    each size (the program launches three untimed, then the timed ones, size
    after size)."""
    import re
    with open(plain_txt) as f:
        printed = [ln.rstrip() for ln in f if ln.startswith("read ")]
    spans = []
    for r in sorted(_rows(trace_dir, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"])):
        if _short(r["Kernel_Name"]).startswith("k_read"):
            spans.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["# HBM read calibration (read-only streaming kernel)", "", "Commands:", "", "```", cmd, "```", "",
             "| size | bytes | us per launch (events, back to back) | GB/s | median dispatch span us (trace) | "
             "GB/s over the span |", "|---|---|---|---|---|---|"]
    pos = 0
    for ln in printed:
        m = re.match(r"read (.+?)\s+(\d+) bytes:\s+([\d.]+) us per launch,\s+([\d.]+) GB/s", ln)
        if not m:
            continue
        what, nbytes, us, gbps = m.group(1), int(m.group(2)), float(m.group(3)), float(m.group(4))
        n = 5 if nbytes >= (1 << 30) else reps  # the program times 5 launches of the GiB sizes
        timed = spans[pos + 3: pos + 3 + n]
        pos += 3 + n
        med = statistics.median(timed) if timed else float("nan")
        lines.append(f"| {what} | {nbytes} | {us:.2f} | {gbps:.1f} | {med:.2f} | {nbytes / (med * 1e-6) / 1e9:.1f} |")
    lines.append("")
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser(description="summarize rocprofv3 runs of bench.py")
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--cmd", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--only", default=None, help="keep the kernels whose name starts with this")
    t.add_argument("--bench-json", default=None, help="bench.py output of the traced run (digest, figures)")
    mf = sub.add_parser("mfma")
    mf.add_argument("runs", nargs="+", help="<counter dir>=<bench.py output of a plain run, same workload and M>")
    mf.add_argument("--cmd", required=True)
    mf.add_argument("--out", required=True)
    cb = sub.add_parser("calib")
    cb.add_argument("plain", help="output of calib/mfma_peak")
    cb.add_argument("counter_dir", help="--pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_I8 SQ_INSTS_VALU_MFMA_MOPS_I8")
    cb.add_argument("util_dir", help="--pmc MfmaUtil")
    cb.add_argument("--cmd", required=True)
    cb.add_argument("--out", required=True)
    hb = sub.add_parser("hbm")
    hb.add_argument("plain", help="output of calib/hbm_read")
    hb.add_argument("trace_dir", help="--kernel-trace of the same program")
    hb.add_argument("--reps", type=int, default=50, help="the launches per size the program was given")
    hb.add_argument("--cmd", required=True)
    hb.add_argument("--out", required=True)
    c = sub.add_parser("traffic")
    c.add_argument("fetch_dir")
    c.add_argument("write_dir")
    c.add_argument("--calib-mib", type=int, required=True)
    c.add_argument("--workload", required=True)
    c.add_argument("--m", type=int, required=True)
    c.add_argument("--fetch-json", required=True, help="bench.py output of the FETCH_SIZE run")
    c.add_argument("--write-json", required=True, help="bench.py output of the WRITE_SIZE run")
    c.add_argument("--cmd", required=True)
    c.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.what == "trace":
        text = trace_summary(a.dir, a.cmd, a.only, a.bench_json)
    elif a.what == "hbm":
        text = hbm_summary(a.plain, a.trace_dir, a.cmd, a.reps)
    elif a.what == "calib":
        text = calib_summary(a.plain, a.counter_dir, a.util_dir, a.cmd)
    elif a.what == "mfma":
        text = mfma_summary([tuple(r.split("=", 1)) for r in a.runs], a.cmd)
    else:
        text = traffic_summary(a.fetch_dir, a.write_dir, a.calib_mib, a.workload, a.m, a.cmd,
                               a.fetch_json, a.write_json)
    with open(a.out, "w") as f:
        f.write(text)
    print(text)


if __name__ == "__main__":
    main()
