"""rocprofv3 harness: per-kernel time, matrix-core use and HBM traffic of one
bench.py workload, each against MI355X's published peaks.

    python3 gated_gqa_causal_amd/rocprof_harness.py run --workload NAME [--bench-args "--weights"]
        [--out DIR] [--calibration FILE]
    python3 gated_gqa_causal_amd/rocprof_harness.py merge DIR/summary.json ...

``run`` starts bench.py under rocprofv3 once per pass, since rocprofv3 only
collects what one hardware pass can hold:

    trace  --kernel-trace --stats           calls and average duration per kernel
    fetch  --pmc FETCH_SIZE                 KiB read from HBM per dispatch
    write  --pmc WRITE_SIZE                 KiB written to HBM per dispatch
    mfma   --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE
    lds    --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_WAVE_CYCLES GRBM_GUI_ACTIVE

and, unless ``--calibration`` names an earlier run's calibration, FETCH_SIZE
and WRITE_SIZE over bench.py's plain 1 GiB device copy: the ratio of the known
size to what each counter reads there scales that counter for every kernel.

Each pass is a child process (rocprofv3 first, the Python program right after
``--``) with a time limit of its own; this process never touches the GPU.
The passes' CSV files, logs and the summary (``summary.md``, ``summary.json``)
go to ``--out``.  Per kernel the summary gives: the trace's average launch
time; for the attention kernel the algorithmic TFLOP/s (bench.py's count of
4 x head_dim FLOPs per visible (row, key, query head)) and the executed bf16
MFMA rate (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 FLOPs), against 2500 TFLOP/s;
matrix-pipe utilisation (busy cycles over the SIMD-cycles of the launch);
the shader clock (GRBM_GUI_ACTIVE per XCD over the launch time); HBM bytes
and GB/s, measured and algorithmic, against 8000 GB/s; LDS bank-conflict
cycles as a share of LDS-active cycles.

``merge`` (no GPU) copies the attention and weights kernels' measured bytes
per launch from summaries into ``profiles/traffic_attention.json`` and
``profiles/traffic_weights.json``, keyed by the workload and bench.py flags
of the run (e.g. "c3_prefix_t8192_qb1024 --cached"), with the kernel source
hash they were measured on; bench.py reports them while that hash matches.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import shlex
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")
KERNEL_SOURCE = os.path.join(ROOT, "gated_gqa_causal_amd", "csrc", "kernels.hip")
TRAFFIC = {"attention": os.path.join(ROOT, "profiles", "traffic_attention.json"),
           "weights": os.path.join(ROOT, "profiles", "traffic_weights.json")}

PEAK_BF16_TFLOPS = 2500.0     # dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
FLOPS_PER_MOP = 512           # SQ_INSTS_VALU_MFMA_MOPS_* counts units of 512 FLOPs

PASSES = {
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE"],
    "mfma": ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE"],
    "lds": ["SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE"],
}

# Library kernels by a part of their name, in the order the summary lists them.
KERNELS = [("attention", "attn_fwd8"), ("weights", "attn_weights"), ("kv_prologue", "kv_prologue"),
           ("mask_pack", "mask_pack"), ("kv_widen", "kv_widen")]


def log(msg: str) -> None:
    print(f"[prof] {msg}", flush=True)


def kernel_source_hash() -> str:
    """sha256 prefix of the kernels' sources (kernels.hip and the headers it
    builds from: the parameter blocks and the work schedule)."""
    h = hashlib.sha256()
    for name in ("kernels.hip", "kernels.h", "schedule.h"):
        with open(os.path.join(os.path.dirname(KERNEL_SOURCE), name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_key(name: str):
    for key, part in KERNELS:
        if part in name:
            return key
    return None


def _col(header, *names):
    low = [h.strip().lower() for h in header]
    for n in names:
        if n.lower() in low:
            return low.index(n.lower())
    raise KeyError(f"none of {names} in CSV header {header}")


def read_kernel_stats(out_dir: str) -> dict:
    """{kernel name: {"calls", "avg_ns", "min_ns", "max_ns"}} from a --stats run."""
    files = glob.glob(os.path.join(out_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *kernel_stats.csv under {out_dir}")
    res = {}
    for path in files:
        with open(path, newline="") as f:
            rows = list(csv.reader(f))
        h = rows[0]
        i_name, i_calls = _col(h, "Name", "KERNEL_NAME"), _col(h, "Calls")
        i_avg = _col(h, "AverageNs", "Average_ns")
        i_min, i_max = _col(h, "MinNs", "Min_ns"), _col(h, "MaxNs", "Max_ns")
        for r in rows[1:]:
            if len(r) <= max(i_name, i_calls, i_avg, i_min, i_max):
                continue
            res[r[i_name]] = {"calls": int(float(r[i_calls])), "avg_ns": float(r[i_avg]),
                              "min_ns": float(r[i_min]), "max_ns": float(r[i_max])}
    return res


def read_dispatches(out_dir: str) -> dict:
    """{kernel name: [duration ns of each dispatch, in dispatch order]} from a
    --kernel-trace run."""
    files = glob.glob(os.path.join(out_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *kernel_trace.csv under {out_dir}")
    rec = []
    for path in files:
        with open(path, newline="") as f:
            rows = list(csv.reader(f))
        h = rows[0]
        i_name, i_disp = _col(h, "Kernel_Name"), _col(h, "Dispatch_Id")
        i_t0, i_t1 = _col(h, "Start_Timestamp"), _col(h, "End_Timestamp")
        for r in rows[1:]:
            if len(r) > max(i_name, i_disp, i_t0, i_t1):
                rec.append((path, int(r[i_disp]), r[i_name], float(r[i_t1]) - float(r[i_t0])))
    res = {}
    for _, _, name, d in sorted(rec):
        res.setdefault(name, []).append(d)
    return res


def read_counters(out_dir: str, last: int = 0) -> dict:
    """{kernel name: {counter: mean over dispatches, "dispatch_ns": mean
    dispatch time in this pass}} from a --pmc run, over each kernel's last
    ``last`` dispatches (all when 0).  Rows of one (dispatch, counter) are
    summed first, in case a counter comes split over hardware instances."""
    files = glob.glob(os.path.join(out_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *counter_collection.csv under {out_dir}")
    per, dur = {}, {}
    for path in files:
        with open(path, newline="") as f:
            rows = list(csv.reader(f))
        h = rows[0]
        i_name = _col(h, "Kernel_Name")
        i_disp = _col(h, "Dispatch_Id", "Correlation_Id")
        i_ctr, i_val = _col(h, "Counter_Name"), _col(h, "Counter_Value")
        i_t0, i_t1 = _col(h, "Start_Timestamp"), _col(h, "End_Timestamp")
        for r in rows[1:]:
            if len(r) <= max(i_name, i_disp, i_ctr, i_val, i_t0, i_t1):
                continue
            key = (r[i_name], path, int(r[i_disp]))
            ctrs = per.setdefault(key, {})
            ctrs[r[i_ctr]] = ctrs.get(r[i_ctr], 0.0) + float(r[i_val])
            dur[key] = float(r[i_t1]) - float(r[i_t0])
    by_name = {}
    for key in sorted(per, key=lambda k: (k[1], k[2])):
        by_name.setdefault(key[0], []).append(key)
    res = {}
    for name, keys in by_name.items():
        keys = keys[-last:] if last else keys
        acc = {}
        for key in keys:
            for ctr, val in per[key].items():
                acc.setdefault(ctr, []).append(val)
        res[name] = {ctr: sum(v) / len(v) for ctr, v in acc.items()}
        res[name]["dispatch_ns"] = sum(dur[k] for k in keys) / len(keys)
    return res


def last_json_line(text: str):
    for line in reversed(text.splitlines()):
        line = line.strip()
        if line.startswith("{") and line.endswith("}"):
            try:
                return json.loads(line)
            except ValueError:
                continue
    return None


def run_pass(name: str, prof_args, bench_args, out_dir: str, timeout: int) -> dict:
    """One rocprofv3 child process over bench.py; returns bench.py's JSON line."""
    d = os.path.join(out_dir, name)
    os.makedirs(d, exist_ok=True)
    cmd = (["rocprofv3"] + prof_args + ["-d", d, "--output-format", "csv", "--",
                                        sys.executable, BENCH] + bench_args)
    env = dict(os.environ, TMPDIR="/tmp")
    log(f"pass {name}: {' '.join(shlex.quote(c) for c in cmd)}")
    t0 = time.time()
    with open(os.path.join(d, "stdout.txt"), "w") as fo, open(os.path.join(d, "stderr.txt"), "w") as fe:
        try:
            rc = subprocess.run(cmd, stdout=fo, stderr=fe, cwd="/tmp", env=env, timeout=timeout).returncode
        except subprocess.TimeoutExpired:
            raise RuntimeError(f"pass {name} exceeded {timeout} s (killed); see {d}/stderr.txt")
    with open(os.path.join(d, "stdout.txt")) as f:
        rec = last_json_line(f.read())
    log(f"pass {name}: rc {rc} in {time.time() - t0:.1f} s")
    # rocprofv3 may itself end with a segmentation fault after the program has
    # finished and its results are written; the program's own JSON line says
    # whether it finished.
    if rec is None or rc not in (0, 139, -11):
        raise RuntimeError(f"pass {name} failed (rc {rc}, JSON line {'found' if rec else 'missing'}); "
                           f"see {d}/stderr.txt")
    return {"cmd": cmd, "bench": rec, "dir": d}


def calibrate(out_dir: str, timeout: int) -> dict:
    """Scale factors of FETCH_SIZE and WRITE_SIZE from a plain device copy."""
    cal = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        r = run_pass(f"copy_{ctr.lower()}", ["--pmc", ctr], ["--mode", "copy", "--steps", "3"], out_dir, timeout)
        nbytes = r["bench"]["bytes_read_per_copy" if ctr == "FETCH_SIZE" else "bytes_written_per_copy"]
        ctrs = read_counters(r["dir"])
        copies = {n: c[ctr] for n, c in ctrs.items() if ctr in c and "copy" in n.lower()}
        if not copies:     # the copy's kernel under another name: take the largest dispatch
            copies = {n: c[ctr] for n, c in ctrs.items() if ctr in c}
        name = max(copies, key=copies.get)
        kib = copies[name]
        cal[ctr] = {"copy_bytes": nbytes, "kernel": name, "kib": kib, "factor": nbytes / (kib * 1024.0)}
        log(f"calibration {ctr}: {kib:.0f} KiB per {nbytes} B copy ({name}) -> factor {cal[ctr]['factor']:.3f}")
    return cal


def summarise(workload, bench_args, trace, counters, cal, cmds, cus, xcds) -> dict:
    """Per-kernel figures.  Times are over each kernel's launches in the trace
    pass's timed steps (its last ``steps`` dispatches: bench.py launches each
    kernel once per step, after the warmup steps and any one-time set-up)."""
    alg = trace["bench"].get("kernels_algorithmic", {})
    steps = int(trace["bench"].get("steps", 0))
    stats = read_kernel_stats(trace["dir"])
    disp = read_dispatches(trace["dir"])
    kernels = []
    for name, st in sorted(stats.items(), key=lambda kv: -kv[1]["avg_ns"] * kv[1]["calls"]):
        key = kernel_key(name)
        k = {"name": name, "key": key, "stats_avg_ns": st["avg_ns"], **st}
        d = disp.get(name, [])
        if key is not None and steps and len(d) >= steps:
            t = sorted(d[-steps:])
            k.update(timed=steps, avg_ns=sum(t) / steps, min_ns=t[0], max_ns=t[-1], median_ns=t[steps // 2])
        sec = k["avg_ns"] * 1e-9
        a = alg.get(key) if key else None
        if a:
            k["alg_read_bytes"], k["alg_write_bytes"] = a["read_bytes"], a["write_bytes"]
            k["alg_gbs"] = (a["read_bytes"] + a["write_bytes"]) / sec / 1e9
            if a.get("flop"):
                k["alg_flop"] = a["flop"]
                k["alg_tflops"] = a["flop"] / sec / 1e12
                k["alg_frac"] = k["alg_tflops"] / PEAK_BF16_TFLOPS
        c = {p: counters[p].get(name, {}) for p in counters}
        fetch, write = c.get("fetch", {}), c.get("write", {})
        if "FETCH_SIZE" in fetch:
            k["read_bytes"] = fetch["FETCH_SIZE"] * 1024.0 * cal["FETCH_SIZE"]["factor"]
        if "WRITE_SIZE" in write:
            k["write_bytes"] = write["WRITE_SIZE"] * 1024.0 * cal["WRITE_SIZE"]["factor"]
        if "read_bytes" in k and "write_bytes" in k:
            k["bytes"] = k["read_bytes"] + k["write_bytes"]
            k["gbs"] = k["bytes"] / sec / 1e9
            k["hbm_frac"] = k["gbs"] / PEAK_HBM_GBS
        mf = c.get("mfma", {})
        if mf.get("SQ_INSTS_VALU_MFMA_MOPS_BF16"):
            k["mfma_flop"] = mf["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * FLOPS_PER_MOP
            k["mfma_tflops"] = k["mfma_flop"] / sec / 1e12
            k["mfma_frac"] = k["mfma_tflops"] / PEAK_BF16_TFLOPS
            # Cycles per XCD of the counter pass's own dispatch, over that
            # dispatch's time: the shader clock, and the share of the SIMDs'
            # cycles with a busy matrix pipe.
            if mf.get("GRBM_GUI_ACTIVE") and mf.get("dispatch_ns"):
                cyc = mf["GRBM_GUI_ACTIVE"] / xcds
                k["cycles_per_xcd"] = cyc
                k["clock_ghz"] = cyc / mf["dispatch_ns"]
                if "SQ_VALU_MFMA_BUSY_CYCLES" in mf:
                    k["mfma_busy"] = mf["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * cus * 4)
        lds = c.get("lds", {})
        if lds.get("SQ_LDS_IDX_ACTIVE"):
            k["lds_conflict"] = lds.get("SQ_LDS_BANK_CONFLICT", 0.0) / lds["SQ_LDS_IDX_ACTIVE"]
        k["counters"] = c
        kernels.append(k)
    return {"workload": workload, "bench_args": bench_args, "kernel_source_sha256_16": kernel_source_hash(),
            "harness_cmd": ["python3", "gated_gqa_causal_amd/rocprof_harness.py"] + sys.argv[1:],
            "calibration": cal, "cus": cus, "xcds": xcds, "commands": cmds, "root": ROOT,
            "python": sys.executable,
            "bench_trace_line": trace["bench"], "kernels": kernels}


def short_name(name: str) -> str:
    name = name.split("(")[0]
    return name[5:] if name.startswith("void ") else name


def fmt(v, spec):
    return "-" if v is None else format(v, spec)


def markdown(s: dict) -> str:
    b = s["bench_trace_line"]
    out = [f"# rocprofv3 summary: {s['workload']} {' '.join(s['bench_args'])}".rstrip(), "",
           f"Kernel source sha256 prefix `{s['kernel_source_sha256_16']}`; peaks: {PEAK_BF16_TFLOPS:.0f} TFLOP/s "
           f"dense bf16, {PEAK_HBM_GBS:.0f} GB/s HBM; {s['cus']} CUs in {s['xcds']} XCDs.", "",
           "Made by (from the repository root R):", "",
           "    " + " ".join(shlex.quote(x) for x in s.get("harness_cmd", [])), "",
           "which ran these passes (from /tmp with TMPDIR=/tmp):", ""]
    out += ["    " + " ".join(shlex.quote(x) for x in c).replace(s["python"], "python3").replace(s["root"], "$R")
            for c in s["commands"]]
    cal = s["calibration"]
    out += ["", "Byte counters scaled by a plain device copy: FETCH_SIZE x "
            f"{cal['FETCH_SIZE']['factor']:.3f}, WRITE_SIZE x {cal['WRITE_SIZE']['factor']:.3f}.",
            f"bench.py's own event timing in the trace pass: {b.get('kernels_ms')}, {b.get('ms_per_step')} ms/step.",
            "", "| Kernel | Launches (timed) | Avg (us) | Min / Max (us) | --stats avg (us) | alg TFLOP/s (frac) | MFMA exec TFLOP/s (frac) "
            "| MFMA busy | Clock (GHz) | HBM read / write (MiB) | HBM GB/s (frac) | alg MiB r / w | alg GB/s | LDS conflict |",
            "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    others = []
    for k in s["kernels"]:
        if k["key"] is None:
            others.append(k)
            continue
        g = k.get
        mib = lambda x: None if x is None else x / 2 ** 20
        out.append("| `{}` | {} ({}) | {} | {} / {} | {} | {} | {} | {} | {} | {} / {} | {} | {} / {} | {} | {} |".format(
            short_name(k["name"]), k["calls"], k.get("timed", "all"), fmt(k["avg_ns"] / 1e3, ".1f"),
            fmt(k["min_ns"] / 1e3, ".1f"), fmt(k["max_ns"] / 1e3, ".1f"), fmt(k["stats_avg_ns"] / 1e3, ".1f"),
            "-" if g("alg_tflops") is None else f"{k['alg_tflops']:.0f} ({k['alg_frac']:.3f})",
            "-" if g("mfma_tflops") is None else f"{k['mfma_tflops']:.0f} ({k['mfma_frac']:.3f})",
            fmt(g("mfma_busy"), ".3f"), fmt(g("clock_ghz"), ".2f"),
            fmt(mib(g("read_bytes")), ".1f"), fmt(mib(g("write_bytes")), ".1f"),
            "-" if g("gbs") is None else f"{k['gbs']:.0f} ({k['hbm_frac']:.3f})",
            fmt(mib(g("alg_read_bytes")), ".1f"), fmt(mib(g("alg_write_bytes")), ".1f"),
            fmt(g("alg_gbs"), ".0f"), fmt(None if g("lds_conflict") is None else 100 * k["lds_conflict"], ".2f")
            + ("" if g("lds_conflict") is None else "%")))
    if others:
        out += ["", "Other kernels in the trace (not the library's): " + "; ".join(
            f"`{short_name(k['name'])}` {k['calls']} x {k['avg_ns'] / 1e3:.1f} us" for k in others) + "."]
    out += ["", "Avg, min and max are over the launches of the timed steps (the last `steps` dispatches of each",
            "kernel); `--stats avg` is rocprofv3's own average over every launch, warmup and set-up included.",
            "Rates divide by the timed average; counters are the means over each counter pass's timed steps,",
            "and the clock and matrix-pipe share come from those dispatches' own times."]
    return "\n".join(out) + "\n"


def cmd_run(a) -> int:
    out_dir = os.path.abspath(a.out or os.path.join("rocprof_out", a.workload))
    os.makedirs(out_dir, exist_ok=True)
    extra = shlex.split(a.bench_args)
    base = ["--workload", a.workload, "--no-cpu-baseline"] + extra
    log(f"workload {a.workload} {' '.join(extra)} -> {out_dir}")
    if a.calibration:
        with open(a.calibration) as f:
            cal = json.load(f)
        cal = cal.get("calibration", cal)
        log(f"calibration from {a.calibration}")
    else:
        cal = calibrate(out_dir, a.pmc_timeout)
    cmds = []
    # (no second spread run: the summary takes the last `steps` launches)
    trace = run_pass("trace", ["--kernel-trace", "--stats"],
                     base + ["--steps", str(a.steps), "--warmup", str(a.warmup), "--no-spread"], out_dir,
                     a.trace_timeout)
    cmds.append(trace["cmd"])
    counters = {}
    for name, ctrs in PASSES.items():
        # Counts do not depend on the clock: no pre-heat under the counters.
        r = run_pass(name, ["--pmc"] + ctrs, base + ["--steps", str(a.pmc_steps), "--warmup", "1",
                                                     "--preheat-ms", "0", "--no-spread"],
                     out_dir, a.pmc_timeout)
        counters[name] = read_counters(r["dir"], last=a.pmc_steps)
        cmds.append(r["cmd"])
    s = summarise(a.workload, extra, trace, counters, cal, cmds, a.cus, a.xcds)
    with open(os.path.join(out_dir, "summary.json"), "w") as f:
        json.dump(s, f, indent=1)
    md = markdown(s)
    with open(os.path.join(out_dir, "summary.md"), "w") as f:
        f.write(md)
    print(md, flush=True)
    return 0


def traffic_key(workload: str, bench_args) -> str:
    """Record key: the workload and the bench.py flags that change what runs."""
    return " ".join([workload] + list(bench_args))


def cmd_merge(a) -> int:
    for path in a.summaries:
        with open(path) as f:
            s = json.load(f)
        wkey = traffic_key(s["workload"], s["bench_args"])
        for key, tpath in TRAFFIC.items():
            k = next((k for k in s["kernels"] if k["key"] == key and "bytes" in k), None)
            if k is None:
                continue
            try:
                with open(tpath) as f:
                    rec = json.load(f)
            except (OSError, ValueError):
                rec = {}
            rec.setdefault("workloads", {})[wkey] = {
                "kernel": short_name(k["name"]), "kernel_source_sha256_16": s["kernel_source_sha256_16"],
                "fetch_bytes_per_launch": round(k["read_bytes"]), "write_bytes_per_launch": round(k["write_bytes"]),
                "bytes_per_launch": round(k["bytes"]),
                "calibration": {c: round(v["factor"], 4) for c, v in s["calibration"].items()}}
            rec["workloads"] = dict(sorted(rec["workloads"].items()))
            with open(tpath, "w") as f:
                json.dump(rec, f, indent=1)
                f.write("\n")
            log(f"{tpath}: {wkey}: {k['bytes'] / 2 ** 20:.1f} MiB per launch")
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--workload", default="c2_dense_s8192_g4")
    r.add_argument("--bench-args", default="", help="extra bench.py flags, e.g. \"--weights\"")
    r.add_argument("--out", default=None, help="output folder (default rocprof_out/<workload>)")
    r.add_argument("--calibration", default=None, help="summary.json (or calibration JSON) of an earlier run")
    r.add_argument("--steps", type=int, default=20)
    r.add_argument("--warmup", type=int, default=3)
    r.add_argument("--pmc-steps", type=int, default=3)
    r.add_argument("--trace-timeout", type=int, default=240)
    r.add_argument("--pmc-timeout", type=int, default=120)
    r.add_argument("--cus", type=int, default=256)
    r.add_argument("--xcds", type=int, default=8)
    m = sub.add_parser("merge")
    m.add_argument("summaries", nargs="+")
    a = ap.parse_args()
    return cmd_run(a) if a.cmd == "run" else cmd_merge(a)


if __name__ == "__main__":
    sys.exit(main())
