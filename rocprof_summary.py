#!/usr/bin/env python3
"""Summaries of rocprofv3 results (its SQLite ``*_results.db`` files) for ``profiles/``.

  python rocprof_summary.py trace DB --command CMD
      kernel-trace summary: calls, mean / median / min / max duration per kernel.
      With --bench-out FILE (the traced bench.py run's stdout) it also quotes that run's own
      JSON line: its value and its per-launch event timing, for comparison with the trace.
  python rocprof_summary.py pmc DB --command CMD
      per-kernel mean of each collected counter, plus MFMA utilisation, LDS bank-conflict
      rate and VALU instruction mix when their counters are present.
  python rocprof_summary.py traffic --fetch DB --write DB --copy-fetch DB --copy-write DB
                           --workload NAME --command CMD [--out JSON]
      HBM bytes per launch of the attention kernel: FETCH_SIZE and WRITE_SIZE (KiB per
      dispatch), each scaled by what the same counter reads for a plain copy of known
      size (bench.py --calibrate-copy).  Writes the JSON bench.py reads, stamped with the
      hash of the kernel sources, so bench.py reports null once the kernel has changed.
      A workload NAME/splitkv records the split-KV attention kernel of NAME.

Summaries are printed as text; redirect them into profiles/.
"""

from __future__ import annotations

import argparse
import json
import os
import sqlite3
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_KEY = "fa_fwd_kernel"
SIMDS = 256 * 4
XCCS = 8


def _rows(db, sql):
    con = sqlite3.connect(db)
    try:
        return list(con.execute(sql))
    finally:
        con.close()


def short(name, n=96):
    return name if len(name) <= n else name[:n - 3] + "..."


def bench_of_run(path):
    """Lines comparing the trace with the bench.py line printed by the traced run itself:
    its value and its own per-launch event timing (mean, from HIP events)."""
    line = None
    with open(path, errors="replace") as f:
        for raw in f:
            raw = raw.strip()
            if raw.startswith('{"metric"'):
                line = json.loads(raw)
    if line is None:
        return ["", "# bench.py line of the same run: not found in " + os.path.basename(path)]
    k = line.get("kernel_us", {})
    out = ["", "# bench.py line of the same run (HIP events on the launch stream):",
           f"#   workload {line['config']['workload']}, path {line['config'].get('path')}, "
           f"kernel {line['config'].get('kernel')}",
           f"#   value {line['value']} {line['unit']}, kernel_us mean {k.get('mean')} "
           f"median {k.get('median')} min {k.get('min')}"]
    if "ms_per_step" in line:
        out.append(f"#   ms_per_step {line['ms_per_step']}")
    pc = line.get("peak_check") or {}
    if "mfma_loop_tflops" in pc:
        # The box's own real-data MFMA rate: box-to-box clock spread shows here.
        frac = (f", the run's value is {line['value'] / pc['mfma_loop_tflops']:.3f} of it"
                if line.get("unit") == "TFLOP/s" else "")
        out.append(f"#   peak_check: bf16 MFMA loop on random operands {pc['mfma_loop_tflops']} "
                   f"TFLOP/s at {pc.get('mfma_loop_clock_ghz')} GHz (derived peak "
                   f"{pc.get('derived_peak_tflops')}){frac}")
    return out


def _kernel_rows(db):
    """(name, duration ns) of every dispatch, in order of start time when the table has one."""
    try:
        return _rows(db, "select name, duration from kernels order by start")
    except sqlite3.OperationalError:
        return _rows(db, "select name, duration from kernels")


def _bench_steps(path):
    """`steps` of the bench.py line in the traced run's stdout, or None."""
    with open(path, errors="replace") as f:
        for raw in f:
            raw = raw.strip()
            if raw.startswith('{"metric"'):
                return json.loads(raw).get("steps")
    return None


def trace(db, command, bench_out=None):
    by = {}
    for name, dur in _kernel_rows(db):
        by.setdefault(name, []).append(dur / 1e3)  # ns -> us, in dispatch order
    out = [f"# rocprofv3 kernel trace summary", f"# command: {command}",
           f"# source: {os.path.basename(db)}", "",
           f"{'kernel':<98} {'calls':>5} {'mean_us':>9} {'median_us':>9} {'min_us':>9} {'max_us':>9}"]
    for name, d in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"{short(name):<98} {len(d):>5} {statistics.mean(d):>9.1f} "
                   f"{statistics.median(d):>9.1f} {min(d):>9.1f} {max(d):>9.1f}")
    if bench_out:
        steps = _bench_steps(bench_out)
        timed = [(n, d[-2 * steps:]) for n, d in by.items() if steps and len(d) >= 2 * steps]
        if timed:
            # bench.py times K launches back to back, then K more with an event pair around
            # each: the last 2K dispatches of each kernel are the timed ones (the rest are the
            # warm-up, at a ramping clock).
            out += ["", f"# the {2 * steps} timed dispatches of each kernel (the last ones of the run):",
                    f"{'kernel':<98} {'calls':>5} {'mean_us':>9} {'median_us':>9}"]
            for name, d in sorted(timed, key=lambda kv: -sum(kv[1])):
                out.append(f"{short(name):<98} {len(d):>5} {statistics.mean(d):>9.1f} "
                           f"{statistics.median(d):>9.1f}")
        out += bench_of_run(bench_out)
    return "\n".join(out)


def pmc_means(db):
    rows = _rows(db, "select name, dispatch_id, counter_name, counter_value from pmc_events")
    per = {}
    for name, disp, cname, val in rows:
        d = per.setdefault(name, {}).setdefault(cname, {})
        d[disp] = d.get(disp, 0.0) + val   # sum the counter's instances within a dispatch
    return {k: {c: statistics.mean(v.values()) for c, v in cs.items()} for k, cs in per.items()}


def pmc(db, command):
    means = pmc_means(db)
    out = [f"# rocprofv3 counter summary (mean per dispatch)", f"# command: {command}",
           f"# source: {os.path.basename(db)}", ""]
    for name, cs in means.items():
        out.append(f"kernel: {short(name, 140)}")
        for c in sorted(cs):
            out.append(f"  {c:<32} {cs[c]:>18.1f}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in cs and "GRBM_GUI_ACTIVE" in cs:
            gui = cs["GRBM_GUI_ACTIVE"] / XCCS
            out.append(f"  {'derived MFMA busy %':<32} {100 * cs['SQ_VALU_MFMA_BUSY_CYCLES'] / (gui * SIMDS):>18.1f}"
                       f"   (MFMA busy cycles / (GUI-active cycles per XCC x {SIMDS} SIMDs))")
        if "SQ_LDS_BANK_CONFLICT" in cs and "SQ_LDS_IDX_ACTIVE" in cs:
            act = cs["SQ_LDS_IDX_ACTIVE"]
            conf = cs["SQ_LDS_BANK_CONFLICT"]
            out.append(f"  {'derived LDS conflict cycles %':<32} {100 * conf / act if act else 0:>18.2f}"
                       f"   (bank-conflict stall cycles / LDS indexed-active cycles)")
        if "TCC_HIT_sum" in cs and "TCC_MISS_sum" in cs:
            tot = cs["TCC_HIT_sum"] + cs["TCC_MISS_sum"]
            out.append(f"  {'derived L2 hit %':<32} {100 * cs['TCC_HIT_sum'] / tot if tot else 0:>18.2f}"
                       f"   (TCC hits / (hits + misses))")
        if "SQ_INSTS_VALU" in cs and "SQ_INSTS_MFMA" in cs:
            out.append(f"  {'derived VALU / MFMA insts':<32} {cs['SQ_INSTS_VALU'] / max(1, cs['SQ_INSTS_MFMA']):>18.2f}")
        out.append("")
    return "\n".join(out)


def _counter(db, cname, key):
    for name, cs in pmc_means(db).items():
        if key in name and cname in cs:
            return cs[cname]
    raise SystemExit(f"{cname} for a kernel matching '{key}' not found in {db}")


def traffic(a):
    sys.path.insert(0, ROOT)
    import bench

    fetch_kib = _counter(a.fetch, "FETCH_SIZE", KERNEL_KEY)
    write_kib = _counter(a.write, "WRITE_SIZE", KERNEL_KEY)
    cf_kib = _counter(a.copy_fetch, "FETCH_SIZE", "copyBuffer")
    cw_kib = _counter(a.copy_write, "WRITE_SIZE", "copyBuffer")
    f_fetch = bench.COPY_BYTES / (cf_kib * 1024.0)
    f_write = bench.COPY_BYTES / (cw_kib * 1024.0)
    hbm = fetch_kib * 1024.0 * f_fetch + write_kib * 1024.0 * f_write
    w, fp8 = bench.workload(a.workload.split("/")[0])   # NAME or NAME/splitkv
    algo = bench.algorithmic_bytes(w, fp8)
    path = a.out or bench.TRAFFIC_FILE
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {}
    sha = bench.kernel_source_hash()
    if data.get("kernel_source_sha") != sha:
        data = {"kernel_source_sha": sha, "workloads": {}}
    data["workloads"][a.workload] = {
        "hbm_bytes_per_launch": round(hbm),
        "fetch_kib_raw": fetch_kib, "write_kib_raw": write_kib,
        "copy_fetch_kib_raw": cf_kib, "copy_write_kib_raw": cw_kib,
        "fetch_scale": f_fetch, "write_scale": f_write,
        "algorithmic_bytes": algo, "command": a.command,
    }
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    return "\n".join([
        "# HBM traffic per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by a copy calibration",
        f"# command: {a.command}",
        f"# kernel sources sha256[:16]: {sha}", "",
        f"workload                     {a.workload}",
        f"FETCH_SIZE (KiB/dispatch)    {fetch_kib:.1f}   x scale {f_fetch:.4f}",
        f"WRITE_SIZE (KiB/dispatch)    {write_kib:.1f}   x scale {f_write:.4f}",
        f"copy of {bench.COPY_BYTES} B: FETCH_SIZE {cf_kib:.1f} KiB, WRITE_SIZE {cw_kib:.1f} KiB",
        f"HBM bytes per launch         {hbm:.0f}  ({hbm / 2**20:.1f} MiB)",
        f"algorithmic bytes            {algo}  ({algo / 2**20:.1f} MiB: q, k, v read once; o, lse written once)",
        f"ratio                        {hbm / algo:.2f}",
    ])


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    for n in ("trace", "pmc"):
        s = sub.add_parser(n)
        s.add_argument("db")
        s.add_argument("--command", default="")
        if n == "trace":
            s.add_argument("--bench-out", default=None,
                           help="stdout of the traced bench.py run, to quote its own timing")
    t = sub.add_parser("traffic")
    for k in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--workload"):
        t.add_argument(k, required=True)
    t.add_argument("--command", default="")
    t.add_argument("--out", default=None)
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        print(trace(a.db, a.command, a.bench_out))
    elif a.cmd == "pmc":
        print(pmc(a.db, a.command))
    else:
        print(traffic(a))
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
