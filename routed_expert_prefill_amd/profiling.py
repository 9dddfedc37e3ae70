"""Summaries of rocprofv3 output (kernel traces and counter runs).

  python -m routed_expert_prefill_amd.profiling trace <run_results.db> [--skip N]
      per-kernel table (calls, total, average, share) of a --kernel-trace run;
      with --skip N also each kernel's average over its calls after the first N
  python -m routed_expert_prefill_amd.profiling traffic --fetch <csv> --write <csv>
          --kernel <name prefix> --workload <name> --out <json>
      HBM bytes per launch of one kernel from a FETCH_SIZE run and a
      WRITE_SIZE run (--output-format csv), each scaled by what the same
      counter reads for the 1 GiB device copy that bench.py --copy-calibration
      runs in the same process; records the kernel source hash bench.py checks.
  python -m routed_expert_prefill_amd.profiling mfma --csv <csv> --kernel <name prefix>
          [--avg-us <average duration from a kernel trace>]
      MFMA counters per launch of one kernel from a run with
      --pmc MfmaUtil MfmaFlopsBF16 SQ_INSTS_VALU_MFMA_MOPS_F8 GRBM_GUI_ACTIVE:
      the share of SIMD cycles the matrix units were busy (MfmaUtil, the
      busy cycles of all SIMDs over active cycles times SIMDs), the flops the
      matrix units executed (bf16, and fp8 as MOPS x 512), and with --avg-us
      the executed rate.
"""
import argparse
import csv
import json
import os
import sqlite3
import sys


def trace_table(db, skip=0):
    """Per-kernel table; with skip > 0 also the average of each kernel's
    calls after its first `skip` (the warm-up calls of the run)."""
    c = sqlite3.connect(db)
    rows = c.execute("select name, total_calls, total_duration, average, percentage "
                     "from top_kernels order by total_duration desc").fetchall()
    steady = {}
    if skip > 0:
        per = {}
        for name, dur in c.execute("select name, duration from kernels order by start"):
            per.setdefault(name, []).append(dur / 1000.0)
        steady = {n: sum(v[skip:]) / len(v[skip:]) for n, v in per.items() if len(v) > skip}
    head = "| kernel | calls | total (us) | average (us) | share |"
    rule = "|---|---|---|---|---|"
    if skip > 0:
        head += f" average after the first {skip} calls (us) |"
        rule += "---|"
    out = [head, rule]
    for name, calls, tot, avg, pct in rows:
        line = f"| `{name.split('(')[0]}` | {calls} | {tot:.1f} | {avg:.2f} | {pct:.2f}% |"
        if skip > 0:
            line += f" {steady[name]:.2f} |" if name in steady else " — |"
        out.append(line)
    return "\n".join(out)


def _per_kernel(csv_path, counter):
    vals = {}
    with open(csv_path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return vals


def _match(vals, prefix):
    hits = [v for k, v in vals.items() if k.startswith(prefix)]
    if not hits:
        raise SystemExit(f"no dispatch of a kernel starting with {prefix!r}")
    flat = [x for v in hits for x in v]
    return sum(flat) / len(flat), len(flat)


def _copy_kib(vals):
    # the 1 GiB copy is the largest single dispatch of a copy kernel in the run
    best = None
    for name, v in vals.items():
        if "copy" in name.lower() or "elementwise" in name.lower():
            m = max(v)
            best = m if best is None or m > best else best
    if best is None:
        raise SystemExit("no copy kernel in the counter run (run bench.py with --copy-calibration)")
    return best


def traffic(args):
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench

    fetch = _per_kernel(args.fetch, "FETCH_SIZE")
    write = _per_kernel(args.write, "WRITE_SIZE")
    f_kib, nf = _match(fetch, args.kernel)
    w_kib, nw = _match(write, args.kernel)
    gib_kib = (1 << 30) / 1024.0
    f_scale = gib_kib / _copy_kib(fetch)   # copy reads exactly 1 GiB
    w_scale = gib_kib / _copy_kib(write)   # and writes exactly 1 GiB
    rec = {
        "kernel": args.kernel,
        "workload": args.workload,
        "fetch_kib_raw": round(f_kib, 1),
        "write_kib_raw": round(w_kib, 1),
        "fetch_scale": round(f_scale, 4),
        "write_scale": round(w_scale, 4),
        "dispatches": [nf, nw],
        "bytes_per_launch": int(round((f_kib * f_scale + w_kib * w_scale) * 1024)),
        "source_sha": bench.source_hash(),
    }
    with open(args.out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


def mfma(args):
    names = ["MfmaUtil", "MfmaFlopsBF16", "SQ_INSTS_VALU_MFMA_MOPS_F8", "GRBM_GUI_ACTIVE"]
    rec = {"kernel": args.kernel}
    for n in names:
        v, cnt = _match(_per_kernel(args.csv, n), args.kernel)
        rec[n] = v
        rec["dispatches"] = cnt
    flops = rec["MfmaFlopsBF16"] + rec["SQ_INSTS_VALU_MFMA_MOPS_F8"] * 512
    rec["executed_flops"] = flops
    lines = [f"| quantity ({args.kernel}, mean of {rec['dispatches']} launches) | value |", "|---|---|",
             f"| MfmaUtil (matrix-unit busy share of SIMD cycles) | {rec['MfmaUtil']:.1f}% |",
             f"| executed MFMA flops, bf16 | {rec['MfmaFlopsBF16'] / 1e12:.4f} TFLOP |",
             f"| executed MFMA flops, fp8 | {rec['SQ_INSTS_VALU_MFMA_MOPS_F8'] * 512 / 1e12:.4f} TFLOP |",
             f"| GRBM_GUI_ACTIVE | {rec['GRBM_GUI_ACTIVE']:.0f} cycles |"]
    if args.avg_us:
        lines.append(f"| executed rate at {args.avg_us:.1f} us per launch | "
                     f"{flops / (args.avg_us * 1e-6) / 1e12:.1f} TFLOP/s |")
    print("\n".join(lines))


def main(argv=None):
    argv = list(sys.argv[1:] if argv is None else argv)
    if argv and argv[0].endswith(".db"):
        argv = ["trace"] + argv  # older form: a bare database path
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--skip", type=int, default=0,
                   help="also average each kernel over its calls after the first SKIP")
    f = sub.add_parser("traffic")
    f.add_argument("--fetch", required=True)
    f.add_argument("--write", required=True)
    f.add_argument("--kernel", required=True)
    f.add_argument("--workload", required=True)
    f.add_argument("--out", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("--csv", required=True)
    m.add_argument("--kernel", required=True)
    m.add_argument("--avg-us", type=float, default=None)
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        print(trace_table(a.db, a.skip))
    elif a.cmd == "mfma":
        mfma(a)
    else:
        traffic(a)


if __name__ == "__main__":
    main()
