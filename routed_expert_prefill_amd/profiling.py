"""Print a per-kernel table (calls, total, average, share) from a rocprofv3
kernel-trace database: python -m routed_expert_prefill_amd.profiling <run_results.db>."""
import sqlite3
import sys


def main(db):
    c = sqlite3.connect(db)
    rows = c.execute("select name, total_calls, total_duration, average, percentage "
                     "from top_kernels order by total_duration desc").fetchall()
    print("| kernel | calls | total (us) | average (us) | share |")
    print("|---|---|---|---|---|")
    for name, calls, tot, avg, pct in rows:
        print(f"| `{name.split('(')[0]}` | {calls} | {tot:.1f} | {avg:.2f} | {pct:.2f}% |")


if __name__ == "__main__":
    main(sys.argv[1])
