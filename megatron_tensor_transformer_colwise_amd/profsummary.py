"""Prints the per-kernel summary (calls, total and average duration in us) that
rocprofv3 stores in the ``top_kernels`` view of its results database.

Usage: python -m megatron_tensor_transformer_colwise_amd.profsummary RESULTS_DB
"""
import sqlite3
import sys


def summary(db_path: str) -> str:
    db = sqlite3.connect(db_path)
    rows = db.execute("select name, total_calls, total_duration, average, percentage "
                      "from top_kernels order by total_duration desc").fetchall()
    lines = [f"{'calls':>6} {'total_us':>12} {'avg_us':>10} {'pct':>6}  kernel"]
    for name, calls, total, avg, pct in rows:
        short = name if len(name) < 110 else name[:107] + "..."
        lines.append(f"{calls:>6} {total:>12.1f} {avg:>10.2f} {pct:>6.2f}  {short}")
    return "\n".join(lines)


if __name__ == "__main__":
    print(summary(sys.argv[1]))
