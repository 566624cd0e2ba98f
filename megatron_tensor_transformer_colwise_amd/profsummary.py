"""Summaries of rocprofv3 results databases.

Kernel traces: the per-kernel summary (calls, total and average duration in
us) that rocprofv3 stores in the ``top_kernels`` view.

Counter runs (``--pmc``): per kernel, the range over its dispatches of each
collected counter, the dispatch duration, and, when GRBM_GUI_ACTIVE and
SQ_VALU_MFMA_BUSY_CYCLES were both collected, the matrix-core busy share
SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs) and the
mean graphics clock GRBM_GUI_ACTIVE / 8 / duration.

Usage: python -m megatron_tensor_transformer_colwise_amd.profsummary RESULTS_DB
       python -m megatron_tensor_transformer_colwise_amd.profsummary --pmc RESULTS_DB
"""
import collections
import sqlite3
import sys

XCDS = 8
SIMDS = 1024


def summary(db_path: str) -> str:
    db = sqlite3.connect(db_path)
    rows = db.execute("select name, total_calls, total_duration, average, percentage "
                      "from top_kernels order by total_duration desc").fetchall()
    lines = [f"{'calls':>6} {'total_us':>12} {'avg_us':>10} {'pct':>6}  kernel"]
    for name, calls, total, avg, pct in rows:
        short = name if len(name) < 110 else name[:107] + "..."
        lines.append(f"{calls:>6} {total:>12.1f} {avg:>10.2f} {pct:>6.2f}  {short}")
    return "\n".join(lines)


def _short(name: str) -> str:
    name = name.replace("tpk::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    name = name.split("(")[0] if not name.startswith("void at::") else name[:60]
    return name.replace("void ", "")


def pmc_summary(db_path: str) -> str:
    db = sqlite3.connect(db_path)
    rows = db.execute("select dispatch_id, kernel_name, counter_name, sum(value), min(start), max(end) "
                      "from counters_collection group by dispatch_id, counter_name "
                      "order by dispatch_id").fetchall()
    disp = collections.OrderedDict()
    for did, name, counter, value, start, end in rows:
        d = disp.setdefault(did, {"name": _short(name), "us": (end - start) / 1000.0})
        d[counter] = value
    per_kernel = collections.OrderedDict()
    for d in disp.values():
        per_kernel.setdefault(d["name"], []).append(d)
    lines = []
    for name, ds in per_kernel.items():
        counters = sorted(k for k in ds[0] if k not in ("name", "us"))
        us = [d["us"] for d in ds]
        parts = [f"{name}: {len(ds)} dispatches, {min(us):.1f}-{max(us):.1f} us"]
        if "GRBM_GUI_ACTIVE" in counters and "SQ_VALU_MFMA_BUSY_CYCLES" in counters:
            busy = [d["SQ_VALU_MFMA_BUSY_CYCLES"] / (d["GRBM_GUI_ACTIVE"] / XCDS * SIMDS) for d in ds]
            clk = [d["GRBM_GUI_ACTIVE"] / XCDS / d["us"] / 1e3 for d in ds if d["us"] > 0]
            parts.append(f"MFMA busy {100 * min(busy):.1f}-{100 * max(busy):.1f}%")
            if clk:
                parts.append(f"clock {min(clk):.2f}-{max(clk):.2f} GHz")
        for c in counters:
            v = [d[c] for d in ds]
            parts.append(f"{c} {min(v):.4g}-{max(v):.4g}")
        lines.append("; ".join(parts))
    return "\n".join(lines)


if __name__ == "__main__":
    if sys.argv[1] == "--pmc":
        print(pmc_summary(sys.argv[2]))
    else:
        print(summary(sys.argv[1]))
