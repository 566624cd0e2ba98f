"""Summaries of rocprofv3 results databases.

Kernel traces: the per-kernel summary (calls, total and average duration in
us) that rocprofv3 stores in the ``top_kernels`` view.

Counter runs (``--pmc``): per kernel, the range over its dispatches of each
collected counter, the dispatch duration, and, when GRBM_GUI_ACTIVE and
SQ_VALU_MFMA_BUSY_CYCLES were both collected, the matrix-core busy share
SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs) and the
mean graphics clock GRBM_GUI_ACTIVE / 8 / duration.

Per-workload reports (``bench.py --configs`` JSON lines): one markdown table
row per measured call, its synchronised median/minimum and, where measured,
its back-to-back mean (calls issued without synchronisation, as in a model).

Usage: python -m megatron_tensor_transformer_colwise_amd.profsummary RESULTS_DB
       python -m megatron_tensor_transformer_colwise_amd.profsummary --pmc RESULTS_DB
       python -m megatron_tensor_transformer_colwise_amd.profsummary --configs JSONL
"""
import collections
import json
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
    # launches of one kernel that do different matrix work (a main launch and
    # a split-k tail) are told apart by their MFMA op count
    per_kernel = collections.OrderedDict()
    for d in disp.values():
        key = (d["name"], d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16"))
        per_kernel.setdefault(key, []).append(d)

    def describe(ds):
        counters = sorted(k for k in ds[0] if k not in ("name", "us"))
        us = [d["us"] for d in ds]
        parts = [f"{len(ds)} dispatches, {min(us):.1f}-{max(us):.1f} us"]
        if "GRBM_GUI_ACTIVE" in counters and "SQ_VALU_MFMA_BUSY_CYCLES" in counters:
            busy = [d["SQ_VALU_MFMA_BUSY_CYCLES"] / (d["GRBM_GUI_ACTIVE"] / XCDS * SIMDS) for d in ds]
            clk = [d["GRBM_GUI_ACTIVE"] / XCDS / d["us"] / 1e3 for d in ds if d["us"] > 0]
            parts.append(f"MFMA busy {100 * min(busy):.1f}-{100 * max(busy):.1f}%")
            if clk:
                parts.append(f"clock {min(clk):.2f}-{max(clk):.2f} GHz")
        for c in counters:
            v = [d[c] for d in ds]
            parts.append(f"{c} {min(v):.4g}-{max(v):.4g}")
        return "; ".join(parts)

    lines = []
    for (name, _), ds in per_kernel.items():
        lines.append(f"{name}: " + describe(ds))
        if len(ds) > 2:  # the first dispatch of a pass also counts what ran before it on the idle chip
            lines.append(f"{name}, after the first: " + describe(ds[1:]))
    return "\n".join(lines)


def _pct(tflops) -> float:
    return round(tflops / 25.0, 2)  # of the published 2500 TFLOP/s


def configs_table(path: str) -> str:
    rows = [json.loads(line) for line in open(path) if line.strip()]
    out = ["| workload | call | median ms | min ms | TFLOP/s | % MFMA peak | back-to-back ms (TFLOP/s, % peak) "
           "| shard-sum GB/s (% HBM) |",
           "|---|---|---|---|---|---|---|---|"]

    def row(w, call, ms="", mn="", tf="", pct="", b2b="", gbs=""):
        out.append(f"| {w} | {call} | {ms} | {mn} | {tf} | {pct} | {b2b} | {gbs} |")

    def b2b(r, prefix=""):
        k = prefix + "b2b_ms"
        if k not in r:
            return ""
        tf = r[prefix + "b2b_tflops"]
        return f"{r[k]} ({tf}, {_pct(tf)})"

    for r in rows:
        w = r["workload"]
        if w == "packed_single_stream":
            row(f"{w} ({r['shape']})", r["call"], r["ms"], r["min_ms"], r["tflops"], r["pct_mfma_peak"])
            row(w, "all 4 ranks + the sum of 8 partials", r["all_ranks_and_sum_ms"], "", r["all_ranks_tflops"],
                _pct(r["all_ranks_tflops"]))
        elif w == "llama70b_mlp_backward_t8":
            row(f"{w} ({r['shape']})", f"{r['call']}: recomputed pre-activation + 5 GEMMs + transposes", r["ms"],
                r["min_ms"], r["tflops"], r["pct_mfma_peak"])
        elif w == "llama70b_attn_backward_t8":
            row(f"{w} ({r['shape']})", r["call"], r["ms"], r["min_ms"], r["tflops"], r["pct_mfma_peak"])
            row(w, r["core_call"], r["core_ms"], r["core_min_ms"], r["core_tflops"], r["core_pct_mfma_peak"])
        elif w == "vocab_parallel_ce":
            row(f"{w} ({r['shape']})", r["call"], r["ms"], r["min_ms"], r["tflops"], r["pct_mfma_peak"])
            row(w, "statistics kernel alone (one rank's [m, v/t] float32 logits)", r["stats_ms"], gbs=
                f"{r['stats_gbs']} ({round(r['stats_gbs'] / 80, 1)})")
            row(w, "all 4 ranks + the combination", r["all_ranks_and_combine_ms"], "", r["all_ranks_tflops"],
                _pct(r["all_ranks_tflops"]))
        elif "call" in r:
            row(w, r["call"], r["ms"], r["min_ms"], r["tflops"], r["pct_mfma_peak"], b2b(r),
                f"{r['shard_sum_gbs']} ({r['shard_sum_pct_hbm']})")
            if "grouped_all_ranks_ms" in r:
                row(w, "tp_shard_mlp_group (all ranks, one launch pair)", r["grouped_all_ranks_ms"],
                    r["grouped_min_ms"], r["grouped_tflops"], _pct(r["grouped_tflops"]))
        else:
            row(w, "tp_shard_attn (rank 0)", r["attn_call_ms"], r["attn_min_ms"], r["attn_tflops"],
                r["attn_pct_mfma_peak"], b2b(r, "attn_"))
            row(w, "tp_shard_mlp (rank 0)", r["mlp_call_ms"], r["mlp_min_ms"], r["mlp_tflops"],
                r["mlp_pct_mfma_peak"], b2b(r, "mlp_"))
            row(w, "shard-sum of the MLP partials + f32 residual", r["shard_sum_ms"], r["shard_sum_min_ms"],
                gbs=f"{r['shard_sum_gbs']} ({r['shard_sum_pct_hbm']})")
            row(w, "whole block, all ranks (forward)", r["block_step_ms"], r["block_step_min_ms"],
                r["block_step_tflops"], _pct(r["block_step_tflops"]))
            if "block_backward_step_ms" in r:
                row(w, "whole block backward, all ranks (after the forward)", r["block_backward_step_ms"],
                    r["block_backward_step_min_ms"], r["block_backward_step_tflops"],
                    _pct(r["block_backward_step_tflops"]))
                row(w, "sum of the MLP dX partials + RMSNorm backward + dZ (dh1, float32 and bf16, dgain)",
                    r["norm_backward_ms"], gbs=f"{r['norm_backward_gbs']} ({round(r['norm_backward_gbs'] / 80, 1)})")
            if "sequence_parallel_backward_step_ms" in r:
                row(w, "whole block backward, sequence-parallel form", r["sequence_parallel_backward_step_ms"], "",
                    r["sequence_parallel_backward_step_tflops"], _pct(r["sequence_parallel_backward_step_tflops"]))
            if "saved_backward_step_ms" in r:
                row(w, "whole block forward keeping its activations, all ranks", r["saving_forward_step_ms"])
                row(w, "whole block backward from the saved activations, all ranks", r["saved_backward_step_ms"],
                    r["saved_backward_step_min_ms"], r["saved_backward_step_tflops"],
                    _pct(r["saved_backward_step_tflops"]))
            if "sequence_parallel_step_ms" in r:
                row(w, "whole block, sequence-parallel form", r["sequence_parallel_step_ms"], "",
                    r["sequence_parallel_step_tflops"], _pct(r["sequence_parallel_step_tflops"]))
    return "\n".join(out)


if __name__ == "__main__":
    if sys.argv[1] == "--pmc":
        print(pmc_summary(sys.argv[2]))
    elif sys.argv[1] == "--configs":
        print(configs_table(sys.argv[2]))
    else:
        print(summary(sys.argv[1]))
