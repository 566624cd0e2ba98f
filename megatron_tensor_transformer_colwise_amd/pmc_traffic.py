"""HBM traffic of one kernel from two rocprofv3 counter passes.

Reads the results databases of ``rocprofv3 --pmc FETCH_SIZE`` and
``rocprofv3 --pmc WRITE_SIZE`` runs of ``bench.py --pmc-pass``.  That mode
launches a plain device copy of a known size (the shard-sum kernel with one
partial, shard_sum_kernel<1>: n float32 read, n written) before the measured kernel, so each
counter is scaled by bytes_known / counter_reading_of_the_copy.  Writes the
per-launch traffic of the measured kernel, with the hash of the source it was
taken on, to a JSON file that bench.py reports while the source is unchanged.

A call of the measured entry point may be several dispatches (a main range
and a tail range of tiles); every dispatch whose name contains
KERNEL_SUBSTRING is summed and divided by CALLS.

Usage: python -m megatron_tensor_transformer_colwise_amd.pmc_traffic \\
           FETCH_DB WRITE_DB COPY_BYTES KERNEL_SUBSTRING CALLS SOURCE_FILE OUT_JSON
"""
import hashlib
import json
import sqlite3
import sys
from pathlib import Path


def per_dispatch(db_path: str, counter: str) -> list[tuple[str, float]]:
    db = sqlite3.connect(db_path)
    rows = db.execute("select dispatch_id, kernel_name, sum(value) from counters_collection "
                      "where counter_name = ? group by dispatch_id order by dispatch_id",
                      (counter,)).fetchall()
    return [(name, float(v)) for _, name, v in rows]


def source_hash(path: str) -> str:
    return hashlib.sha256(Path(path).read_bytes()).hexdigest()[:16]


def main(fetch_db, write_db, copy_bytes, kernel_sub, calls, source, out_json):
    copy_bytes = float(copy_bytes)
    calls = int(calls)
    res = {}
    for counter, db in (("FETCH_SIZE", fetch_db), ("WRITE_SIZE", write_db)):
        d = per_dispatch(db, counter)
        copy = [v for n, v in d if "shard_sum_kernel<1>" in n]
        kern = [v for n, v in d if kernel_sub in n]
        if not copy or not kern:
            raise SystemExit(f"{counter}: no copy or no '{kernel_sub}' dispatches in {db}")
        copy_kib = sorted(copy)[len(copy) // 2]
        scale = copy_bytes / (copy_kib * 1024.0)
        kern_kib = sum(kern) / calls
        res[counter] = {"copy_kib": copy_kib, "scale": scale, "kernel_kib_per_call": kern_kib,
                        "kernel_bytes": kern_kib * 1024.0 * scale, "dispatches": len(kern),
                        "calls": calls}
    out = {
        "kernel": kernel_sub,
        "source": Path(source).name,
        "source_sha256_16": source_hash(source),
        "copy_bytes_each_way": copy_bytes,
        "fetch": res["FETCH_SIZE"],
        "write": res["WRITE_SIZE"],
        "traffic_bytes_per_launch": res["FETCH_SIZE"]["kernel_bytes"] + res["WRITE_SIZE"]["kernel_bytes"],
    }
    Path(out_json).write_text(json.dumps(out, indent=2) + "\n")
    print(json.dumps(out, indent=2))


if __name__ == "__main__":
    main(*sys.argv[1:8])
