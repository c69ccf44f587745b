"""HBM traffic of the fused GEMM from rocprofv3 byte counters.

Reads two rocprofv3 ``--pmc`` counter files of the same ``bench.py
--copy-calibration`` run (one with FETCH_SIZE, one with WRITE_SIZE; both in
KiB per dispatch), scales every reading by what the counter gives for a plain
1 GiB streaming copy (the calibration dispatches), and writes the bytes per
bench step of the GEMM launches, stamped with the kernel source hash so that
a later kernel change invalidates them.

    python w8a8_int8_quantized_token_amd/traffic.py FETCH.csv WRITE.csv \\
        --runs 2 --out profiles/gemm_traffic.json

``--runs`` is the number of bench steps the profiled run executed (warm-up
plus timed).
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
GEMM_SOURCE = os.path.join(HERE, "csrc", "gemm_i8.hip")
COPY_BYTES = 1 << 30
GEMM_KERNEL = "gemm_i8_kernel"
CALIB_KERNEL = "bitwise_not"


def per_dispatch(path: str, counter: str):
    """{dispatch id: (kernel name, grid size, summed counter value)}."""
    out = {}
    acc = collections.defaultdict(float)
    for row in csv.DictReader(open(path)):
        if row["Counter_Name"] != counter:
            continue
        d = int(row["Dispatch_Id"])
        acc[d] += float(row["Counter_Value"])
        out[d] = (row["Kernel_Name"], int(row["Grid_Size"]))
    return {d: (name, grid, acc[d]) for d, (name, grid) in out.items()}


def calibrate(disp) -> float:
    """Bytes per counter unit: each calibration dispatch (a streaming 1 GiB
    elementwise copy, bitwise_not of uint8) reads and writes exactly
    COPY_BYTES."""
    cands = sorted((v for name, _, v in disp.values() if CALIB_KERNEL in name), reverse=True)
    if not cands:
        raise SystemExit("no calibration dispatch found: profile bench.py with --copy-calibration")
    top = cands[:3]
    return COPY_BYTES / sorted(top)[len(top) // 2]


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("fetch_csv")
    ap.add_argument("write_csv")
    ap.add_argument("--runs", type=int, required=True, help="bench steps in the profiled run")
    ap.add_argument("--out", required=True)
    args = ap.parse_args()

    rec = {"gemm_source_sha256": hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest(),
           "copy_bytes": COPY_BYTES, "runs": args.runs}
    total = 0.0
    for key, path, counter in (("fetch", args.fetch_csv, "FETCH_SIZE"),
                               ("write", args.write_csv, "WRITE_SIZE")):
        disp = per_dispatch(path, counter)
        factor = calibrate(disp)
        gemm = [(d, g, v) for d, (name, g, v) in sorted(disp.items()) if GEMM_KERNEL in name]
        if not gemm or len(gemm) % args.runs:
            raise SystemExit(f"{len(gemm)} GEMM dispatches do not split into {args.runs} runs")
        per_run = len(gemm) // args.runs
        last = gemm[-per_run:]
        bytes_last = [v * factor for _, _, v in last]
        rec[key] = {"counter": counter, "bytes_per_counter_unit": factor,
                    "launches_per_step": per_run,
                    "per_launch_bytes": [round(b) for b in bytes_last],
                    "per_launch_grid": [g for _, g, _ in last],
                    "bytes_per_step": round(sum(bytes_last))}
        total += sum(bytes_last)
    rec["bytes_per_step"] = round(total)
    with open(args.out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps({"bytes_per_step": rec["bytes_per_step"],
                      "fetch_factor": rec["fetch"]["bytes_per_counter_unit"],
                      "write_factor": rec["write"]["bytes_per_counter_unit"]}))


if __name__ == "__main__":
    main()
