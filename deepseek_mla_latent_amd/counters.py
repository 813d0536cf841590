"""Per-kernel summary of rocprofv3 counter passes over ``bench.py``.

Each pass is one ``rocprofv3 --pmc <counters> --output-format csv -d <dir> -o k -- python3 bench.py
... --copy-probe-mib 1024`` run (one counter set per run: rocprofv3 does not split counters over
passes).  The 1 GiB device copy the bench runs first calibrates the byte counters: FETCH_SIZE and
WRITE_SIZE report KiB per dispatch in units that differ from a byte count by a fixed factor on this
chip, so each is scaled by (1 GiB) / (what it reads for the copy).

Per kernel (median over its dispatches):
  * fetch / write bytes: FETCH_SIZE, WRITE_SIZE x 1024 x their calibration factor;
  * MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs), the fraction of
    SIMD cycles the matrix cores were busy while the kernel ran;
  * MFMA FLOPs: SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (the counter counts units of 512 FLOPs).
GRBM_GUI_ACTIVE also counts cycles around a dispatch, so for kernels of a few microseconds the busy
fraction reads low; the FLOP count over the unprofiled kernel duration is the better rate there.

usage: python -m deepseek_mla_latent_amd.counters <pass dir> [<pass dir> ...] [--json OUT]
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import statistics
import sys

XCDS, SIMDS = 8, 1024
COPY_BYTES = 1 << 30


def _kernel(name: str) -> str:
    if "copyBuffer" in name or "CopyBuffer" in name:
        return "copy"
    return name.split("(")[0].replace("void ", "").strip()


def collect(dirs):
    """{kernel: {counter: [values]}} and {kernel: [durations ns]} over the pass directories."""
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(list)
    for d in dirs:
        path = os.path.join(d, "k_counter_collection.csv")
        seen = set()
        for r in csv.DictReader(open(path)):
            k = _kernel(r["Kernel_Name"])
            per[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
            key = (r.get("Dispatch_Id"), k)
            if "Start_Timestamp" in r and key not in seen and d == dirs[0]:
                seen.add(key)
                dur[k].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return per, dur


def summarise(dirs):
    per, dur = collect(dirs)
    copy = per.get("copy", {})
    ff = COPY_BYTES / (max(copy["FETCH_SIZE"]) * 1024) if copy.get("FETCH_SIZE") else None
    wf = COPY_BYTES / (max(copy["WRITE_SIZE"]) * 1024) if copy.get("WRITE_SIZE") else None
    out = {"fetch_factor": ff, "write_factor": wf, "kernels": {}}
    for k, c in per.items():
        if not k.startswith("mla::"):
            continue
        med = {n: statistics.median(v) for n, v in c.items()}
        rec = {"dispatches": max(len(v) for v in c.values())}
        if dur.get(k):
            rec["us"] = statistics.median(dur[k]) / 1e3
        if "FETCH_SIZE" in med and ff:
            rec["fetch_MB"] = med["FETCH_SIZE"] * 1024 * ff / 1e6
        if "WRITE_SIZE" in med and wf:
            rec["write_MB"] = med["WRITE_SIZE"] * 1024 * wf / 1e6
        g = med.get("GRBM_GUI_ACTIVE")
        if g and "SQ_VALU_MFMA_BUSY_CYCLES" in med:
            rec["mfma_busy_pct"] = 100.0 * med["SQ_VALU_MFMA_BUSY_CYCLES"] / (g / XCDS * SIMDS)
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in med:
            rec["mfma_bf16_gflop"] = med["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / 1e9
        out["kernels"][k] = rec
    return out


def markdown(summary) -> str:
    cols = [("us", "duration us (profiled)"), ("fetch_MB", "FETCH MB"), ("write_MB", "WRITE MB"),
            ("mfma_busy_pct", "MFMA busy %"), ("mfma_bf16_gflop", "bf16 MFMA GFLOP")]
    lines = ["| kernel | " + " | ".join(c[1] for c in cols) + " |", "|---" * (len(cols) + 1) + "|"]
    for k, r in sorted(summary["kernels"].items()):
        vals = [("%.2f" % r[c]) if c in r else "" for c, _ in cols]
        lines.append(f"| `{k}` | " + " | ".join(vals) + " |")
    f, w = summary["fetch_factor"], summary["write_factor"]
    lines.append("")
    lines.append(f"Calibration (1 GiB copy): FETCH factor {f:.4f}, WRITE factor {w:.4f}." if f and w else
                 "Calibration: not in these passes.")
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("dirs", nargs="+")
    ap.add_argument("--json")
    a = ap.parse_args(argv)
    s = summarise(a.dirs)
    print(markdown(s))
    if a.json:
        json.dump(s, open(a.json, "w"), indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
