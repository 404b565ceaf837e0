"""Summaries of rocprofv3 output for the library's kernels.

* kernel statistics from a ``rocprofv3 --kernel-trace --stats
  --output-format csv`` run (``*_kernel_stats.csv``);
* HBM traffic per dispatch from two ``rocprofv3 --pmc`` runs, one with
  FETCH_SIZE and one with WRITE_SIZE (KiB per dispatch). Each counter is
  scaled by what it reads for a plain device-to-device copy of known size in
  the same run (the ``__amd_rocclr_copyBuffer`` dispatch of a 1 GiB copy),
  so the figures are bytes moved, not raw counter units.

The summary is a markdown file holding the commands, the tables and one
JSON block; ``read_traffic`` returns the traffic of a kernel from that block
when the block's hash of the sources it names (the csrc files the profiled
kernels are built from) still matches them, else None.

Usage: python -m sample_grad_norms_amd.profiling --trace DIR --fetch DIR
--write DIR --out FILE --cmd "..." [--cmd "..."]
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
from typing import Dict, List, Optional

HERE = os.path.dirname(os.path.abspath(__file__))
COPY_KERNEL = "__amd_rocclr_copyBuffer"
CALIB_BYTES = 1 << 30


def source_files() -> List[str]:
    """Names of the library's HIP sources and headers (csrc/)."""
    return sorted(os.path.basename(p) for p in glob.glob(os.path.join(HERE, "csrc", "*"))
                  if p.endswith((".hip", ".h", ".cpp")))


def source_hash(files: Optional[List[str]] = None) -> str:
    """sha256 over the named csrc files (default: all of them). A file that
    no longer exists hashes as missing, so the summary reads as stale."""
    h = hashlib.sha256()
    for name in sorted(files if files is not None else source_files()):
        h.update(name.encode())
        path = os.path.join(HERE, "csrc", name)
        h.update(open(path, "rb").read() if os.path.exists(path) else b"<missing>")
    return h.hexdigest()


def short_name(name: str) -> str:
    if COPY_KERNEL in name:
        return "copyBuffer"
    m = re.search(r"dpn::(k_\w+)(<[^>]*>)?", name)
    if m:
        return m.group(1) + (m.group(2) or "")
    return name.split("(")[0][:60]


def kernel_stats(trace_dir: str) -> List[Dict]:
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *kernel_stats.csv under {trace_dir}")
    rows = []
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            rows.append({"name": short_name(r["Name"]), "calls": int(r["Calls"]),
                         "avg_us": float(r["AverageNs"]) / 1e3, "total_ms": float(r["TotalDurationNs"]) / 1e6,
                         "pct": float(r["Percentage"])})
    return rows


def counter_values(pmc_dir: str, counter: str) -> Dict[str, List[float]]:
    files = glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *counter_collection.csv under {pmc_dir}")
    out: Dict[str, List[float]] = {}
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            out.setdefault(short_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return out


def scaled_bytes(vals: Dict[str, List[float]]) -> Dict[str, float]:
    """Mean bytes per dispatch for each kernel, scaled by the 1 GiB copy."""
    calib = max(vals.get("copyBuffer", [0.0]))
    if calib <= 0:
        raise ValueError("no calibration copy dispatch in the counter run")
    factor = CALIB_BYTES / (calib * 1024.0)
    return {k: sum(v) / len(v) * 1024.0 * factor for k, v in vals.items()}, factor


def summarize(trace_dir: str, fetch_dir: str, write_dir: str, out: str, cmds: List[str], title: str,
              sources: Optional[List[str]] = None) -> Dict:
    stats = kernel_stats(trace_dir)
    fetch, ffac = scaled_bytes(counter_values(fetch_dir, "FETCH_SIZE"))
    write, wfac = scaled_bytes(counter_values(write_dir, "WRITE_SIZE"))
    traffic = {k: fetch.get(k, 0.0) + write.get(k, 0.0) for k in set(fetch) | set(write) if k.startswith("k_")}
    files = sorted(sources) if sources else source_files()
    block = {"source_files": files, "source_sha256": source_hash(files), "fetch_scale": ffac, "write_scale": wfac,
             "traffic_bytes_per_dispatch": traffic,
             "fetch_bytes_per_dispatch": {k: v for k, v in fetch.items() if k.startswith("k_")},
             "write_bytes_per_dispatch": {k: v for k, v in write.items() if k.startswith("k_")},
             "avg_us": {r["name"]: r["avg_us"] for r in stats}}
    lines = [f"# {title}", "", "Commands (run from the repository root on the GPU box):", ""]
    lines += ["```", *cmds, "```", "", "## Kernel statistics (rocprofv3 --kernel-trace --stats)", "",
              "| kernel | calls | avg us | total ms | % |", "|---|---|---|---|---|"]
    for r in stats[:12]:
        lines.append(f"| {r['name']} | {r['calls']} | {r['avg_us']:.1f} | {r['total_ms']:.2f} | {r['pct']:.1f} |")
    lines += ["", f"## HBM traffic per dispatch (FETCH_SIZE x {ffac:.3f}, WRITE_SIZE x {wfac:.3f}; "
              "scales from a 1 GiB device-to-device copy)", "", "| kernel | read GB | written GB |", "|---|---|---|"]
    for k in sorted(traffic):
        lines.append(f"| {k} | {fetch.get(k, 0.0) / 1e9:.4f} | {write.get(k, 0.0) / 1e9:.4f} |")
    lines += ["", "```json", json.dumps(block, indent=1, sort_keys=True), "```", ""]
    with open(out, "w") as f:
        f.write("\n".join(lines))
    return block


def read_block(path: str) -> Optional[Dict]:
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    return json.loads(m.group(1)) if m else None


def read_traffic(path: str, kernel_prefix: str) -> Optional[float]:
    """Bytes per dispatch of the first kernel whose name starts with
    ``kernel_prefix``, or None when the summary is missing or the kernel
    sources changed since it was taken."""
    block = read_block(path)
    if not block or block.get("source_sha256") != source_hash(block.get("source_files")):
        return None
    for k, v in block["traffic_bytes_per_dispatch"].items():
        if k.startswith(kernel_prefix):
            return v
    return None


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--title", default="rocprofv3 summary")
    ap.add_argument("--cmd", action="append", default=[])
    ap.add_argument("--sources", nargs="*", default=None,
                    help="csrc files the profiled kernels are built from (default: all); the summary "
                         "reads as stale once any of them changes")
    a = ap.parse_args()
    block = summarize(a.trace, a.fetch, a.write, a.out, a.cmd, a.title, a.sources)
    print(json.dumps(block["traffic_bytes_per_dispatch"]))


if __name__ == "__main__":
    main()
