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
--write DIR --out FILE --cmd "..." [--cmd "..."], or, for utilisation
counters (MFMA, LDS, waits, L2 hits) of one or more --pmc runs,
python -m sample_grad_norms_amd.profiling --pmc DIR [--pmc DIR] --out FILE
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


_COMMENT = re.compile(r"/\*.*?\*/|//[^\n]*", re.S)


def code_text(src: str) -> str:
    """C/HIP source without its comments and with whitespace runs collapsed:
    what a summary's counters depend on (a comment edit leaves it valid)."""
    return " ".join(_COMMENT.sub(" ", src).split())


def source_hash(files: Optional[List[str]] = None) -> str:
    """sha256 over the code (comments and layout dropped) of the named csrc
    files (default: all of them). A file that no longer exists hashes as
    missing, so the summary reads as stale."""
    h = hashlib.sha256()
    for name in sorted(files if files is not None else source_files()):
        h.update(name.encode())
        path = os.path.join(HERE, "csrc", name)
        h.update(code_text(open(path, encoding="utf-8").read()).encode() if os.path.exists(path) else b"<missing>")
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
    shown = stats[:12] + [r for r in stats[12:] if r["name"].startswith("k_")]   # the library's kernels always
    for r in shown:
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


# MI355X: 8 XCDs of 32 CUs, 4 SIMDs per CU. GRBM_GUI_ACTIVE is reported summed
# over the XCDs, so one XCD's active cycles are the sum over N_XCD.
N_XCD, N_CU, N_SIMD = 8, 256, 1024

# (label, numerator, denominator, scale) of the derived utilisation figures
DERIVED = (
    ("MFMA pipe busy (per SIMD)", "SQ_VALU_MFMA_BUSY_CYCLES", "simd_cycles", 1.0),
    ("LDS busy (indexed ops, per CU)", "SQ_LDS_IDX_ACTIVE", "cu_cycles", 1.0),
    ("LDS cycles stalled by bank conflicts / LDS busy", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", 1.0),
    ("wave time waiting on a dependency (s_waitcnt)", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES", 1.0),
    ("L2 hit rate", "TCC_HIT_sum", "tcc_requests", 1.0),
)


def counter_means(pmc_dirs: List[str]) -> Dict[str, Dict[str, float]]:
    """Mean per dispatch of every counter of every dpn:: kernel, over the
    counter_collection.csv files of several --pmc runs."""
    out: Dict[str, Dict[str, List[float]]] = {}
    for d in pmc_dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise FileNotFoundError(f"no *counter_collection.csv under {d}")
        with open(files[0]) as f:
            for r in csv.DictReader(f):
                if "dpn::" not in r["Kernel_Name"]:
                    continue
                out.setdefault(short_name(r["Kernel_Name"]), {}).setdefault(r["Counter_Name"], []).append(
                    float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in out.items()}


def derived(c: Dict[str, float]) -> Dict[str, Optional[float]]:
    """Utilisation ratios of one kernel's mean counters (None where a counter is missing)."""
    v = dict(c)
    if "GRBM_GUI_ACTIVE" in v:
        cycles = v["GRBM_GUI_ACTIVE"] / N_XCD
        v["simd_cycles"] = cycles * N_SIMD
        v["cu_cycles"] = cycles * N_CU
    if "TCC_HIT_sum" in v and "TCC_MISS_sum" in v:
        v["tcc_requests"] = v["TCC_HIT_sum"] + v["TCC_MISS_sum"]
    res: Dict[str, Optional[float]] = {}
    for label, num, den, scale in DERIVED:
        res[label] = scale * v[num] / v[den] if num in v and v.get(den) else None
    return res


def counters_summary(pmc_dirs: List[str], out: str, cmds: List[str], title: str) -> Dict:
    """Markdown summary of utilisation counters per kernel (means per dispatch
    and the ratios of DERIVED)."""
    means = counter_means(pmc_dirs)
    names = sorted({c for cs in means.values() for c in cs})
    lines = [f"# {title}", "", "Commands (run from the repository root on the GPU box):", "", "```", *cmds, "```", "",
             "## Utilisation", "", "| kernel | " + " | ".join(l for (l, _, _, _) in DERIVED) + " |",
             "|---" * (len(DERIVED) + 1) + "|"]
    for k in sorted(means):
        dv = derived(means[k])
        lines.append(f"| {k} | " + " | ".join("—" if dv[l] is None else f"{100 * dv[l]:.1f} %"
                                               for (l, _, _, _) in DERIVED) + " |")
    lines += ["", f"Cycles: GRBM_GUI_ACTIVE / {N_XCD} (it is summed over the XCDs); {N_SIMD} SIMDs, {N_CU} CUs.", "",
              "## Mean counter values per dispatch", "", "| kernel | " + " | ".join(names) + " |",
              "|---" * (len(names) + 1) + "|"]
    for k in sorted(means):
        lines.append(f"| {k} | " + " | ".join(f"{means[k][c]:.4g}" if c in means[k] else "—" for c in names) + " |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    return means


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--pmc", action="append", default=[],
                    help="utilisation mode: a --pmc run directory (repeat for several runs)")
    ap.add_argument("--trace")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--out", required=True)
    ap.add_argument("--title", default="rocprofv3 summary")
    ap.add_argument("--cmd", action="append", default=[])
    ap.add_argument("--sources", nargs="*", default=None,
                    help="csrc files the profiled kernels are built from (default: all); the summary "
                         "reads as stale once any of them changes")
    a = ap.parse_args()
    if a.pmc:
        counters_summary(a.pmc, a.out, a.cmd, a.title)
        return
    if not (a.trace and a.fetch and a.write):
        ap.error("--trace, --fetch and --write are required (or --pmc for the utilisation summary)")
    block = summarize(a.trace, a.fetch, a.write, a.out, a.cmd, a.title, a.sources)
    print(json.dumps(block["traffic_bytes_per_dispatch"]))


if __name__ == "__main__":
    main()
