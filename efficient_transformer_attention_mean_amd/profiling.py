"""Text summaries of rocprofv3 output, for the ``profiles/`` directory.

Two summaries are produced from the CSV files rocprofv3 writes with
``--output-format csv``:

* ``stats``: the per-kernel table of a ``--kernel-trace --stats`` run (calls,
  mean / min / max duration, share of GPU time);
* ``traffic``: HBM bytes per dispatch from two ``--pmc`` runs (``FETCH_SIZE``
  then ``WRITE_SIZE``, both in KiB per dispatch).  Each counter is scaled by
  what it reads for a plain copy kernel of known size (``bench.py
  --copy-calibration`` launches one: a 256 MiB fp32 elementwise add), so the
  figures are bytes, whatever unit the counter's request size implies.

Both record the commands that produced their input and a digest of the
kernel sources, so a reader (and ``bench.py``) can tell whether a summary
still describes the current kernels.

Usage::

    python -m efficient_transformer_attention_mean_amd.profiling stats CSV --command CMD --out FILE
    python -m efficient_transformer_attention_mean_amd.profiling traffic --fetch DIR --write DIR \\
        --fetch-command CMD --write-command CMD --out FILE
    python -m efficient_transformer_attention_mean_amd.profiling counters --run DIR CMD [--run DIR CMD ...] \\
        --out FILE

A third summary, ``counters``, lists the mean of every counter per kernel
from any number of ``--pmc`` runs with figures derived from them (matrix-core
busy share, L2 hit rate, LDS bank conflicts).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
import statistics
import sys

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
# The copy kernel of known size launched by bench.py --copy-calibration (an
# fp32 elementwise add): reads and writes 256 MiB.  The fill that creates its
# input is also an elementwise kernel, hence the "add" in the pattern.
CALIB_BYTES = 256 * 2 ** 20
CALIB_RE = re.compile(r"elementwise.*add")


def sources_digest() -> str:
    """sha256 over the kernel sources (file names and contents, sorted)."""
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if path.endswith((".hip", ".hpp", ".h")):
            h.update(os.path.basename(path).encode())
            with open(path, "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def short_name(name: str) -> str:
    """Kernel name without the argument list and namespace."""
    base = name.replace("(anonymous namespace)::", "").split("(")[0]
    base = re.sub(r"^void ", "", base)
    return base.replace("nys::", "")


def family(name: str) -> str:
    """Kernel family used by the bench's per-kernel timers (k_apply -> apply)."""
    s = short_name(name)
    s = re.sub(r"<.*", "", s)
    return s[2:] if s.startswith("k_") else s


def _rows(pattern: str) -> list[dict]:
    rows: list[dict] = []
    for path in sorted(glob.glob(pattern, recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def stats_summary(csv_path: str, command: str, title: str) -> str:
    rows = _rows(csv_path)
    if not rows:
        raise SystemExit(f"no rows in {csv_path}")
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    out = [f"# {title}", "", "Command (run from the repository root; rocprofv3 writes CSV files):", "",
           f"    {command}", "", f"Kernel sources sha256: {sources_digest()}", "",
           "| kernel | calls | mean us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        out.append(f"| {short_name(r['Name'])} | {int(r['Calls'])} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{100 * float(r['TotalDurationNs']) / total:.1f}% |")
    return "\n".join(out) + "\n"


def _counter_means(directory: str, counter: str) -> dict[str, float]:
    per: dict[str, list[float]] = {}
    for r in _rows(os.path.join(directory, "**", "*counter_collection.csv")):
        if r["Counter_Name"] != counter:
            continue
        per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: statistics.fmean(v) for k, v in per.items()}


def traffic_summary(fetch_dir: str, write_dir: str, fetch_cmd: str, write_cmd: str, title: str) -> str:
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")
    calib_f = [v for k, v in fetch.items() if CALIB_RE.search(k)]
    calib_w = [v for k, v in write.items() if CALIB_RE.search(k)]
    if not calib_f or not calib_w:
        raise SystemExit("calibration copy kernel not found in the counter files")
    # KiB reported for CALIB_BYTES read (resp. written) -> bytes per reported KiB.
    f_scale = CALIB_BYTES / calib_f[0]
    w_scale = CALIB_BYTES / calib_w[0]
    out = [f"# {title}", "", "Commands (run from the repository root):", "", f"    {fetch_cmd}", f"    {write_cmd}", "",
           f"Kernel sources sha256: {sources_digest()}", "",
           f"Calibration: the {CALIB_BYTES // 2**20} MiB copy kernel reads FETCH_SIZE {calib_f[0]:.0f} KiB and "
           f"WRITE_SIZE {calib_w[0]:.0f} KiB per dispatch; scale factors {f_scale / 1024:.4f} (fetch) and "
           f"{w_scale / 1024:.4f} (write) true KiB per reported KiB.", "",
           "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes (scaled) | written bytes (scaled) | traffic bytes |",
           "|---|---|---|---|---|---|"]
    lines = []
    for k in sorted(set(fetch) | set(write), key=lambda k: -(fetch.get(k, 0) + write.get(k, 0))):
        if "elementwise" in k:  # the calibration copy and its input fill
            continue
        fb, wb = fetch.get(k, 0.0) * f_scale, write.get(k, 0.0) * w_scale
        out.append(f"| {short_name(k)} | {fetch.get(k, 0):.0f} | {write.get(k, 0):.0f} | {fb:.4g} | {wb:.4g} | "
                   f"{fb + wb:.4g} |")
        lines.append(f"traffic_bytes_per_launch {family(k)} {fb + wb:.6g}")
    return "\n".join(out + ["", "Machine-readable lines (kernel family, scaled bytes per dispatch):", ""] +
                     ["    " + s for s in lines]) + "\n"


# Derived figures of a counter summary: (label, numerator, denominator,
# factor).  SQ_BUSY_CU_CYCLES sums busy cycles over compute units and
# SQ_VALU_MFMA_BUSY_CYCLES busy cycles over the 4 SIMDs of each, so their ratio
# over 4 is the matrix cores' busy share while the kernel occupies the CUs.
DERIVED = [
    ("MFMA busy (% of SIMD cycles while CUs busy)", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", 25.0),
    ("L2 hit rate (%)", "TCC_HIT_sum", "TCC_HIT_sum+TCC_MISS_sum", 100.0),
    ("LDS bank-conflict cycles per LDS instruction", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS", 1.0),
    ("LDS bank-conflict cycles (% of CU busy cycles)", "SQ_LDS_BANK_CONFLICT", "SQ_BUSY_CU_CYCLES", 100.0),
    ("LDS wait (% of CU busy cycles)", "SQ_WAIT_INST_LDS", "SQ_BUSY_CU_CYCLES", 100.0),
]


def counters_summary(runs: list[tuple[str, str]], title: str, kernels: str | None = None) -> str:
    """Mean of every counter per kernel over its dispatches, from one or
    more ``--pmc`` runs (directory, command), plus the DERIVED figures."""
    per: dict[str, dict[str, list[float]]] = {}
    for directory, _ in runs:
        for r in _rows(os.path.join(directory, "**", "*counter_collection.csv")):
            k = short_name(r["Kernel_Name"])
            if kernels and not re.search(kernels, k):
                continue
            per.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not per:
        raise SystemExit("no counter rows")
    out = [f"# {title}", "", "Commands (run from the repository root; one rocprofv3 pass each):", ""]
    out += [f"    {cmd}" for _, cmd in runs]
    out += ["", f"Kernel sources sha256: {sources_digest()}", "",
            "Counters are means per dispatch, summed over the device's units as rocprofv3 reports them.", ""]
    for k in sorted(per):
        cs = {c: statistics.fmean(v) for c, v in per[k].items()}
        out += [f"## {k}", "", "| counter | mean per dispatch |", "|---|---|"]
        out += [f"| {c} | {v:.6g} |" for c, v in sorted(cs.items())]
        rows = []
        for label, num, den, fac in DERIVED:
            if num in cs and all(d in cs for d in den.split("+")):
                dv = sum(cs[d] for d in den.split("+"))
                if dv > 0:
                    rows.append(f"| {label} | {fac * cs[num] / dv:.4g} |")
        if rows:
            out += ["", "| derived | value |", "|---|---|"] + rows
        out.append("")
    return "\n".join(out)


def read_kernel_mean_us(path: str, kernel_family: str) -> float | None:
    """Mean traced duration (us) of a kernel family from a stats summary, or
    None when the file is missing or was made from other kernel sources."""
    try:
        with open(path) as f:
            text = f.read()
    except OSError:
        return None
    m = re.search(r"Kernel sources sha256: ([0-9a-f]+)", text)
    if not m or m.group(1) != sources_digest():
        return None
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 6 and cells[0] and family(cells[0]) == kernel_family:
            try:
                return float(cells[2])
            except ValueError:
                return None
    return None


def read_traffic(path: str, kernel_family: str) -> float | None:
    """Scaled bytes per dispatch for a kernel family from a traffic summary,
    or None when the file is missing or was made from other kernel sources."""
    try:
        with open(path) as f:
            text = f.read()
    except OSError:
        return None
    m = re.search(r"Kernel sources sha256: ([0-9a-f]+)", text)
    if not m or m.group(1) != sources_digest():
        return None
    m = re.search(rf"traffic_bytes_per_launch {re.escape(kernel_family)} ([0-9.eE+-]+)", text)
    return float(m.group(1)) if m else None


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv", help="rocprofv3 *_kernel_stats.csv")
    s.add_argument("--command", required=True)
    s.add_argument("--title", default="Kernel durations")
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True, help="directory of the FETCH_SIZE run")
    t.add_argument("--write", required=True, help="directory of the WRITE_SIZE run")
    t.add_argument("--fetch-command", required=True)
    t.add_argument("--write-command", required=True)
    t.add_argument("--title", default="HBM traffic per dispatch")
    t.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--run", nargs=2, action="append", metavar=("DIR", "COMMAND"), required=True,
                   help="directory of one --pmc run and the command that made it (repeatable)")
    c.add_argument("--kernels", default=None, help="regular expression: keep only matching kernel names")
    c.add_argument("--title", default="Hardware counters per dispatch")
    c.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        text = stats_summary(a.csv, a.command, a.title)
    elif a.cmd == "counters":
        text = counters_summary([tuple(r) for r in a.run], a.title, a.kernels)
    else:
        text = traffic_summary(a.fetch, a.write, a.fetch_command, a.write_command, a.title)
    with open(a.out, "w") as f:
        f.write(text)
    print(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
