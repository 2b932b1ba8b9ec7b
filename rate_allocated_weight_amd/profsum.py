"""Summaries of rocprofv3 runs of `bench.py`: per-kernel durations and HBM bytes per launch.

Reads the CSV files rocprofv3 writes (`--output-format csv`) for

* a kernel trace (`--kernel-trace --stats`): the `*_kernel_stats.csv` table,
* a `--pmc FETCH_SIZE` run and a `--pmc WRITE_SIZE` run of the same command
  (`*_counter_collection.csv`, KiB per dispatch),
* the same two counters for a plain device copy of known size (`bench.py
  --copy-calibration-mib M`), which turns the counter readings into bytes,
* optionally a `--pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE` run: the matrix-core busy
  fraction per kernel, SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs),

and writes, for one workload:

* `traffic_<workload>.txt`: a JSON record per kernel family (read and written bytes per launch,
  the kernel's source file and its SHA-256, so that a later edit of the kernel voids the record);
  `bench.py` reads it for the roofline's `traffic`,
* `<name>_kernel_trace.md` and `<name>_counters.md`: the tables, with the commands that made them.

    python -m rate_allocated_weight_amd.profsum --workload attn_4096 --name attn_4096 \
        --trace DIR --fetch DIR --write DIR --calib-fetch DIR --calib-write DIR --calib-mib 1024 \
        --cmd "..." --out profiles

Host-side text processing only; it runs no kernel.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = "rate_allocated_weight_amd/csrc"

# kernel family (the library's launch name) -> (kernel symbol pattern, source file)
FAMILY_KERNELS = {
    "sic_leaf": (r"^k_sic_(super|leaf)\b", "k_sic.hip"),
    "gemm_trail_i8": (r"^k_gemm_i8\b", "k_limb.hip"),
    "gemm_y": (r"^k_gemm_y\b", "k_gemm.hip"),
    "chol_step": (r"^k_chol_step\b", "k_chol.hip"),
    "potrf_panel": (r"^k_potrf_panel\b", "k_chol.hip"),
    "syrk_bf16": (r"^k_syrk_bf16", "k_cov.hip"),
    "hist": (r"^k_hist$", "k_hist.hip"),
    "dist_resid": (r"^k_dist_resid\b", "k_dist.hip"),
    "logits_bf16": (r"^k_logits_bf16\b", "k_softmax.hip"),
    "curvature": (r"^k_curvature\b", "k_softmax.hip"),
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _short(name: str) -> str:
    """Kernel symbol without namespaces, argument list or trailing launch suffix."""
    n = name.strip()
    n = re.sub(r"\.kd$", "", n).replace("(anonymous namespace)::", "")
    depth = 0
    cut = len(n)
    for i, ch in enumerate(n):  # drop the argument list: the first '(' outside template brackets
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    n = n[:cut]
    n = re.sub(r"^(void\s+)", "", n)
    # strip leading namespaces outside template arguments
    depth = 0
    last = 0
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == ":" and depth == 0 and i + 1 < len(n) and n[i + 1] == ":":
            last = i + 2
    return n[last:].strip()


def _find(d: str, suffix: str) -> list[str]:
    return sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))


def read_counters(d: str, counter: str) -> dict[str, list[float]]:
    """Per kernel (short name): the counter's value per dispatch, in dispatch order."""
    per_dispatch: dict[tuple, float] = defaultdict(float)
    names: dict[tuple, str] = {}
    files = _find(d, "counter_collection.csv")
    if not files:
        raise FileNotFoundError(f"no *counter_collection.csv under {d}")
    for f in files:
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter:
                    continue
                key = (f, int(row["Dispatch_Id"]))
                per_dispatch[key] += float(row["Counter_Value"])
                names[key] = _short(row["Kernel_Name"])
    out: dict[str, list[float]] = defaultdict(list)
    for key in sorted(per_dispatch):
        out[names[key]].append(per_dispatch[key])
    return dict(out)


def read_stats(d: str) -> list[dict]:
    files = _find(d, "kernel_stats.csv")
    if not files:
        raise FileNotFoundError(f"no *kernel_stats.csv under {d}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                rows.append(dict(name=_short(row["Name"]), calls=int(row["Calls"]),
                                 total_ns=float(row["TotalDurationNs"]),
                                 avg_ns=float(row["AverageNs"]), pct=float(row["Percentage"])))
    rows.sort(key=lambda r: -r["total_ns"])
    return rows


def copy_scale(d: str, counter: str, nbytes: float) -> float:
    """Bytes per counted KiB: the known copy size over the copy kernel's largest reading."""
    vals = read_counters(d, counter).get(COPY_KERNEL)
    if not vals:
        raise ValueError(f"{COPY_KERNEL} not found in the {counter} calibration run")
    return nbytes / (1024.0 * max(vals))


def family_of(kernel: str):
    for fam, (pat, _src) in FAMILY_KERNELS.items():
        if re.search(pat, kernel):
            return fam
    return None


def traffic_record(workload: str, fetch: dict, write: dict, s_read: float, s_write: float,
                   commands: list[str]) -> dict:
    fams: dict[str, dict] = {}
    for fam, (_pat, src) in FAMILY_KERNELS.items():
        ks = sorted(k for k in fetch if family_of(k) == fam)
        if not ks:
            continue
        rd = [v for k in ks for v in fetch[k]]
        wr = [v for k in ks for v in write.get(k, [])]
        if not wr or len(wr) != len(rd):
            continue
        path = f"{CSRC}/{src}"
        sha = hashlib.sha256(open(os.path.join(ROOT, path), "rb").read()).hexdigest()
        fams[fam] = dict(kernel=" + ".join(ks), source=path, source_sha256=sha,
                         read_bytes_per_launch=1024.0 * s_read * sum(rd) / len(rd),
                         write_bytes_per_launch=1024.0 * s_write * sum(wr) / len(wr),
                         launches_profiled=len(rd))
    return dict(workload=workload, commands=commands, copy_scale_read=round(s_read, 5),
                copy_scale_write=round(s_write, 5), families=fams)


def trace_md(title: str, cmd: str, stats: list[dict], top: int = 24) -> str:
    lines = [f"# Kernel trace: {title}", "", "Command (from the repository root):", "", "```", cmd,
             "```", "", "Averages per dispatch over every step the command ran.", "",
             "| kernel | calls | avg us | total ms | % |", "|---|---:|---:|---:|---:|"]
    for r in stats[:top]:
        lines.append(f"| `{r['name']}` | {r['calls']} | {r['avg_ns'] / 1e3:.2f} | "
                     f"{r['total_ns'] / 1e6:.3f} | {r['pct']:.1f} |")
    return "\n".join(lines) + "\n"


def mfma_busy(d: str) -> dict[str, float]:
    """Per kernel: matrix-core busy fraction, averaged over its dispatches."""
    busy = read_counters(d, "SQ_VALU_MFMA_BUSY_CYCLES")
    gui = read_counters(d, "GRBM_GUI_ACTIVE")
    out = {}
    for k, b in busy.items():
        g = gui.get(k, [])
        if len(g) == len(b) and sum(g) > 0:
            out[k] = sum(b) / (sum(g) / 8.0 * 1024.0)
    return out


def counters_md(title: str, cmds: list[str], fetch: dict, write: dict, s_read: float,
                s_write: float, calib_mib: int, top: int = 20, busy: dict | None = None) -> str:
    rows = []
    for k, rd in fetch.items():
        wr = write.get(k, [])
        r = 1024.0 * s_read * sum(rd) / len(rd) / 2**20
        w = 1024.0 * s_write * sum(wr) / len(wr) / 2**20 if wr else float("nan")
        rows.append((r * len(rd), k, len(rd), r, w))
    rows.sort(key=lambda t: -t[0])
    lines = [f"# HBM traffic per kernel: {title}", "", "Commands (from the repository root):", "",
             "```", *cmds, "```", "",
             "FETCH_SIZE / WRITE_SIZE are KiB per dispatch; each is scaled by what the same counter "
             f"reads for a plain {calib_mib} MiB device copy (`{COPY_KERNEL}`).", "",
             f"copy calibration: scale read {s_read:.4f}, write {s_write:.4f} (bytes per counted byte)",
             "", "| kernel | launches | read MiB/launch | write MiB/launch |", "|---|---:|---:|---:|"]
    for _, k, n, r, w in rows[:top]:
        lines.append(f"| `{k}` | {n} | {r:.3f} | {w:.3f} |")
    if busy:
        lines += ["", "Matrix cores: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs).",
                  "", "| kernel | MFMA busy |", "|---|---:|"]
        for k, v in sorted(busy.items(), key=lambda t: -t[1]):
            if v >= 0.001:
                lines.append(f"| `{k}` | {v:.3f} |")
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--name", required=True, help="file stem of the markdown summaries")
    ap.add_argument("--title", default="")
    ap.add_argument("--trace", help="rocprofv3 --kernel-trace --stats output folder")
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--calib-fetch", required=True)
    ap.add_argument("--calib-write", required=True)
    ap.add_argument("--calib-mib", type=int, default=1024)
    ap.add_argument("--mfma", help="rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE folder")
    ap.add_argument("--cmd", action="append", default=[],
                    help="command lines that made the runs (trace first, if any)")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    a = ap.parse_args(argv)

    nbytes = a.calib_mib * float(1 << 20)
    s_read = copy_scale(a.calib_fetch, "FETCH_SIZE", nbytes)
    s_write = copy_scale(a.calib_write, "WRITE_SIZE", nbytes)
    fetch = read_counters(a.fetch, "FETCH_SIZE")
    write = read_counters(a.write, "WRITE_SIZE")
    title = a.title or a.workload
    os.makedirs(a.out, exist_ok=True)
    rec = traffic_record(a.workload, fetch, write, s_read, s_write, a.cmd)
    with open(os.path.join(a.out, f"traffic_{a.workload}.txt"), "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    pmc_cmds = [c for c in a.cmd if "--kernel-trace" not in c]
    with open(os.path.join(a.out, f"{a.name}_counters.md"), "w") as fh:
        fh.write(counters_md(title, pmc_cmds, fetch, write, s_read, s_write, a.calib_mib,
                             busy=mfma_busy(a.mfma) if a.mfma else None))
    if a.trace:
        tcmd = next((c for c in a.cmd if "--kernel-trace" in c), "")
        with open(os.path.join(a.out, f"{a.name}_kernel_trace.md"), "w") as fh:
            fh.write(trace_md(title, tcmd, read_stats(a.trace)))
    print(json.dumps({f: (round(v["read_bytes_per_launch"] / 2**20, 3),
                          round(v["write_bytes_per_launch"] / 2**20, 3))
                      for f, v in rec["families"].items()}))


if __name__ == "__main__":
    main()
