"""Build libwsic.so (HIP, gfx950) in-tree: ``python -m rate_allocated_weight_amd.build``.

Every ``csrc/*.hip`` file is compiled with hipcc to an object for gfx950 and the objects are
linked into ``rate_allocated_weight_amd/libwsic.so``. Objects go to ``_build/`` at the repo
root (not committed).

The gfx950 assembly of every source is kept (``-save-temps``) and checked for one known
miscompilation before the library is linked: a divergent branch lowered as
``s_and_saveexec_b64 s[x], ...; s_cbranch_execz L`` whose join block ``L`` carries vector
register writes (copies, spills, rematerialized constants) ahead of the exec-mask restore
``s_or_b64 exec, exec, s[x]``. Those writes run with the branch's partial (often empty) mask,
so lanes that skipped the branch keep stale values. The compiler produced this in the SIC
super-block kernel (the check's shared-memory addresses and spill copies), where it showed
up as nondeterministic re-derivations; the build now refuses such code.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libwsic.so")

ARCH = "gfx950"
CXXFLAGS = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    f"--offload-arch={ARCH}",
    "-munsafe-fp-atomics",
    "-I", INCLUDE,
    "-I", CSRC,
    "-Wall",
    "-Wno-unused-function",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libwsic)")


def exec_join_writes(asm: str):
    """(function, line, label, [instructions]) for every join block that writes vector registers
    before restoring the exec mask saved by the simple if-lowering that branched to it."""
    lines = asm.splitlines()
    labels = {}
    func = []
    cur = None
    for i, l in enumerate(lines):
        m = re.match(r"^(\.LBB\d+_\d+):", l)
        if m:
            labels[m.group(1)] = i
        m = re.match(r"^([A-Za-z_.][A-Za-z0-9_.$]*):", l)
        if m and not l.startswith(".L"):
            cur = m.group(1)
        func.append(cur)
    found = []
    for i, l in enumerate(lines):
        m = re.match(r"^\s*s_cbranch_execz\s+(\.LBB\d+_\d+)", l)
        if not m:
            continue
        k = i - 1
        while k > 0 and (not lines[k].strip() or lines[k].strip().startswith(";")):
            k -= 1
        sm = re.match(r"^\s*s_and_saveexec_b64\s+(s\[\d+:\d+\]),", lines[k])
        if not sm or m.group(1) not in labels:
            continue  # not the simple if-lowering (if/else and loops restore differently)
        restore = re.compile(r"s_or_b64\s+exec,\s*exec,\s*" + re.escape(sm.group(1)) + r"\s*$")
        writes = []
        for t in lines[labels[m.group(1)] + 1:labels[m.group(1)] + 200]:
            t = t.strip()
            if not t or t.startswith(";"):
                continue
            if restore.match(t):
                if writes:
                    found.append((func[i], i + 1, m.group(1), writes))
                break
            if t.startswith(".LBB") or re.match(r"s_(branch|cbranch|endpgm|setpc|\w*saveexec)", t):
                break
            if re.match(r"(v_|ds_read|global_load|buffer_load|flat_load)", t) and not re.match(
                    r"v_(writelane|readlane|readfirstlane)", t):
                writes.append(t)
    return found


def _compile(src: str, hipcc: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc, *CXXFLAGS, "-save-temps=obj", "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    stem = os.path.splitext(os.path.basename(src))[0]
    asm_path = os.path.join(BUILD, f"{stem}-hip-amdgcn-amd-amdhsa-{ARCH}.s")
    if not os.path.exists(asm_path):
        raise RuntimeError(f"device assembly of {src} not found at {asm_path}")
    bad = exec_join_writes(open(asm_path).read())
    if bad:
        msg = "\n".join(f"  {f} (asm line {ln}, join {lab}): {w[:4]}" for f, ln, lab, w in bad)
        raise RuntimeError(f"{src}: vector writes ahead of an exec-mask restore (lanes that skip "
                           f"the branch keep stale registers); restructure the branch:\n{msg}")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every HIP source and link libwsic.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError(f"no HIP sources under {CSRC}")
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build()
