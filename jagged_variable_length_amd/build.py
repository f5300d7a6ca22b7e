"""Build libjattn.so (HIP kernels for gfx950 + host planner/C ABI) in-tree.

    python -m jagged_variable_length_amd.build [--incremental] [-j N]

Every kernel translation unit is compiled with hipcc for gfx950 only; the
result is jagged_variable_length_amd/libjattn.so.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libjattn.so")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include"), "-Wno-unused-result"]

# fp32 inputs (with fp32 outputs and gradients) run the first-generation
# forward and backward kernels (fwd_inst.hip, bwd_inst.hip); bf16 inputs run
# the LDS-DMA kernels (fwd2/dkdv2/dq2) and take only the Di pass from
# bwd_inst.hip.
F32_DIMS = (64, 32)
BF16_DIMS = (128, 64, 32)


def units():
    """(source, object name, extra defines) of every translation unit."""
    u = [("api.cpp", "api", []), ("planner.cpp", "planner", []), ("block_inst.hip", "block", []),
         ("l2norm.hip", "l2norm", []), ("fixed_scratch.hip", "fixed_scratch", [])]
    for d in BF16_DIMS:
        u.append(("fwd2_inst.hip", f"fwd2_{d}", [f"-DJ_D={d}"]))
        for tg in ("bf16", "f32"):
            u.append(("bwd2_inst.hip", f"dkdv2_{d}_{tg}", [f"-DJ_D={d}", f"-DJ_TG={tg}"]))
            u.append(("dq2_inst.hip", f"dq2_{d}_{tg}", [f"-DJ_D={d}", f"-DJ_TG={tg}"]))
        u.append(("bwd_inst.hip", f"di_{d}_bf16", [f"-DJ_D={d}", "-DJ_TI=bf16", "-DJ_TG=bf16", "-DJ_DI",
                                                   "-DJ_DI_ONLY"]))
    for tg in ("bf16", "f32"):
        u.append(("bwd_pair_inst.hip", f"dkdv_pair_128_{tg}", ["-DJ_D=128", f"-DJ_TG={tg}"]))
    for d in (128, 64):
        u.append(("mx_inst.hip", f"mx_{d}", [f"-DJ_D={d}"]))
    for d in F32_DIMS:
        u.append(("fwd_inst.hip", f"fwd_{d}_f32_f32", [f"-DJ_D={d}", "-DJ_TI=f32", "-DJ_TO=f32"]))
        u.append(("bwd_inst.hip", f"bwd_{d}_f32_f32", [f"-DJ_D={d}", "-DJ_TI=f32", "-DJ_TG=f32", "-DJ_DI"]))
    return u


def _deps():
    return [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + [os.path.join(ROOT, "include", "jattn.h")]


def _scratch_kernels(text):
    """Kernels whose resource-usage remark reports scratch (private) memory.
    Scratch accesses are vector memory operations: their waits would also
    wait on the kernels' in-flight LDS prefetches, so none may use it."""
    bad, name = [], None
    for line in text.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0:
            bad.append(f"{name} ({m.group(1)} bytes/lane)")
    return bad


def _dep_files(depfile):
    """Files a translation unit depends on, from the compiler's make-style
    dependency output (None if it is missing)."""
    try:
        text = open(depfile).read().replace("\\\n", " ")
    except OSError:
        return None
    deps = []
    for line in text.splitlines():
        if ":" in line:
            deps += line.split(":", 1)[1].split()
    return deps


def _up_to_date(out, depfile):
    if not os.path.exists(out):
        return False
    deps = _dep_files(depfile)
    if not deps:
        deps = _deps()
    try:
        return os.path.getmtime(out) >= max(os.path.getmtime(p) for p in deps + [__file__])
    except OSError:
        return False


def _compile(src, name, defs, incremental):
    out = os.path.join(OBJ, name + ".o")
    depfile = os.path.join(OBJ, name + ".d")
    if incremental and _up_to_date(out, depfile):
        return out, None
    hip = src.endswith(".hip")
    xflags = ["-x", "hip", "-Rpass-analysis=kernel-resource-usage"] if hip else []
    cmd = [HIPCC] + FLAGS + defs + xflags + ["-MD", "-MF", depfile, "-c", os.path.join(CSRC, src), "-o", out]
    p = subprocess.run(cmd, capture_output=True, text=True)
    text = p.stdout + p.stderr
    errs = "\n".join(l for l in text.splitlines()
                     if "packed-fp32-ops" not in l and "kernel-resource-usage" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{errs}")
    bad = _scratch_kernels(text)
    if bad:
        os.remove(out)
        raise RuntimeError(f"{src} {' '.join(defs)}: kernels use scratch memory: {', '.join(bad)}")
    return out, errs.strip() or None


def build(incremental: bool = False, jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 4)
    objs = []
    with cf.ThreadPoolExecutor(jobs) as ex:
        futs = [ex.submit(_compile, s, n, d, incremental) for s, n, d in units()]
        for f in futs:
            o, msg = f.result()
            objs.append(o)
            if msg and verbose:
                print(msg, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{p.stdout}{p.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--incremental", action="store_true")
    ap.add_argument("-j", type=int, default=None)
    ap.add_argument("-v", action="store_true")
    a = ap.parse_args()
    print(build(a.incremental, a.j, a.v))


if __name__ == "__main__":
    main()
