"""Compile the HIP sources into libspecverify.so (gfx950), in-tree.

    python -m speculative_decoding_decode_amd.build [-v]
    python -m speculative_decoding_decode_amd.build --gemv-max-rows N --out PATH

Each csrc/*.hip file is compiled to an object under _build/ in parallel, then linked into a
shared library next to this file.  Packed-fp32 instructions are disabled for all device code.
`--gemv-max-rows N` builds a variant whose lm-head serves calls of up to N rows with the GEMV
(0: always the MFMA contraction; 8: the GEMV up to 8 rows) into PATH, for timing one kernel
against the other (bench.py --lm-head-rows with SPEC_VERIFY_LIB=PATH); the in-tree library
keeps the measured default.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB_NAME = "libspecverify.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument", "-I" + INCLUDE, "-I" + CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 target feature and says so; that is harmless
    lines = [l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l]
    return p.returncode, "\n".join(lines)


def build(verbose: bool = False, jobs: int | None = None, gemv_max_rows: int | None = None,
          out: str | None = None) -> str:
    cc = hipcc()
    tag = "" if gemv_max_rows is None else f"_gemv{gemv_max_rows}"
    bdir = BUILD + tag
    os.makedirs(bdir, exist_ok=True)
    defs = [] if gemv_max_rows is None else [f"-DSPEC_GEMV_MAX_ROWS={int(gemv_max_rows)}"]
    objs, cmds = [], []
    for src in sources():
        obj = os.path.join(bdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmds.append([cc, *COMMON, *defs, "-c", src, "-o", obj])
    jobs = jobs or min(len(cmds), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, msg) in zip(cmds, results):
        if verbose or rc != 0:
            print(" ".join(cmd))
            if msg:
                print(msg)
        if rc != 0:
            raise RuntimeError(f"compilation failed: {cmd[-3]}")
    target = out or LIB_PATH
    tmp = target + ".tmp"
    rc, log = _run([cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp])
    if rc != 0:
        print(log)
        raise RuntimeError("link failed")
    os.replace(tmp, target)
    return target


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("-v", action="store_true")
    ap.add_argument("--gemv-max-rows", type=int, default=None)
    ap.add_argument("--out", default=None)
    a = ap.parse_args()
    if (a.gemv_max_rows is None) != (a.out is None):
        ap.error("--gemv-max-rows and --out go together (a variant never replaces the library)")
    print(build(verbose=a.v, gemv_max_rows=a.gemv_max_rows, out=a.out))
