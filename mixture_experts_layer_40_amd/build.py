"""Build libmoe.so (all HIP sources, gfx950) in-tree next to this file, and
libmoe_peaks.so (the achievable-peak probes of include/moe_peaks.h).

    python -m mixture_experts_layer_40_amd.build [--verbose]

Each library is plain hipcc output: one shared object exporting a C ABI.
Packed-fp32 instruction selection is disabled for device code
(-packed-fp32-ops); hipcc's host pass warns that it does not know the
feature, which is harmless.
"""

from __future__ import annotations

import argparse
import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libmoe.so")
PEAKS_DIR = os.path.join(PKG_DIR, "probes")
PEAKS_LIB_PATH = os.path.join(PKG_DIR, "libmoe_peaks.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; libmoe needs ROCm's hipcc to build")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "is not a recognized feature for this target" not in l)
    return res.returncode, out


def _compile(srcs, path, verbose, extra_flags):
    """Each source compiles to an object of its own, in parallel, then one
    link step writes the shared object (replaced atomically)."""
    flags = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"] + list(extra_flags or [])
    tag = os.path.splitext(os.path.basename(path))[0]
    objdir = os.path.join(ROOT, "_build", tag)
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.splitext(os.path.basename(s))[0] + ".o") for s in srcs]
    jobs = [[hipcc()] + flags + ["-c", s, "-o", o] for s, o in zip(srcs, objs)]
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(lambda c: _run(c, verbose), jobs))
    for (rc, out), s in zip(results, srcs):
        if rc != 0:
            raise RuntimeError(f"{os.path.basename(s)} failed to compile:\n" + out)
        if verbose and out.strip():
            print(out)
    tmp = path + ".tmp"
    rc, out = _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    if rc != 0:
        raise RuntimeError(f"{os.path.basename(path)} link failed:\n" + out)
    os.replace(tmp, path)
    return path


def build(verbose: bool = False, extra_flags=None) -> str:
    return _compile(sources(), LIB_PATH, verbose, extra_flags)


def build_peaks(verbose: bool = False, extra_flags=None) -> str:
    return _compile(sorted(glob.glob(os.path.join(PEAKS_DIR, "*.hip"))), PEAKS_LIB_PATH, verbose,
                    extra_flags)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true",
                    help="print per-kernel register/LDS usage from the compiler")
    args = ap.parse_args(argv)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if args.resource_usage else []
    for fn in (build, build_peaks):
        print(fn(verbose=args.verbose or args.resource_usage, extra_flags=extra))


if __name__ == "__main__":
    sys.exit(main())
