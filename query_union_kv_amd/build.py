"""Builds libpw.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(os.path.dirname(HERE), "_build")
LIB = os.path.join(HERE, "libpw.so")
# the same library with -DPW_DEBUG (device-side invariant counters)
DEBUG_LIB = os.path.join(HERE, "libpw_debug.so")
# read-bandwidth probes used by the benchmark (not part of the library's method)
PROBE_LIB = os.path.join(HERE, "libpw_probe.so")
PROBE_SOURCES = ["probe.hip"]
ARCH = "gfx950"

SOURCES = ["api.cpp", "kvcache.hip", "prep.hip", "pageunion.hip", "attn.hip", "noalloc.hip"]
# Packed fp32 ops are disabled for every device compile on this hardware.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found")
    return exe


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def _compile_all(hipcc, out_dir, extra, verbose):
    os.makedirs(out_dir, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(out_dir, src + ".o")
        objs.append(obj)
        cmd = [hipcc, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    return objs, procs


def _finish(hipcc, objs, procs, lib, verbose):
    for cmd, pr in procs:
        out, _ = pr.communicate()
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if pr.returncode != 0:
            raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
        if verbose and out.strip():
            print(out)
    tmp = lib + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, lib)


def build(verbose: bool = False, debug: bool = True) -> str:
    """libpw.so, libpw_probe.so and (debug=True) libpw_debug.so, the same sources with
    -DPW_DEBUG: device-side invariant counters, read by pw_debug_violations()."""
    hipcc = _hipcc()
    rel = _compile_all(hipcc, BUILD, [], verbose)
    dbg = _compile_all(hipcc, os.path.join(BUILD, "debug"), ["-DPW_DEBUG"], verbose) if debug else None
    _finish(hipcc, *rel, LIB, verbose)
    if dbg:
        _finish(hipcc, *dbg, DEBUG_LIB, verbose)
    pobjs = []
    for src in PROBE_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run([hipcc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        pobjs.append(obj)
    tmp = PROBE_LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *pobjs, "-o", tmp], verbose)
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
