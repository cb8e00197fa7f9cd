"""Build liblongflow.so in-tree with hipcc for gfx950.

    python -m decode_kv_cache_02_amd.build            # the library
    python -m decode_kv_cache_02_amd.build --phases   # its measurement build

Every HIP source is compiled with packed-FP32 instructions disabled. The
library lands next to this file, where the binding loads it. The measurement
build, liblongflow_phases.so, is the same source compiled with
LF_PHASE_STAMPS=1: its decode kernels also record when each phase of a step
ends (lf_probe_decode_phases), which costs the latency-bound launches a few
hundred nanoseconds, so the library itself leaves the stamps out.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "liblongflow.so")
PHASES_LIB_PATH = os.path.join(PKG_DIR, "liblongflow_phases.so")
SOURCES = ("lf_decode_w4.hip", "lf_decode_w8.hip", "lf_decode_w4i.hip", "lf_decode_w8i.hip",
           "lf_kernels.hip", "lf_runtime.cpp", "lf_probe.hip", "lf_scratch.hip")
HEADERS = ("lf_decode.h", "lf_internal.h")
ARCH = os.environ.get("LONGFLOW_OFFLOAD_ARCH", "gfx950")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the LongFlow HIP library cannot be built")


def compile_commands(obj_dir: str, phases: bool = False) -> list:
    """One hipcc -c per source (they build in parallel)."""
    extra = ["-DLF_PHASE_STAMPS=1"] if phases else []
    return [[hipcc(), f"--offload-arch={ARCH}", *FLAGS, *extra, "-I", INCLUDE, "-c",
             os.path.join(CSRC, src), "-o", os.path.join(obj_dir, src + ".o")]
            for src in SOURCES]


def link_command(obj_dir: str, out_path: str) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC",
            *[os.path.join(obj_dir, src + ".o") for src in SOURCES], "-o", out_path]


def build(verbose: bool = False, phases: bool = False) -> str:
    """Build liblongflow.so, or with `phases` its measurement build."""
    lib_path = PHASES_LIB_PATH if phases else LIB_PATH
    with tempfile.TemporaryDirectory(prefix="longflow_build_") as obj_dir:
        procs = []
        for cmd in compile_commands(obj_dir, phases):
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                          text=True))
        failed = False
        for p in procs:
            out, err = p.communicate()
            if p.returncode != 0:
                failed = True
                sys.stderr.write(out + err)
            elif verbose and err.strip():
                sys.stderr.write(err)
        if failed:
            raise RuntimeError("hipcc failed")
        tmp = lib_path + ".tmp"
        cmd = link_command(obj_dir, tmp)
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc link failed with exit code {res.returncode}")
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, phases="--phases" in sys.argv))
