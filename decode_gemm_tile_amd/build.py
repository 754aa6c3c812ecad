"""Build libdgt.so in-tree for gfx950 (hipcc; the four weight formats compile in
parallel).  Run ``python -m decode_gemm_tile_amd.build`` or call ``build()``."""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdgt.so")
PROBES = os.path.join(HERE, "..", "tests", "probes")
PROBE_LIB = os.path.join(PROBES, "libmfma_probe.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 VALU instructions: the compiler would otherwise form them
    # from scalar and float2 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]
FORMATS = {"int8": 1, "int4": 2, "fp8": 3, "bf16": 4, "int4p": 5, "bf16e": 6, "bf16p": 7,
           "bf16w": 8}


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libdgt")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), out))
    return out


def _stale(obj, src):
    """True if obj is missing or older than its source or any header."""
    if not os.path.exists(obj):
        return True
    deps = [src, os.path.join(HERE, "..", "include", "dgt.h")]
    deps += [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(d) > t for d in deps)


def build(verbose: bool = False, jobs: int = None, incremental: bool = False) -> str:
    """Compile every HIP/C++ source and link libdgt.so; returns its path.
    incremental=True recompiles only objects older than their sources."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 4)
    steps = []
    host_obj = os.path.join(BUILD, "dgt_host.o")
    steps.append(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-c",
                  os.path.join(CSRC, "dgt_host.cpp"), "-o", host_obj])
    objs = [host_obj]
    for name, val in FORMATS.items():
        obj = os.path.join(BUILD, f"dgt_fmt_{name}.o")
        steps.append([hipcc] + HIP_FLAGS + [f"-DDGT_FMT={val}", "-c",
                                            os.path.join(CSRC, "dgt_fmt.hip"), "-o", obj])
        objs.append(obj)
    api_obj = os.path.join(BUILD, "dgt_api.o")
    steps.append([hipcc] + HIP_FLAGS + ["-c", os.path.join(CSRC, "dgt_api.hip"), "-o", api_obj])
    objs.append(api_obj)
    if incremental:
        steps = [c for c in steps if _stale(c[-1], c[-3])]
    with cf.ThreadPoolExecutor(jobs) as ex:
        for out in ex.map(_run, steps):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs + ["-lpthread"])
    os.replace(tmp, LIB)
    # the matrix-instruction precision probe the GPU tests load (not part of libdgt)
    probe_src = os.path.join(PROBES, "mfma_precision.hip")
    if os.path.exists(probe_src) and (not incremental or _stale(PROBE_LIB, probe_src)):
        _run([hipcc] + HIP_FLAGS + ["-shared", probe_src, "-o", PROBE_LIB + ".tmp"])
        os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, incremental="--incremental" in sys.argv))
