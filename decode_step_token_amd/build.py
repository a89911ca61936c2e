"""Build the HIP library in-tree: ``decode_step_token_amd/lib/libdst_sampler.so``.

Every source is compiled for gfx950 only, with packed-FP32 instruction
selection switched off (hipcc warns on the host pass that it does not know
the feature; that warning is harmless).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libdst_sampler.so")
# the library's sources with AddressSanitizer and UndefinedBehaviorSanitizer
# on the host side only, linked into a driver program (csrc/host_check.cpp)
HOST_CHECK = os.path.join(LIBDIR, "host_check")
SAN_BUILD = os.path.join(PKG, "_build", "host_san")

SOURCES = ["sample_stream.hip", "sample_split.hip", "sample_exact.hip", "argmax.hip",
           "write_tokens.hip", "prepare.hip", "page_table.hip", "sampler_api.hip"]
HEADERS = ["device_common.hpp", "kernels.hpp", "exact_path.hpp"]

ARCH = "gfx950"
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CFLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]
LDFLAGS = ["-shared", f"--offload-arch={ARCH}", "-Wl,-rpath,/opt/rocm/lib"]
# every sanitizer flag is host-only (-Xarch_host): the device code is built
# exactly as in the library
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


# sources whose kernels must use no scratch memory: the per-row kernel fills
# every VGPR of a CU, and a spill to scratch costs ~10 us per launch
NO_SCRATCH = ("sample_stream.hip",)
RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{p.stdout}")
    if RESOURCE_REMARKS in cmd:
        kernel = None
        for line in p.stdout.splitlines():
            if "Function Name:" in line:
                kernel = line.split("Function Name:")[1].split()[0]
            elif "ScratchSize [bytes/lane]:" in line:
                n = int(line.split("ScratchSize [bytes/lane]:")[1].split()[0])
                if n:
                    raise RuntimeError(f"{kernel} uses {n} bytes of scratch per lane: {' '.join(cmd)}")
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "warning generated" not in l and "remark:" not in l)
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False, jobs: int | None = None, host_check: bool = True) -> str:
    """Compile every source and link the shared library (and, with
    host_check, the host-sanitized driver program); returns the library's
    path."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(SAN_BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    objs, san_objs = [], []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *CFLAGS, *([RESOURCE_REMARKS] if src in NO_SCRATCH else []),
                     "-c", os.path.join(CSRC, src), "-o", obj])
    if host_check:
        for src in SOURCES + ["host_check.cpp"]:
            obj = os.path.join(SAN_BUILD, os.path.splitext(src)[0] + ".o")
            san_objs.append(obj)
            lang = ["-x", "hip"] if src.endswith(".cpp") else []
            cmds.append([HIPCC, *CFLAGS, *HOST_SAN, "-g", *lang, "-c", os.path.join(CSRC, src), "-o", obj])
    # the two largest sources first
    cmds.sort(key=lambda c: 0 if any(n in c[-3] for n in ("sample_stream", "sample_split")) else 1)
    jobs = jobs or min(len(cmds), max(1, os.cpu_count() or 2), 16)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([HIPCC, *LDFLAGS, *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    if host_check:
        tmp = HOST_CHECK + ".tmp"
        _run([HIPCC, *HOST_SAN, f"--offload-arch={ARCH}", *san_objs, "-o", tmp, "-Wl,-rpath,/opt/rocm/lib"],
             verbose)
        os.replace(tmp, HOST_CHECK)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
