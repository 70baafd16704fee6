"""Build libbqmm.so in-tree with hipcc for gfx950 only.

    python -m bit_quantized_matmul_quantize_amd.build [--sanitize]

Each HIP source compiles to its own object (in parallel), then one shared
library is linked next to this file.  Flags: -O3, IEEE-correct binary32
division (the q8_1 codes depend on it), no fast-math, and packed-FP32
instruction selection turned off.

--sanitize builds libbqmm_san.so instead: the C ABI layer (capi.cpp, all the
argument checking) with AddressSanitizer and UndefinedBehaviorSanitizer on
its host code only (device code is never instrumented), linked with the
ordinary kernel objects.  It needs clang's ASan runtime preloaded into the
process; tests/run_sanitized.sh runs the CPU test suite that way.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libbqmm.so")
LIB_SAN = os.path.join(HERE, "libbqmm_san.so")
# host-only sanitizers: each -fsanitize applies to the host compilation pass
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-shared-libsan", "-g"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["quantize.hip", "quantize_q4k.hip", "elementwise.hip", "gemv.hip", "gemv_mfma.hip",
           "gemv_q4k.hip", "mmq_q2.hip", "mmq_q4k.hip", "gemm_bf16.hip", "capi.cpp"]

COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(HERE, "..", "include"),
]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        san = sanitize and src.endswith(".cpp")
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ("_san.o" if san else ".o"))
        cmd = [HIPCC, *COMMON, *(SANITIZE if san else [])]
        if src.endswith(".cpp"):
            cmd += ["-x", "hip"]
        cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = "\n".join(l for l in out.decode(errors="replace").splitlines()
                         if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write(text + "\n")
        elif verbose and text.strip():
            print(text)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    lib = LIB_SAN if sanitize else LIB
    tmp = lib + ".tmp%d" % os.getpid()
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if sanitize:
        link[3:3] = ["-fsanitize=address,undefined", "-shared-libsan"]
    subprocess.check_call(link)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
