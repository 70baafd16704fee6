"""Measured ceilings of the benchmark (bench-only): a ctypes binding of
libceilings.so, built from ceilings.hip for gfx950.  Nothing in the
bit_quantized_matmul_quantize_amd package uses it."""
from __future__ import annotations

import ctypes
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "ceilings.hip")
LIB_PATH = os.path.join(_HERE, "libceilings.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
_lib = None


def build() -> str:
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", SRC, "-o", tmp],
                          stderr=subprocess.DEVNULL)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with ceilings.build()")
        l = ctypes.CDLL(LIB_PATH)
        P, U32, U64 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64
        for name, args in (("ceil_empty", [U32, U32, P]), ("ceil_stream_read", [P, U64, P, U32, P]),
                           ("ceil_stream_read_write", [P, U64, P, U32, U32, P]),
                           ("ceil_mfma_i8", [U32, U32, P, P]), ("ceil_mfma_f16", [U32, U32, P, P]),
                           ("ceil_valu_mad", [U32, U32, P, P]),
                           ("ceil_mix", [U32, U32, ctypes.c_int, U32, P, P]),
                           ("ceil_lds", [U32, U32, ctypes.c_int, P, P])):
            f = getattr(l, name)
            f.restype = ctypes.c_int
            f.argtypes = args
        _lib = l
    return _lib


def call(name, *args):
    status = getattr(lib(), name)(*args)
    if status != 0:
        raise RuntimeError(f"{name}: HIP error {status}")
