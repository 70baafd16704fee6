"""ctypes binding of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__.py
and the cpu_baseline leg of bench.py may import this module.  The product
library never imports, links or calls it, and it imports nothing from the
product package.

All arrays are numpy arrays on the host: bf16 and fp16 values travel as their
uint16 bit patterns, packed weights and q8_1 buffers as uint8 byte arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# BQMM_SANITIZE=1 selects an AddressSanitizer + UndefinedBehaviorSanitizer
# build (clang, whose runtime the sanitized C ABI library shares); it is for
# the CPU test suite only (tests/run_sanitized.sh).
_SANITIZE = os.environ.get("BQMM_SANITIZE") == "1"
_LIB_PATH = os.path.join(_HERE, "liboracle_san.so" if _SANITIZE else "liboracle.so")
_CLANG = os.environ.get("BQMM_CLANG", "/opt/rocm/llvm/bin/clang")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (plain -O2, no fast-math),
    or, under BQMM_SANITIZE=1, into liboracle_san.so with clang and the
    address and undefined-behaviour sanitizers."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        if _SANITIZE:
            cmd = [_CLANG, "-std=c11", "-O1", "-g", "-Wall", "-Wextra", "-fPIC", "-shared",
                   "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                   "-shared-libsan", _SRC, "-o", tmp, "-lm"]
        else:
            cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        U32, U64 = ctypes.c_uint32, ctypes.c_uint64
        sig = {
            "oracle_f16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
            "oracle_f32_to_f16": (ctypes.c_uint16, [ctypes.c_float]),
            "oracle_bf16_to_f64": (ctypes.c_double, [ctypes.c_uint16]),
            "oracle_f64_to_bf16": (ctypes.c_uint16, [ctypes.c_double]),
            "oracle_q8_1_kpad": (U64, [U32]),
            "oracle_q8_1_bytes": (U64, [U32, U32]),
            "oracle_quantize_act_q8_1": (ctypes.c_int64, [P, P, U32, U32]),
            "oracle_dequant_q8_1": (None, [P, P, U32, U32]),
            "oracle_q2_0_bytes": (U64, [U32, U32, U32]),
            "oracle_q2_0_decode": (None, [P, P, U32, U32, U32]),
            "oracle_dequant_q2_0_to_bf16": (None, [P, P, U32, U32, U32]),
            "oracle_q2_0_blockdots": (None, [P, P, P, U32, U32, U32]),
            "oracle_q2_0_mmq": (None, [P, P, P, U32, U32, U32]),
            "oracle_q2_0_gemv": (None, [P, P, P, U32, U32, U32]),
            "oracle_dense_gemm_bf16": (None, [P, P, P, U32, U32, U32]),
            "oracle_silu_mul_bf16": (None, [P, P, P, U64]),
            "oracle_round_bf16": (None, [P, P, U64]),
            "oracle_q4k_bytes": (U64, [U32, U32]),
            "oracle_q4k_decode": (None, [P, P, U32, U32]),
            "oracle_q4k_blockdots": (None, [P, P, P, U32, U32, U32]),
            "oracle_q4k_mmq": (None, [P, P, P, U32, U32, U32]),
            "oracle_q4k_gemv": (None, [P, P, P, U32, U32, U32]),
            "oracle_quantize_weight_q4k": (ctypes.c_int64, [P, P, U32, U32]),
        }
        for name, (res, args) in sig.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def _u8(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint8, a.dtype
    return a


# --- scalar conversions ----------------------------------------------------

def f16_to_f32(h: int) -> float:
    return _load().oracle_f16_to_f32(int(h))


def f32_to_f16(x: float) -> int:
    return _load().oracle_f32_to_f16(float(np.float32(x)))


def bf16_to_f64(b: int) -> float:
    return _load().oracle_bf16_to_f64(int(b))


def f64_to_bf16(x: float) -> int:
    return _load().oracle_f64_to_bf16(float(x))


# --- q8_1 ------------------------------------------------------------------

def q8_1_kpad(k: int) -> int:
    return int(_load().oracle_q8_1_kpad(k))


def q8_1_bytes(m: int, k: int) -> int:
    return int(_load().oracle_q8_1_bytes(m, k))


def quantize_act_q8_1(act_bf16: np.ndarray, m: int, k: int):
    """bf16 bits [m][k] -> (q8_1 byte buffer, number of out-of-range blocks)."""
    a = _u16(act_bf16).reshape(-1)
    assert a.size == m * k
    out = np.zeros(q8_1_bytes(m, k), dtype=np.uint8)
    flagged = _load().oracle_quantize_act_q8_1(_ptr(a), _ptr(out), m, k)
    return out, int(flagged)


def dequant_q8_1(q8: np.ndarray, m: int, k: int) -> np.ndarray:
    kp = q8_1_kpad(k)
    out = np.zeros((m, kp), dtype=np.float64)
    _load().oracle_dequant_q8_1(_ptr(_u8(q8)), _ptr(out), m, k)
    return out


# --- Q2_0 ------------------------------------------------------------------

def q2_0_bytes(n: int, k: int, group: int = 128) -> int:
    return int(_load().oracle_q2_0_bytes(n, k, group))


def q2_0_decode(w: np.ndarray, n: int, k: int, group: int = 128) -> np.ndarray:
    out = np.zeros((n, k), dtype=np.float64)
    _load().oracle_q2_0_decode(_ptr(_u8(w)), _ptr(out), n, k, group)
    return out


def dequant_q2_0_to_bf16(w: np.ndarray, n: int, k: int, group: int = 128) -> np.ndarray:
    out = np.zeros((n, k), dtype=np.uint16)
    _load().oracle_dequant_q2_0_to_bf16(_ptr(_u8(w)), _ptr(out), n, k, group)
    return out


def q2_0_blockdots(q8: np.ndarray, w: np.ndarray, m: int, n: int, k: int) -> np.ndarray:
    out = np.zeros((m, n, k // 32), dtype=np.int32)
    _load().oracle_q2_0_blockdots(_ptr(_u8(q8)), _ptr(_u8(w)), _ptr(out), m, n, k)
    return out


def q2_0_mmq(q8: np.ndarray, w: np.ndarray, m: int, n: int, k: int) -> np.ndarray:
    out = np.zeros((m, n), dtype=np.float64)
    _load().oracle_q2_0_mmq(_ptr(_u8(q8)), _ptr(_u8(w)), _ptr(out), m, n, k)
    return out


def q2_0_gemv(act_bf16: np.ndarray, w: np.ndarray, m: int, n: int, k: int) -> np.ndarray:
    out = np.zeros((m, n), dtype=np.float64)
    _load().oracle_q2_0_gemv(_ptr(_u16(act_bf16)), _ptr(_u8(w)), _ptr(out), m, n, k)
    return out


def dense_gemm_bf16(a_bf16: np.ndarray, w_bf16: np.ndarray, m: int, n: int, k: int) -> np.ndarray:
    out = np.zeros((m, n), dtype=np.float64)
    _load().oracle_dense_gemm_bf16(_ptr(_u16(a_bf16)), _ptr(_u16(w_bf16)), _ptr(out), m, n, k)
    return out


def silu_mul_bf16(gate_bf16: np.ndarray, up_bf16: np.ndarray) -> np.ndarray:
    g = _u16(gate_bf16)
    u = _u16(up_bf16)
    assert g.shape == u.shape
    out = np.zeros(g.shape, dtype=np.uint16)
    _load().oracle_silu_mul_bf16(_ptr(g), _ptr(u), _ptr(out), g.size)
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint16)
    _load().oracle_round_bf16(_ptr(x), _ptr(out), x.size)
    return out


# --- Q4_K ------------------------------------------------------------------

def q4k_bytes(n: int, k: int) -> int:
    return int(_load().oracle_q4k_bytes(n, k))


def q4k_decode(w: np.ndarray, n: int, k: int) -> np.ndarray:
    out = np.zeros((n, k), dtype=np.float64)
    _load().oracle_q4k_decode(_ptr(_u8(w)), _ptr(out), n, k)
    return out


def q4k_blockdots(q8: np.ndarray, w: np.ndarray, m: int, n: int, k: int) -> np.ndarray:
    out = np.zeros((m, n, k // 32), dtype=np.int32)
    _load().oracle_q4k_blockdots(_ptr(_u8(q8)), _ptr(_u8(w)), _ptr(out), m, n, k)
    return out


def q4k_mmq(q8: np.ndarray, w: np.ndarray, m: int, n: int, k: int) -> np.ndarray:
    out = np.zeros((m, n), dtype=np.float64)
    _load().oracle_q4k_mmq(_ptr(_u8(q8)), _ptr(_u8(w)), _ptr(out), m, n, k)
    return out


def q4k_gemv(act_bf16: np.ndarray, w: np.ndarray, m: int, n: int, k: int) -> np.ndarray:
    out = np.zeros((m, n), dtype=np.float64)
    _load().oracle_q4k_gemv(_ptr(_u16(act_bf16)), _ptr(_u8(w)), _ptr(out), m, n, k)
    return out


def quantize_weight_q4k(w_bf16: np.ndarray, n: int, k: int):
    """bf16 weight bits [n][k] -> (block_q4_K bytes, number of super-blocks
    outside the supported range)."""
    w = _u16(w_bf16)
    assert w.size == n * k and k % 256 == 0
    out = np.zeros(q4k_bytes(n, k), dtype=np.uint8)
    flagged = _load().oracle_quantize_weight_q4k(_ptr(w), _ptr(out), n, k)
    return out, int(flagged)


# --- chains (compositions of the functions above) ---------------------------

def ffn_chain_gemv(x_bf16: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray,
                   m: int, hidden: int, inter: int):
    """gate = GEMV(x, Wg); up = GEMV(x, Wu); h = silu(gate) * up; out = GEMV(h, Wd).

    [page layers/dense_ffn_decode_batch.rs, fn forward_km_q2.]  Rounded to
    bf16 at the same points as the device chain: after each projection and
    after silu_mul.  Returns (gate, up, h) as bf16 bits and out in fp64.
    """
    gate = round_bf16(q2_0_gemv(x_bf16, wg, m, inter, hidden))
    up = round_bf16(q2_0_gemv(x_bf16, wu, m, inter, hidden))
    h = silu_mul_bf16(gate, up)
    out = q2_0_gemv(h, wd, m, hidden, inter)
    return gate, up, h, out
