"""Packed low-bit weight-quantized matmul for AMD Instinct MI355X (gfx950).

Thin ctypes binding over libbqmm.so (C ABI in include/bqmm.h).  The binding
only marshals arguments: every step runs in the library's HIP kernels.  torch
is used for device memory and the current stream; tensors must be contiguous
CUDA (HIP) tensors.  bf16 data travels as torch.bfloat16 (or int16/uint16
views), packed weights and q8_1 buffers as torch.uint8.

The library must be built first (python -m bit_quantized_matmul_quantize_amd.build);
there is no fallback implementation: a missing library raises ImportError on
first use.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# BQMM_SANITIZE=1 selects the host-sanitized build of the same library (see
# build.py); it is for the CPU test suite only.
LIB_PATH = os.path.join(_HERE, "libbqmm_san.so" if os.environ.get("BQMM_SANITIZE") == "1" else "libbqmm.so")

BQ_OK, BQ_EINVAL, BQ_EUNSUPPORTED, BQ_EALIGN, BQ_EHIP = 0, -1, -2, -3, -4

# name -> (restype, argtypes); P = pointer, U32/U64 = unsigned ints, I = int
_P, _U32, _U64, _I = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int
EXPORTS = {
    "bq_last_error": (ctypes.c_char_p, []),
    "bq_status_string": (ctypes.c_char_p, [_I]),
    "q8_1_act_bytes": (_U64, [_U32, _U32]),
    "q2_0_weight_bytes": (_U64, [_U32, _U32, _U32]),
    "q4k_weight_bytes": (_U64, [_U32, _U32]),
    "quantize_act_q8_1": (_I, [_P, _P, _U32, _U32, _P]),
    "silu_mul_quantize_q8_1": (_I, [_P, _P, _P, _U32, _U32, _P]),
    "q2_0_mmq_gemm": (_I, [_P, _P, _P, _U32, _U32, _U32, _P]),
    "q2_0_mmq_gemm_ldc": (_I, [_P, _P, _P, _U32, _U32, _U32, _U32, _P]),
    "q4k_mmq_gemm_ldc": (_I, [_P, _P, _P, _U32, _U32, _U32, _U32, _P]),
    "q2_0_gemv_vec": (_I, [_P, _P, _P, _U32, _U32, _P]),
    "q2_0_gemv_vec_batchm": (_I, [_P, _P, _P, _U32, _U32, _U32, _P]),
    "q2_0_gemv_gate_up_silu": (_I, [_P, _P, _P, _P, _U32, _U32, _U32, _P]),
    "dequant_q2_0_to_bf16": (_I, [_P, _P, _U32, _U32, _U32, _P]),
    "dense_gemm_bf16": (_I, [_P, _P, _P, _U32, _U32, _U32, _P]),
    "q2_0_prefill_gemm": (_I, [_P, _P, _P, _P, _P, _U32, _U32, _U32, _U32, _I, _P]),
    "q2_0_prefill_gemm_noalloc": (_I, [_P, _P, _P, _U32, _U32, _U32, _U32, _I, _P]),
    "q4k_mmq_gemm": (_I, [_P, _P, _P, _U32, _U32, _U32, _P]),
    "q4k_gemv_vec": (_I, [_P, _P, _P, _U32, _U32, _P]),
    "quantize_weight_q4k": (_I, [_P, _P, _U32, _U32, _P]),
    "silu_mul_bf16": (_I, [_P, _P, _P, _U64, _P]),
    "q2_0_mmq_blockdots": (_I, [_P, _P, _P, _U32, _U32, _U32, _U32, _U32, _U32, _U32, _P]),
    "q4k_mmq_blockdots": (_I, [_P, _P, _P, _U32, _U32, _U32, _U32, _U32, _U32, _U32, _P]),
}

_lib = None


class BqmmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


def lib():
    """Load libbqmm.so (raises ImportError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m bit_quantized_matmul_quantize_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def _check(status: int):
    if status != BQ_OK:
        raise BqmmError(status, lib().bq_last_error().decode())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _bf16(t, what):
    import torch
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{what}: expected bfloat16 data, got {t.dtype}")
    return t


def _u8(t, what):
    import torch
    if t.dtype != torch.uint8:
        raise TypeError(f"{what}: expected uint8 bytes, got {t.dtype}")
    return t


# ---- sizes ------------------------------------------------------------------

def q8_1_act_bytes(m: int, k: int) -> int:
    return int(lib().q8_1_act_bytes(m, k))


def q2_0_weight_bytes(n: int, k: int, group: int = 128) -> int:
    return int(lib().q2_0_weight_bytes(n, k, group))


def q4k_weight_bytes(n: int, k: int) -> int:
    return int(lib().q4k_weight_bytes(n, k))


# ---- calls (same names as the C ABI) -----------------------------------------
#
# Each wrapper checks, before anything reaches the library: dtypes, that every
# tensor holds at least the bytes its shape arguments address (the C ABI sees
# plain pointers and cannot), and that all tensors are contiguous device
# tensors on one device.

def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _need(t, nbytes: int, what: str):
    if t is not None and _nbytes(t) < nbytes:
        raise ValueError(f"{what}: {_nbytes(t)} bytes, the shape arguments address {nbytes}")
    return t


def _same_device(*tensors):
    devs = {t.device for t in tensors if t is not None and t.is_cuda}
    if len(devs) > 1:
        raise ValueError(f"tensors on different devices: {sorted(str(d) for d in devs)}")


def _ptrs(*tensors):
    """Device pointers of the given contiguous tensors (None passes through), all on one device."""
    _same_device(*tensors)
    return [_ptr(t) for t in tensors]


def _bf(m: int, k: int) -> int:
    return 2 * m * k


def quantize_act_q8_1(act, out_q8, m: int, k: int, stream=None):
    _need(_bf16(act, "act"), _bf(m, k), "act")
    _need(_u8(out_q8, "out_q8"), q8_1_act_bytes(m, k), "out_q8")
    _check(lib().quantize_act_q8_1(*_ptrs(act, out_q8), m, k, _stream(stream)))


def silu_mul_quantize_q8_1(gate, up, out_q8, m: int, k: int, stream=None):
    _need(_bf16(gate, "gate"), _bf(m, k), "gate")
    _need(_bf16(up, "up"), _bf(m, k), "up")
    _need(_u8(out_q8, "out_q8"), q8_1_act_bytes(m, k), "out_q8")
    _check(lib().silu_mul_quantize_q8_1(*_ptrs(gate, up, out_q8), m, k, _stream(stream)))


def q2_0_mmq_gemm(act_q8, w_q2, out, m: int, n: int, k: int, stream=None):
    _need(_u8(act_q8, "act_q8"), q8_1_act_bytes(m, k), "act_q8")
    _need(_u8(w_q2, "w_q2"), q2_0_weight_bytes(n, k), "w_q2")
    _need(_bf16(out, "out"), _bf(m, n), "out")
    _check(lib().q2_0_mmq_gemm(*_ptrs(act_q8, w_q2, out), m, n, k, _stream(stream)))


def _ptr_rows(t, m: int, n: int, ldc: int, what):
    """A [m, n] bf16 view whose rows are ldc elements apart (a column range of a wider buffer)."""
    _bf16(t, what)
    if tuple(t.shape) != (m, n) or (m > 1 and t.stride(0) != ldc) or (n > 1 and t.stride(1) != 1):
        raise ValueError(f"{what}: expected an [{m}, {n}] view with row stride {ldc}")
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    return ctypes.c_void_p(t.data_ptr())


def q2_0_mmq_gemm_ldc(act_q8, w_q2, out, m: int, n: int, k: int, ldc: int, stream=None):
    _need(_u8(act_q8, "act_q8"), q8_1_act_bytes(m, k), "act_q8")
    _need(_u8(w_q2, "w_q2"), q2_0_weight_bytes(n, k), "w_q2")
    out_p = _ptr_rows(out, m, n, ldc, "out")
    _same_device(act_q8, w_q2, out)
    a_p, w_p = _ptrs(act_q8, w_q2)
    _check(lib().q2_0_mmq_gemm_ldc(a_p, w_p, out_p, m, n, k, ldc, _stream(stream)))


def q4k_mmq_gemm_ldc(act_q8, w_q4k, out, m: int, n: int, k: int, ldc: int, stream=None):
    _need(_u8(act_q8, "act_q8"), q8_1_act_bytes(m, k), "act_q8")
    _need(_u8(w_q4k, "w_q4k"), q4k_weight_bytes(n, k), "w_q4k")
    out_p = _ptr_rows(out, m, n, ldc, "out")
    _same_device(act_q8, w_q4k, out)
    a_p, w_p = _ptrs(act_q8, w_q4k)
    _check(lib().q4k_mmq_gemm_ldc(a_p, w_p, out_p, m, n, k, ldc, _stream(stream)))


def q2_0_gemv_vec(act, w_q2, out, n: int, k: int, stream=None):
    _need(_bf16(act, "act"), _bf(1, k), "act")
    _need(_u8(w_q2, "w_q2"), q2_0_weight_bytes(n, k), "w_q2")
    _need(_bf16(out, "out"), _bf(1, n), "out")
    _check(lib().q2_0_gemv_vec(*_ptrs(act, w_q2, out), n, k, _stream(stream)))


def q2_0_gemv_vec_batchm(act, w_q2, out, m: int, n: int, k: int, stream=None):
    _need(_bf16(act, "act"), _bf(m, k), "act")
    _need(_u8(w_q2, "w_q2"), q2_0_weight_bytes(n, k), "w_q2")
    _need(_bf16(out, "out"), _bf(m, n), "out")
    _check(lib().q2_0_gemv_vec_batchm(*_ptrs(act, w_q2, out), m, n, k, _stream(stream)))


def q2_0_gemv_gate_up_silu(act, w_gate, w_up, out, m: int, n: int, k: int, stream=None):
    _need(_bf16(act, "act"), _bf(m, k), "act")
    _need(_u8(w_gate, "w_gate"), q2_0_weight_bytes(n, k), "w_gate")
    _need(_u8(w_up, "w_up"), q2_0_weight_bytes(n, k), "w_up")
    _need(_bf16(out, "out"), _bf(m, n), "out")
    _check(lib().q2_0_gemv_gate_up_silu(*_ptrs(act, w_gate, w_up, out), m, n, k, _stream(stream)))


def dequant_q2_0_to_bf16(w_q2, out, n: int, k: int, group: int = 128, stream=None):
    _need(_u8(w_q2, "w_q2"), q2_0_weight_bytes(n, k, group), "w_q2")
    _need(_bf16(out, "out"), _bf(n, k), "out")
    _check(lib().dequant_q2_0_to_bf16(*_ptrs(w_q2, out), n, k, group, _stream(stream)))


def dense_gemm_bf16(a, w, out, m: int, n: int, k: int, stream=None):
    _need(_bf16(a, "a"), _bf(m, k), "a")
    _need(_bf16(w, "w"), _bf(n, k), "w")
    _need(_bf16(out, "out"), _bf(m, n), "out")
    _check(lib().dense_gemm_bf16(*_ptrs(a, w, out), m, n, k, _stream(stream)))


def q2_0_prefill_gemm(act, w_q2, out, scratch, act_q8, m: int, n: int, k: int, group: int = 128,
                      use_mmq: bool = True, stream=None):
    _need(_bf16(act, "act"), _bf(m, k), "act")
    _need(_u8(w_q2, "w_q2"), q2_0_weight_bytes(n, k, group), "w_q2")
    _need(_bf16(out, "out"), _bf(m, n), "out")
    if use_mmq and group == 128:  # the MMQ branch writes act_q8, the dequant branch scratch
        _need(act_q8, q8_1_act_bytes(m, k), "act_q8")
    else:
        _need(scratch, _bf(n, k), "scratch")
    _check(lib().q2_0_prefill_gemm(*_ptrs(act, w_q2, out, scratch, act_q8), m, n, k, group,
                                   int(bool(use_mmq)), _stream(stream)))


def q2_0_prefill_gemm_noalloc(act, w_q2, out, m: int, n: int, k: int, group: int = 128,
                              use_mmq: bool = True, stream=None):
    _need(_bf16(act, "act"), _bf(m, k), "act")
    _need(_u8(w_q2, "w_q2"), q2_0_weight_bytes(n, k, group), "w_q2")
    _need(_bf16(out, "out"), _bf(m, n), "out")
    _check(lib().q2_0_prefill_gemm_noalloc(*_ptrs(act, w_q2, out), m, n, k, group, int(bool(use_mmq)),
                                           _stream(stream)))


def q4k_mmq_gemm(act_q8, w_q4k, out, m: int, n: int, k: int, stream=None):
    _need(_u8(act_q8, "act_q8"), q8_1_act_bytes(m, k), "act_q8")
    _need(_u8(w_q4k, "w_q4k"), q4k_weight_bytes(n, k), "w_q4k")
    _need(_bf16(out, "out"), _bf(m, n), "out")
    _check(lib().q4k_mmq_gemm(*_ptrs(act_q8, w_q4k, out), m, n, k, _stream(stream)))


def q4k_gemv_vec(act, w_q4k, out, n: int, k: int, stream=None):
    _need(_bf16(act, "act"), _bf(1, k), "act")
    _need(_u8(w_q4k, "w_q4k"), q4k_weight_bytes(n, k), "w_q4k")
    _need(_bf16(out, "out"), _bf(1, n), "out")
    _check(lib().q4k_gemv_vec(*_ptrs(act, w_q4k, out), n, k, _stream(stream)))


def quantize_weight_q4k(w, out_q4k, n: int, k: int, stream=None):
    _need(_bf16(w, "w"), _bf(n, k), "w")
    _need(_u8(out_q4k, "out_q4k"), q4k_weight_bytes(n, k), "out_q4k")
    _check(lib().quantize_weight_q4k(*_ptrs(w, out_q4k), n, k, _stream(stream)))


def silu_mul_bf16(gate, up, out, count: int | None = None, stream=None):
    count = gate.numel() if count is None else count
    for t, what in ((gate, "gate"), (up, "up"), (out, "out")):
        _need(_bf16(t, what), 2 * count, what)
    _check(lib().silu_mul_bf16(*_ptrs(gate, up, out), count, _stream(stream)))


def _blockdots(fn, act_q8, w, w_bytes, out_i32, m0, mt, n0, nt, m, n, k, stream):
    import torch
    _need(_u8(act_q8, "act_q8"), q8_1_act_bytes(m, k), "act_q8")
    _need(_u8(w, "w"), w_bytes, "w")
    if out_i32.dtype != torch.int32:
        raise TypeError(f"out_i32: expected int32, got {out_i32.dtype}")
    _need(out_i32, 4 * mt * nt * (k // 32), "out_i32")
    _check(fn(*_ptrs(act_q8, w, out_i32), m0, mt, n0, nt, m, n, k, _stream(stream)))


def q2_0_mmq_blockdots(act_q8, w_q2, out_i32, m0: int, mt: int, n0: int, nt: int, m: int, n: int, k: int,
                       stream=None):
    _blockdots(lib().q2_0_mmq_blockdots, act_q8, w_q2, q2_0_weight_bytes(n, k), out_i32, m0, mt, n0, nt,
               m, n, k, stream)


def q4k_mmq_blockdots(act_q8, w_q4k, out_i32, m0: int, mt: int, n0: int, nt: int, m: int, n: int, k: int,
                      stream=None):
    _blockdots(lib().q4k_mmq_blockdots, act_q8, w_q4k, q4k_weight_bytes(n, k), out_i32, m0, mt, n0, nt,
               m, n, k, stream)
