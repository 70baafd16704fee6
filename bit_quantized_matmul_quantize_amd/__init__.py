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
LIB_PATH = os.path.join(_HERE, "libbqmm.so")

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

def quantize_act_q8_1(act, out_q8, m: int, k: int, stream=None):
    _check(lib().quantize_act_q8_1(_ptr(_bf16(act, "act")), _ptr(_u8(out_q8, "out_q8")), m, k, _stream(stream)))


def silu_mul_quantize_q8_1(gate, up, out_q8, m: int, k: int, stream=None):
    _check(lib().silu_mul_quantize_q8_1(_ptr(_bf16(gate, "gate")), _ptr(_bf16(up, "up")),
                                        _ptr(_u8(out_q8, "out_q8")), m, k, _stream(stream)))


def q2_0_mmq_gemm(act_q8, w_q2, out, m: int, n: int, k: int, stream=None):
    _check(lib().q2_0_mmq_gemm(_ptr(_u8(act_q8, "act_q8")), _ptr(_u8(w_q2, "w_q2")), _ptr(_bf16(out, "out")),
                               m, n, k, _stream(stream)))


def _ptr_rows(t, m: int, n: int, ldc: int, what):
    """A [m, n] bf16 view whose rows are ldc elements apart (a column range of a wider buffer)."""
    _bf16(t, what)
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if tuple(t.shape) != (m, n) or (m > 1 and t.stride(0) != ldc) or (n > 1 and t.stride(1) != 1):
        raise ValueError(f"{what}: expected an [{m}, {n}] view with row stride {ldc}")
    return ctypes.c_void_p(t.data_ptr())


def q2_0_mmq_gemm_ldc(act_q8, w_q2, out, m: int, n: int, k: int, ldc: int, stream=None):
    _check(lib().q2_0_mmq_gemm_ldc(_ptr(_u8(act_q8, "act_q8")), _ptr(_u8(w_q2, "w_q2")),
                                   _ptr_rows(out, m, n, ldc, "out"), m, n, k, ldc, _stream(stream)))


def q4k_mmq_gemm_ldc(act_q8, w_q4k, out, m: int, n: int, k: int, ldc: int, stream=None):
    _check(lib().q4k_mmq_gemm_ldc(_ptr(_u8(act_q8, "act_q8")), _ptr(_u8(w_q4k, "w_q4k")),
                                  _ptr_rows(out, m, n, ldc, "out"), m, n, k, ldc, _stream(stream)))


def q2_0_gemv_vec(act, w_q2, out, n: int, k: int, stream=None):
    _check(lib().q2_0_gemv_vec(_ptr(_bf16(act, "act")), _ptr(_u8(w_q2, "w_q2")), _ptr(_bf16(out, "out")),
                               n, k, _stream(stream)))


def q2_0_gemv_vec_batchm(act, w_q2, out, m: int, n: int, k: int, stream=None):
    _check(lib().q2_0_gemv_vec_batchm(_ptr(_bf16(act, "act")), _ptr(_u8(w_q2, "w_q2")),
                                      _ptr(_bf16(out, "out")), m, n, k, _stream(stream)))


def q2_0_gemv_gate_up_silu(act, w_gate, w_up, out, m: int, n: int, k: int, stream=None):
    _check(lib().q2_0_gemv_gate_up_silu(_ptr(_bf16(act, "act")), _ptr(_u8(w_gate, "w_gate")),
                                        _ptr(_u8(w_up, "w_up")), _ptr(_bf16(out, "out")), m, n, k,
                                        _stream(stream)))


def dequant_q2_0_to_bf16(w_q2, out, n: int, k: int, group: int = 128, stream=None):
    _check(lib().dequant_q2_0_to_bf16(_ptr(_u8(w_q2, "w_q2")), _ptr(_bf16(out, "out")), n, k, group,
                                      _stream(stream)))


def dense_gemm_bf16(a, w, out, m: int, n: int, k: int, stream=None):
    _check(lib().dense_gemm_bf16(_ptr(_bf16(a, "a")), _ptr(_bf16(w, "w")), _ptr(_bf16(out, "out")),
                                 m, n, k, _stream(stream)))


def q2_0_prefill_gemm(act, w_q2, out, scratch, act_q8, m: int, n: int, k: int, group: int = 128,
                      use_mmq: bool = True, stream=None):
    _check(lib().q2_0_prefill_gemm(_ptr(_bf16(act, "act")), _ptr(_u8(w_q2, "w_q2")), _ptr(_bf16(out, "out")),
                                   _ptr(scratch), _ptr(act_q8), m, n, k, group, int(bool(use_mmq)),
                                   _stream(stream)))


def q4k_mmq_gemm(act_q8, w_q4k, out, m: int, n: int, k: int, stream=None):
    _check(lib().q4k_mmq_gemm(_ptr(_u8(act_q8, "act_q8")), _ptr(_u8(w_q4k, "w_q4k")), _ptr(_bf16(out, "out")),
                              m, n, k, _stream(stream)))


def q4k_gemv_vec(act, w_q4k, out, n: int, k: int, stream=None):
    _check(lib().q4k_gemv_vec(_ptr(_bf16(act, "act")), _ptr(_u8(w_q4k, "w_q4k")), _ptr(_bf16(out, "out")),
                              n, k, _stream(stream)))


def quantize_weight_q4k(w, out_q4k, n: int, k: int, stream=None):
    _check(lib().quantize_weight_q4k(_ptr(_bf16(w, "w")), _ptr(_u8(out_q4k, "out_q4k")), n, k,
                                     _stream(stream)))


def silu_mul_bf16(gate, up, out, count: int | None = None, stream=None):
    count = gate.numel() if count is None else count
    _check(lib().silu_mul_bf16(_ptr(_bf16(gate, "gate")), _ptr(_bf16(up, "up")), _ptr(_bf16(out, "out")),
                               count, _stream(stream)))


def q2_0_mmq_blockdots(act_q8, w_q2, out_i32, m0: int, mt: int, n0: int, nt: int, m: int, n: int, k: int,
                       stream=None):
    _check(lib().q2_0_mmq_blockdots(_ptr(_u8(act_q8, "act_q8")), _ptr(_u8(w_q2, "w_q2")), _ptr(out_i32),
                                    m0, mt, n0, nt, m, n, k, _stream(stream)))


def q4k_mmq_blockdots(act_q8, w_q4k, out_i32, m0: int, mt: int, n0: int, nt: int, m: int, n: int, k: int,
                      stream=None):
    _check(lib().q4k_mmq_blockdots(_ptr(_u8(act_q8, "act_q8")), _ptr(_u8(w_q4k, "w_q4k")), _ptr(out_i32),
                                   m0, mt, n0, nt, m, n, k, _stream(stream)))
