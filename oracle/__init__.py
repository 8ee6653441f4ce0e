"""CPU oracle for C = A·Bᵀ (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU product path never imports,
links or calls it, and the two share no code.

The arithmetic lives in ``gemm_ref.c`` (plain C, fp64 accumulation in
increasing k, exact decoders for the 16-bit and OCP 8-bit input formats, IEEE
round-to-nearest-even encoders, and an exact int64 path for 8-bit integer
inputs); this module only builds it with gcc, loads it with ctypes and marshals numpy
arrays.  The tolerance rules are in ``oracle.tolerance``.

Definition followed ("Optimizing Blackwell matrix multiplication in Mojo
(part 2)", section "Starting from the 4-line kernel"; "Chapter 7: Writing
custom kernels with Pallas", sections 4.1 and 4.1'):

    C[i, j] = sum_k A[i, k] * B[j, k],   A: M x K row-major, B: N x K row-major.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

F32, F16, BF16, FP8_E4M3, FP8_E5M2 = 0, 1, 2, 3, 4
_NAMES = {"f32": F32, "f16": F16, "bf16": BF16, "e4m3": FP8_E4M3, "e5m2": FP8_E5M2}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_ref.c")
_SO = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile gemm_ref.c with gcc (no fast-math, no FMA contraction)."""
    if not force and os.path.exists(_SO) and os.path.getmtime(_SO) >= os.path.getmtime(_SRC):
        return _SO
    tmp = _SO + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            lib = ctypes.CDLL(_SO)
            p = ctypes.c_void_p
            i64 = ctypes.c_int64
            ci = ctypes.c_int
            lib.orc_gemm_bt.argtypes = [p, p, i64, i64, i64, ci, p, p, p, ci]
            lib.orc_gemm_bt.restype = ci
            lib.orc_gemm_bt_entries.argtypes = [p, p, i64, i64, i64, ci, p, p, i64, p, ci]
            lib.orc_gemm_bt_entries.restype = ci
            lib.orc_row_norms.argtypes = [p, i64, i64, ci, p, ci]
            lib.orc_row_norms.restype = ci
            lib.orc_decode.argtypes = [p, i64, ci, p]
            lib.orc_decode.restype = None
            lib.orc_round.argtypes = [p, i64, ci, p]
            lib.orc_round.restype = None
            lib.orc_max_threads.restype = ci
            lib.orc_gemm_bt_i8.argtypes = [p, p, i64, i64, i64, p, ci]
            lib.orc_gemm_bt_i8.restype = ci
            lib.orc_gemm_bt_i8_entries.argtypes = [p, p, i64, i64, i64, p, p, i64, p, ci]
            lib.orc_gemm_bt_i8_entries.restype = ci
            _lib = lib
    return _lib


def dtype_code(d) -> int:
    if isinstance(d, str):
        return _NAMES[d]
    return int(d)


def _u16(x: np.ndarray) -> np.ndarray:
    """Input bits as uint16 words: 16-bit codes as they are, 8-bit codes widened."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint8:
        return x.astype(np.uint16)
    if x.dtype != np.uint16:
        x = x.view(np.uint16)
    return x


def _ptr(x: np.ndarray):
    return x.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    return int(_load().orc_max_threads())


def decode(bits: np.ndarray, in_dtype) -> np.ndarray:
    """Exact value of each bf16/f16/e4m3/e5m2 bit pattern, as float64."""
    b = _u16(bits)
    out = np.empty(b.shape, dtype=np.float64)
    _load().orc_decode(_ptr(b), b.size, dtype_code(in_dtype), _ptr(out))
    return out


def round_to(x: np.ndarray, out_dtype) -> np.ndarray:
    """IEEE round-to-nearest-even of float64 values to the output format.

    Returns uint32 bits for f32, uint16 bits for f16/bf16.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    code = dtype_code(out_dtype)
    out = np.empty(x.shape, dtype=np.uint32 if code == F32 else np.uint16)
    _load().orc_round(_ptr(x), x.size, code, _ptr(out))
    return out


def gemm_bt_ref(a_bits: np.ndarray, b_bits: np.ndarray, in_dtype, nthreads: int = 0):
    """Full product in fp64: returns (C (M,N) float64, ‖A_i‖₂ (M,), ‖B_j‖₂ (N,))."""
    a = _u16(a_bits)
    b = _u16(b_bits)
    M, K = a.shape
    N, K2 = b.shape
    if K != K2:
        raise ValueError("A is %dx%d but B is %dx%d" % (M, K, N, K2))
    C = np.empty((M, N), dtype=np.float64)
    nA = np.empty(M, dtype=np.float64)
    nB = np.empty(N, dtype=np.float64)
    rc = _load().orc_gemm_bt(_ptr(a), _ptr(b), M, N, K, dtype_code(in_dtype),
                             _ptr(C), _ptr(nA), _ptr(nB), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected arguments")
    return C, nA, nB


def gemm_bt_entries(a_bits: np.ndarray, b_bits: np.ndarray, in_dtype, I, J,
                    nthreads: int = 0) -> np.ndarray:
    """C[I[t], J[t]] in fp64 for each t (a sample of a large product)."""
    a = _u16(a_bits)
    b = _u16(b_bits)
    M, K = a.shape
    N, K2 = b.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    I = np.ascontiguousarray(I, dtype=np.int64)
    J = np.ascontiguousarray(J, dtype=np.int64)
    if I.shape != J.shape:
        raise ValueError("I and J differ in shape")
    out = np.empty(I.shape, dtype=np.float64)
    rc = _load().orc_gemm_bt_entries(_ptr(a), _ptr(b), M, N, K, dtype_code(in_dtype),
                                     _ptr(I), _ptr(J), I.size, _ptr(out), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected arguments")
    return out


def row_norms(x_bits: np.ndarray, in_dtype, nthreads: int = 0) -> np.ndarray:
    """2-norm of each row of a 16-bit matrix, in fp64."""
    x = _u16(x_bits)
    R, K = x.shape
    out = np.empty(R, dtype=np.float64)
    rc = _load().orc_row_norms(_ptr(x), R, K, dtype_code(in_dtype), _ptr(out), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected arguments")
    return out


def _i8(x: np.ndarray) -> np.ndarray:
    """Two's-complement bytes as an int8 array (int8 or uint8 input)."""
    x = np.ascontiguousarray(x)
    if x.dtype not in (np.int8, np.uint8):
        raise ValueError("8-bit integer inputs must be int8 or uint8 arrays")
    return x.view(np.int8)


def gemm_bt_i8(a: np.ndarray, b: np.ndarray, nthreads: int = 0) -> np.ndarray:
    """Exact product of int8 operands: C (M,N) int64 = sum_k A[i,k]*B[j,k]."""
    a = _i8(a)
    b = _i8(b)
    M, K = a.shape
    N, K2 = b.shape
    if K != K2:
        raise ValueError("A is %dx%d but B is %dx%d" % (M, K, N, K2))
    C = np.empty((M, N), dtype=np.int64)
    if _load().orc_gemm_bt_i8(_ptr(a), _ptr(b), M, N, K, _ptr(C), int(nthreads)) != 0:
        raise ValueError("oracle rejected arguments")
    return C


def gemm_bt_i8_entries(a: np.ndarray, b: np.ndarray, I, J, nthreads: int = 0) -> np.ndarray:
    """C[I[t], J[t]] (int64) for each t, for int8 operands."""
    a = _i8(a)
    b = _i8(b)
    M, K = a.shape
    N, K2 = b.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    I = np.ascontiguousarray(I, dtype=np.int64)
    J = np.ascontiguousarray(J, dtype=np.int64)
    if I.shape != J.shape:
        raise ValueError("I and J differ in shape")
    out = np.empty(I.shape, dtype=np.int64)
    if _load().orc_gemm_bt_i8_entries(_ptr(a), _ptr(b), M, N, K, _ptr(I), _ptr(J), I.size, _ptr(out),
                                      int(nthreads)) != 0:
        raise ValueError("oracle rejected arguments")
    return out


def gemm_bt_batched_ref(a_bits: np.ndarray, b_bits: np.ndarray, in_dtype, nthreads: int = 0):
    """Batched product: C[z] = A[z]·B[z]ᵀ in fp64 for each item z ("Chapter 7: Writing custom kernels
    with Pallas", section 5.2: a batch runs the unchanged product once per item; an operand given
    as 2-D is shared by every item).  Returns (C (Z,M,N), ‖A_z,i‖ (Z,M), ‖B_z,j‖ (Z,N)); int8 inputs
    return (C int64, None, None)."""
    a = np.asarray(a_bits)
    b = np.asarray(b_bits)
    Z = a.shape[0] if a.ndim == 3 else b.shape[0]
    if a.ndim == 3 and b.ndim == 3 and a.shape[0] != b.shape[0]:
        raise ValueError("batch sizes differ")
    Cs, nAs, nBs = [], [], []
    for z in range(Z):
        az = a[z] if a.ndim == 3 else a
        bz = b[z] if b.ndim == 3 else b
        if in_dtype == "i8":
            Cs.append(gemm_bt_i8(az, bz, nthreads))
        else:
            c, nA, nB = gemm_bt_ref(az, bz, in_dtype, nthreads)
            Cs.append(c)
            nAs.append(nA)
            nBs.append(nB)
    if in_dtype == "i8":
        return np.stack(Cs), None, None
    return np.stack(Cs), np.stack(nAs), np.stack(nBs)
