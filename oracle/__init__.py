"""CPU oracle for the quantized-weight matmul -- TEST INFRASTRUCTURE ONLY.

Thin ctypes wrapper over ``qmm_oracle.c`` (plain C, fp64 accumulation).  Only
the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package; the product library never does, and this package
imports nothing from the product package.

Every function here is a definition written out (see the C file's header for
the page/section each one follows); none of them is tuned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qmm_oracle.c")
_LIB = os.path.join(_HERE, "libqmm_oracle.so")

# Type ids (same numeric values as the public C-ABI; defined here on purpose,
# not imported, so the oracle stays independent of the product package).
Q4_0, Q8_0, Q4_K, Q6_K, Q5_0, Q5_K = 0, 1, 2, 3, 4, 5
TYPES = {"Q4_0": Q4_0, "Q8_0": Q8_0, "Q4_K": Q4_K, "Q6_K": Q6_K, "Q5_0": Q5_0, "Q5_K": Q5_K}

GCC_FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
             "-Wall", "-Wextra", "-shared", "-fPIC"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libqmm_oracle.so``."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.oracle_block_elems.argtypes = [ctypes.c_int]
        L.oracle_block_bytes.argtypes = [ctypes.c_int]
        L.oracle_row_bytes.argtypes = [ctypes.c_int, I64]
        L.oracle_row_bytes.restype = ctypes.c_size_t
        L.oracle_half_to_float_array.argtypes = [P, I64, P]
        L.oracle_half_to_float_array.restype = None
        L.oracle_q4k_scale_min.argtypes = [P, ctypes.c_int, P, P]
        L.oracle_q4k_scale_min.restype = None
        L.oracle_dequant.argtypes = [ctypes.c_int, P, I64, I64, P]
        L.oracle_dequant_f64.argtypes = [ctypes.c_int, P, I64, I64, P]
        L.oracle_gemv.argtypes = [ctypes.c_int, P, I64, I64, P, I64, P, P]
        L.oracle_gemm.argtypes = [ctypes.c_int, P, I64, I64, P, I64, P, I64, P, P]
        L.oracle_double_to_half.argtypes = [ctypes.c_double]
        L.oracle_double_to_half.restype = ctypes.c_uint16
        L.oracle_float_to_half_array.argtypes = [P, I64, P]
        L.oracle_float_to_half_array.restype = None
        L.oracle_embed.argtypes = [ctypes.c_int, P, I64, I64, P, I64, P]
        L.oracle_quantize.argtypes = [ctypes.c_int, P, I64, I64, P]
        L.oracle_quantize_f16.argtypes = [ctypes.c_int, P, I64, I64, P]
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        L.oracle_set_threads.restype = None
        L.oracle_max_threads.argtypes = []
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError("oracle %s failed (code %d)" % (what, rc))


def block_elems(t: int) -> int:
    return lib().oracle_block_elems(t)


def block_bytes(t: int) -> int:
    return lib().oracle_block_bytes(t)


def row_bytes(t: int, k: int) -> int:
    return lib().oracle_row_bytes(t, k)


def half_to_float(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().oracle_half_to_float_array(_ptr(h), h.size, _ptr(out))
    return out


def to_half_bits(x) -> np.ndarray:
    """fp32 values -> IEEE binary16 bit patterns (uint16), nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_float_to_half_array(_ptr(x), x.size, _ptr(out))
    return out


def double_to_half_bits(v: float) -> int:
    """One fp64 value -> binary16 bits, nearest-even."""
    return int(lib().oracle_double_to_half(float(v)))


def q4k_scale_min(s12: bytes | np.ndarray, j: int) -> tuple[int, int]:
    s = np.ascontiguousarray(np.frombuffer(bytes(s12), dtype=np.uint8))
    assert s.size == 12
    sc = ctypes.c_int(0)
    m = ctypes.c_int(0)
    lib().oracle_q4k_scale_min(_ptr(s), j, ctypes.addressof(sc), ctypes.addressof(m))
    return sc.value, m.value


def _wbytes(w: np.ndarray, t: int, n: int, k: int) -> np.ndarray:
    w = np.ascontiguousarray(w, dtype=np.uint8).reshape(-1)
    if w.size != n * row_bytes(t, k):
        raise ValueError("weight buffer has %d bytes, expected %d" % (w.size, n * row_bytes(t, k)))
    return w


def dequant(t: int, w: np.ndarray, n: int, k: int) -> np.ndarray:
    """Exact fp32 dequant, row-major [n, k]."""
    w = _wbytes(w, t, n, k)
    out = np.empty((n, k), dtype=np.float32)
    _check(lib().oracle_dequant(t, _ptr(w), n, k, _ptr(out)), "dequant")
    return out


def dequant_f64(t: int, w: np.ndarray, n: int, k: int) -> np.ndarray:
    """Exact weight values in fp64 (no fp32 rounding), [n, k]."""
    w = _wbytes(w, t, n, k)
    out = np.empty((n, k), dtype=np.float64)
    _check(lib().oracle_dequant_f64(t, _ptr(w), n, k, _ptr(out)), "dequant_f64")
    return out


def dequant_f16(t: int, w: np.ndarray, n: int, k: int) -> np.ndarray:
    """fp16 dequant (bits, uint16 [n, k]): the fp32 dequant rounded to
    binary16, nearest-even."""
    return to_half_bits(dequant(t, w, n, k))


def embed(t: int, table: np.ndarray, vocab: int, k: int, ids, f16: bool = False) -> np.ndarray:
    """Embedding gather: row i = fp32 dequant of table row ids[i] (zeros for
    an id outside [0, vocab)); ``f16`` returns binary16 bits instead."""
    table = _wbytes(table, t, vocab, k)
    ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32).reshape(-1))
    out = np.empty((ids.size, k), dtype=np.float32)
    _check(lib().oracle_embed(t, _ptr(table), vocab, k, _ptr(ids), ids.size, _ptr(out)), "embed")
    return to_half_bits(out) if f16 else out


def quantize(t: int, x: np.ndarray) -> np.ndarray:
    """Q8_0 / Q4_0 encoder: x float32 or float16 [n, k] (k a multiple of 32)
    -> block bytes uint8 [n, row_bytes]."""
    x = np.ascontiguousarray(x)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    n, k = x.shape
    out = np.empty((n, row_bytes(t, k) if row_bytes(t, k) else 0), dtype=np.uint8)
    if x.dtype == np.float16:
        xb = np.ascontiguousarray(x.view(np.uint16))
        rc = lib().oracle_quantize_f16(t, _ptr(xb), n, k, _ptr(out))
    else:
        xf = np.ascontiguousarray(x, dtype=np.float32)
        rc = lib().oracle_quantize(t, _ptr(xf), n, k, _ptr(out))
    _check(rc, "quantize")
    return out


def gemv(t: int, w: np.ndarray, n: int, k: int, x: np.ndarray):
    """y[b, n] = sum_k w[n, k] x[b, k] (fp64) and a = sum_k |w x|.

    x: float32 [batch, k] (or [k] for batch 1).  Returns (y, a), each
    float64 [batch, n]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    assert x.shape[1] == k
    B = x.shape[0]
    w = _wbytes(w, t, n, k)
    y = np.empty((B, n), dtype=np.float64)
    a = np.empty((B, n), dtype=np.float64)
    _check(lib().oracle_gemv(t, _ptr(w), n, k, _ptr(x), B, _ptr(y), _ptr(a)), "gemv")
    return y, a


def gemm(t: int, w: np.ndarray, n: int, k: int, x_f16bits: np.ndarray, rows=None):
    """Y[m, n] = sum_k X[m, k] w[n, k] with X as fp16 bits [m, k] (uint16 or
    float16).  ``rows``: optional list of m indices to compute (compact
    output).  Returns (Y, A) float64 [len(rows) or m, n]."""
    xb = np.ascontiguousarray(x_f16bits)
    if xb.dtype == np.float16:
        xb = xb.view(np.uint16)
    xb = np.ascontiguousarray(xb, dtype=np.uint16)
    m = xb.shape[0]
    assert xb.shape[1] == k
    w = _wbytes(w, t, n, k)
    if rows is None:
        rp, nr = None, m
    else:
        rarr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        rp, nr = _ptr(rarr), rarr.size
    y = np.empty((nr, n), dtype=np.float64)
    a = np.empty((nr, n), dtype=np.float64)
    _check(lib().oracle_gemm(t, _ptr(w), n, k, _ptr(xb), m, rp, nr, _ptr(y), _ptr(a)), "gemm")
    return y, a


def set_threads(nthreads: int) -> None:
    lib().oracle_set_threads(int(nthreads))


def max_threads() -> int:
    return lib().oracle_max_threads()
