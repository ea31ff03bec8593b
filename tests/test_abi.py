"""The C-ABI library loads, exports every entry point include/qmm.h declares,
and rejects bad arguments on the host before any HIP call (CPU only: no
compute call is made here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmm.h")
LIB = os.path.join(ROOT, "dequant_matmul_amd", "libqmm.so")


def _lib():
    if not os.path.exists(LIB):
        import importlib.util
        spec = importlib.util.spec_from_file_location("qmm_hip_build", os.path.join(ROOT, "dequant_matmul_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    import dequant_matmul_amd as q
    return q


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"QMM_API\s+[\w\s\*]+?\b(qmm_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    assert {"qmm_dequant", "qmm_dequant_f16", "qmm_embed", "qmm_embed_f16", "qmm_quantize", "qmm_quantize_f16",
            "qmm_gemv", "qmm_gemv_multi", "qmm_gemm_prefill", "qmm_row_bytes", "qmm_block_elems",
            "qmm_block_bytes", "qmm_status_str", "qmm_version", "qmm_gemv_pass"} == set(syms)


def test_library_exports_every_declared_symbol():
    q = _lib()
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for s in declared_symbols():
        assert s in exported, s
        assert hasattr(q.lib, s)
    # nothing else with the qmm_ prefix leaks out
    assert {s for s in exported if s.startswith("qmm_")} == set(declared_symbols())
    assert set(q.SIGNATURES) == set(declared_symbols())


def test_sizes_and_strings():
    q = _lib()
    assert [q.block_elems(t) for t in (q.Q4_0, q.Q8_0, q.Q4_K, q.Q6_K, q.Q5_0, q.Q5_K)] == [32, 32, 256, 256, 32, 256]
    assert [q.block_bytes(t) for t in (q.Q4_0, q.Q8_0, q.Q4_K, q.Q6_K, q.Q5_0, q.Q5_K)] == [18, 34, 144, 210, 22, 176]
    assert q.block_elems(6) == 0 and q.block_bytes(6) == 0
    assert q.row_bytes(q.Q4_K, 4096) == 2304 and q.row_bytes(q.Q6_K, 14336) == 11760
    assert q.row_bytes(q.Q8_0, 48) == 0 and q.row_bytes(q.Q8_0, -32) == 0 and q.row_bytes(9, 32) == 0
    assert q.block_elems(-1) == 0
    assert q.status_str(q.OK) == "ok" and "aligned" in q.status_str(q.ERR_ALIGN)
    assert q.status_str(99) == "unknown status"
    assert "gfx950" in q.version()


# Fake, never-dereferenced device addresses: every call below fails validation
# on the host, so no HIP call is made.
A = 1 << 20          # 16-byte aligned
MIS = A + 4          # not 16-byte aligned


def test_validation_errors_gemv():
    q = _lib()
    L = q.lib
    assert L.qmm_gemv(7, A, 4, 32, A, 1, A, None) == q.ERR_TYPE
    assert L.qmm_gemv(q.Q8_0, A, 4, 48, A, 1, A, None) == q.ERR_SHAPE      # k not a block multiple
    assert L.qmm_gemv(q.Q4_K, A, 4, 128, A, 1, A, None) == q.ERR_SHAPE     # 256-element blocks
    assert L.qmm_gemv(q.Q8_0, A, -1, 32, A, 1, A, None) == q.ERR_SHAPE
    assert L.qmm_gemv(q.Q8_0, A, 4, -32, A, 1, A, None) == q.ERR_SHAPE
    assert L.qmm_gemv(q.Q8_0, A, 4, 32, A, 9, A, None) == q.ERR_SHAPE      # batch > 8
    assert L.qmm_gemv(q.Q8_0, A, 4, 32, A, -1, A, None) == q.ERR_SHAPE
    assert L.qmm_gemv(q.Q8_0, None, 4, 32, A, 1, A, None) == q.ERR_NULL
    assert L.qmm_gemv(q.Q8_0, A, 4, 32, None, 1, A, None) == q.ERR_NULL
    assert L.qmm_gemv(q.Q8_0, A, 4, 32, A, 1, None, None) == q.ERR_NULL
    assert L.qmm_gemv(q.Q8_0, MIS, 4, 32, A, 1, A, None) == q.ERR_ALIGN
    assert L.qmm_gemv(q.Q8_0, A, 4, 32, MIS, 1, A, None) == q.ERR_ALIGN
    assert L.qmm_gemv(q.Q8_0, A, 4, 32, A, 1, MIS, None) == q.ERR_ALIGN
    assert L.qmm_gemv(q.Q8_0, A, 1 << 31, 32, A, 1, A, None) == q.ERR_SHAPE
    # empty problems succeed without touching the device
    assert L.qmm_gemv(q.Q8_0, None, 0, 32, None, 1, None, None) == q.OK
    assert L.qmm_gemv(q.Q8_0, A, 4, 32, A, 0, A, None) == q.OK


def test_validation_errors_dequant_and_gemm():
    q = _lib()
    L = q.lib
    assert L.qmm_dequant(6, A, 4, 32, A, None) == q.ERR_TYPE
    assert L.qmm_dequant(q.Q6_K, A, 4, 200, A, None) == q.ERR_SHAPE
    assert L.qmm_dequant(q.Q6_K, None, 4, 256, A, None) == q.ERR_NULL
    assert L.qmm_dequant(q.Q6_K, A, 4, 256, None, None) == q.ERR_NULL
    assert L.qmm_dequant(q.Q6_K, A, 4, 256, MIS, None) == q.ERR_ALIGN
    assert L.qmm_dequant(q.Q6_K, None, 0, 256, None, None) == q.OK
    assert L.qmm_dequant(q.Q6_K, None, 4, 0, None, None) == q.OK
    assert L.qmm_gemm_prefill(6, A, 4, 32, A, 8, A, None) == q.ERR_TYPE
    assert L.qmm_gemm_prefill(q.Q4_0, A, 4, 16, A, 8, A, None) == q.ERR_SHAPE
    assert L.qmm_gemm_prefill(q.Q4_0, A, 4, 32, A, -8, A, None) == q.ERR_SHAPE
    assert L.qmm_gemm_prefill(q.Q4_0, A, 4, 32, None, 8, A, None) == q.ERR_NULL
    assert L.qmm_gemm_prefill(q.Q4_0, A, 4, 32, A, 8, None, None) == q.ERR_NULL
    assert L.qmm_gemm_prefill(q.Q4_0, MIS, 4, 32, A, 8, A, None) == q.ERR_ALIGN
    assert L.qmm_gemm_prefill(q.Q4_0, A, 4, 32, A + 8, 8, A, None) == q.ERR_ALIGN
    assert L.qmm_gemm_prefill(q.Q4_0, A, 4, 32, A, 0, None, None) == q.OK
    assert L.qmm_gemm_prefill(q.Q4_0, None, 0, 32, None, 8, None, None) == q.OK


def test_validation_errors_dequant_f16_and_embed():
    q = _lib()
    L = q.lib
    assert L.qmm_dequant_f16(6, A, 4, 32, A, None) == q.ERR_TYPE
    assert L.qmm_dequant_f16(q.Q4_K, A, 4, 32, A, None) == q.ERR_SHAPE
    assert L.qmm_dequant_f16(q.Q4_K, None, 4, 256, A, None) == q.ERR_NULL
    assert L.qmm_dequant_f16(q.Q4_K, A, 4, 256, None, None) == q.ERR_NULL
    assert L.qmm_dequant_f16(q.Q4_K, A, 4, 256, A + 8, None) == q.ERR_ALIGN
    assert L.qmm_dequant_f16(q.Q4_K, None, 0, 256, None, None) == q.OK
    for f in (L.qmm_embed, L.qmm_embed_f16):
        assert f(7, A, 100, 32, A, 4, A, None) == q.ERR_TYPE
        assert f(q.Q8_0, A, 100, 40, A, 4, A, None) == q.ERR_SHAPE
        assert f(q.Q8_0, A, -1, 32, A, 4, A, None) == q.ERR_SHAPE        # negative vocab
        assert f(q.Q8_0, A, 100, 32, A, -4, A, None) == q.ERR_SHAPE      # negative seq
        assert f(q.Q8_0, A, 100, 32, A, 1 << 31, A, None) == q.ERR_SHAPE
        assert f(q.Q8_0, None, 100, 32, A, 4, A, None) == q.ERR_NULL
        assert f(q.Q8_0, A, 100, 32, None, 4, A, None) == q.ERR_NULL
        assert f(q.Q8_0, A, 100, 32, A, 4, None, None) == q.ERR_NULL
        assert f(q.Q8_0, MIS, 100, 32, A, 4, A, None) == q.ERR_ALIGN     # table
        assert f(q.Q8_0, A, 100, 32, A + 2, 4, A, None) == q.ERR_ALIGN   # ids need 4-byte alignment
        assert f(q.Q8_0, A, 100, 32, A, 4, MIS, None) == q.ERR_ALIGN
        # empty problems succeed without touching the device
        assert f(q.Q8_0, A, 100, 32, None, 0, None, None) == q.OK
        assert f(q.Q8_0, A, 100, 0, A, 4, None, None) == q.OK


def test_validation_errors_quantize():
    q = _lib()
    L = q.lib
    for f in (L.qmm_quantize, L.qmm_quantize_f16):
        for t in (q.Q4_K, q.Q6_K, q.Q5_0, q.Q5_K, 6, -1):      # the encoder covers Q8_0 and Q4_0 only
            assert f(t, A, 4, 256, A, None) == q.ERR_TYPE
        assert f(q.Q8_0, A, 4, 48, A, None) == q.ERR_SHAPE
        assert f(q.Q4_0, A, -4, 32, A, None) == q.ERR_SHAPE
        assert f(q.Q4_0, A, 4, 32, None, None) == q.ERR_NULL
        assert f(q.Q4_0, None, 4, 32, A, None) == q.ERR_NULL
        assert f(q.Q4_0, MIS, 4, 32, A, None) == q.ERR_ALIGN
        assert f(q.Q4_0, A, 4, 32, A + 2, None) == q.ERR_ALIGN
        assert f(q.Q8_0, None, 0, 32, None, None) == q.OK
        assert f(q.Q8_0, None, 4, 0, None, None) == q.OK


def test_validation_errors_gemv_multi():
    q = _lib()
    L = q.lib
    P2 = ctypes.c_void_p * 2
    N2 = ctypes.c_int64 * 2
    w, x, y = P2(A, A + 4096), P2(A, A), P2(A, A + 256)
    n = N2(4, 8)
    assert L.qmm_gemv_multi(q.Q4_K, 0, None, None, 256, None, 1, None, None) == q.OK
    assert L.qmm_gemv_multi(q.Q4_K, -1, w, n, 256, x, 1, y, None) == q.ERR_SHAPE
    assert L.qmm_gemv_multi(q.Q4_K, 2, None, n, 256, x, 1, y, None) == q.ERR_NULL
    assert L.qmm_gemv_multi(q.Q4_K, 2, w, None, 256, x, 1, y, None) == q.ERR_NULL
    assert L.qmm_gemv_multi(9, 2, w, n, 256, x, 1, y, None) == q.ERR_TYPE
    assert L.qmm_gemv_multi(q.Q4_K, 2, w, n, 128, x, 1, y, None) == q.ERR_SHAPE
    assert L.qmm_gemv_multi(q.Q4_K, 2, w, n, 256, x, 9, y, None) == q.ERR_SHAPE
    assert L.qmm_gemv_multi(q.Q4_K, 2, w, N2(4, -1), 256, x, 1, y, None) == q.ERR_SHAPE
    assert L.qmm_gemv_multi(q.Q4_K, 2, P2(A, A + 4), n, 256, x, 1, y, None) == q.ERR_ALIGN
    assert L.qmm_gemv_multi(q.Q4_K, 2, P2(A, None), n, 256, x, 1, y, None) == q.ERR_NULL
    assert L.qmm_gemv_multi(q.Q4_K, 2, w, n, 256, P2(A, MIS), 1, y, None) == q.ERR_ALIGN
    assert L.qmm_gemv_multi(q.Q4_K, 2, w, n, 256, x, 1, P2(A, None), None) == q.ERR_NULL
    # the second problem is bad: nothing of the first may be enqueued either
    assert L.qmm_gemv_multi(q.Q4_K, 2, w, N2(4, 8), 256, P2(A, None), 1, y, None) == q.ERR_NULL
    assert L.qmm_gemv_multi(q.Q4_K, 2, w, n, 256, x, 0, y, None) == q.OK
    assert L.qmm_gemv_multi(q.Q4_K, 2, P2(None, None), N2(0, 0), 256, x, 1, y, None) == q.OK


def test_validation_errors_gemv_pass():
    q = _lib()
    L = q.lib

    def call(*rows):
        t = (q.PassGemv * len(rows))()
        for i, r in enumerate(rows):
            t[i] = q.PassGemv(*r)
        return L.qmm_gemv_pass(len(rows), ctypes.cast(t, ctypes.c_void_p), None)

    ok = (A, A, A, 64, 4096, q.Q4_K, 0)
    assert L.qmm_gemv_pass(0, None, None) == q.OK
    assert L.qmm_gemv_pass(-1, None, None) == q.ERR_SHAPE
    assert L.qmm_gemv_pass(1, None, None) == q.ERR_NULL
    assert call((A, A, A, 64, 4096, 9, 0)) == q.ERR_TYPE
    assert call((A, A, A, 64, 4000, q.Q4_K, 0)) == q.ERR_SHAPE            # k not a block multiple
    assert call((A, A, A, -1, 4096, q.Q4_K, 0)) == q.ERR_SHAPE
    assert call((A, A, A, 64, -256, q.Q4_K, 0)) == q.ERR_SHAPE
    assert call((A, A, A, 64, 4096, q.Q4_K, -1)) == q.ERR_SHAPE           # negative stage
    assert call((A, A, A, 64, 4096, q.Q4_K, 1), ok) == q.ERR_SHAPE        # stages decrease
    assert call((None, A, A, 64, 4096, q.Q4_K, 0)) == q.ERR_NULL
    assert call((A, None, A, 64, 4096, q.Q4_K, 0)) == q.ERR_NULL
    assert call((A, A, None, 64, 4096, q.Q4_K, 0)) == q.ERR_NULL
    assert call((MIS, A, A, 64, 4096, q.Q4_K, 0)) == q.ERR_ALIGN
    assert call((A, MIS, A, 64, 4096, q.Q4_K, 0)) == q.ERR_ALIGN
    assert call((A, A, MIS, 64, 4096, q.Q4_K, 0)) == q.ERR_ALIGN
    # a bad later problem: nothing of the earlier ones is enqueued either
    assert call(ok, (A, None, A, 64, 4096, q.Q4_K, 1)) == q.ERR_NULL
    # empty problems are skipped (null pointers allowed); nothing to run -> OK
    assert call((None, None, None, 0, 4096, q.Q4_K, 0)) == q.OK


def test_binding_has_no_cpu_fallback():
    """The package refuses to import without the HIP library."""
    code = ("import sys, os; sys.path.insert(0, %r); import dequant_matmul_amd as q" % ROOT)
    env = dict(os.environ)
    # point the loader at a path without the library by copying the package
    import shutil
    import tempfile
    d = tempfile.mkdtemp()
    shutil.copytree(os.path.join(ROOT, "dequant_matmul_amd"), os.path.join(d, "dequant_matmul_amd"),
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    r = subprocess.run(["python", "-c", code.replace(repr(ROOT), repr(d))], capture_output=True, text=True,
                       env=env)
    shutil.rmtree(d)
    assert r.returncode != 0 and "libqmm.so not built" in r.stderr
