"""dequant_matmul_amd -- quantized-weight matmul on AMD MI355X (gfx950).

Python binding of ``libqmm.so`` (C ABI declared in ``include/qmm.h``).  This
module only marshals arguments: it checks tensor dtypes/devices, allocates the
output with torch, and passes raw device pointers plus torch's current HIP
stream to the library, where every step of the computation runs.  There is no
CPU fallback: if the library is missing, importing this package fails.

    import dequant_matmul_amd as qmm
    y = qmm.gemv(w_bytes, qmm.Q4_K, n, k, x)          # x fp32 [B, k] -> y fp32 [B, n]
    Y = qmm.gemm_prefill(w_bytes, qmm.Q4_K, n, k, X)  # X fp16 [m, k] -> Y fp32 [m, n]
    W = qmm.dequant(w_bytes, qmm.Q4_K, n, k)          # -> fp32 [n, k]
    H = qmm.embed(table, qmm.Q8_0, vocab, k, ids)      # ids int32 [seq] -> fp32 [seq, k]
    B = qmm.quantize(kv_f16, qmm.Q8_0)                 # fp16 [n, k] -> Q8_0 blocks

Block types and layouts follow shimmy "Architecture" (Quantization table) and
dotLLM "GPU Inference" (Quantization on GPU table); see include/qmm.h.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmm.so")

Q4_0, Q8_0, Q4_K, Q6_K, Q5_0, Q5_K = 0, 1, 2, 3, 4, 5
TYPE_NAMES = {Q4_0: "Q4_0", Q8_0: "Q8_0", Q4_K: "Q4_K", Q6_K: "Q6_K", Q5_0: "Q5_0", Q5_K: "Q5_K"}
OK, ERR_NULL, ERR_TYPE, ERR_SHAPE, ERR_ALIGN, ERR_HIP = range(6)

# C-ABI entry points and their ctypes signatures (mirrors include/qmm.h).
_P, _I, _I64, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "qmm_block_elems": (_I, [_I]),
    "qmm_block_bytes": (_I, [_I]),
    "qmm_row_bytes": (_SZ, [_I, _I64]),
    "qmm_dequant": (_I, [_I, _P, _I64, _I64, _P, _P]),
    "qmm_dequant_f16": (_I, [_I, _P, _I64, _I64, _P, _P]),
    "qmm_embed": (_I, [_I, _P, _I64, _I64, _P, _I64, _P, _P]),
    "qmm_embed_f16": (_I, [_I, _P, _I64, _I64, _P, _I64, _P, _P]),
    "qmm_quantize": (_I, [_I, _P, _I64, _I64, _P, _P]),
    "qmm_quantize_f16": (_I, [_I, _P, _I64, _I64, _P, _P]),
    "qmm_gemv": (_I, [_I, _P, _I64, _I64, _P, _I64, _P, _P]),
    "qmm_gemv_multi": (_I, [_I, _I, _P, _P, _I64, _P, _I64, _P, _P]),
    "qmm_gemm_prefill": (_I, [_I, _P, _I64, _I64, _P, _I64, _P, _P]),
    "qmm_gemv_pass": (_I, [_I, _P, _P]),
    "qmm_status_str": (ctypes.c_char_p, [_I]),
    "qmm_version": (ctypes.c_char_p, []),
}


class QmmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (what, status_str(status), status))


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError("libqmm.so not built: run `python dequant_matmul_amd/build.py` "
                          "(expected at %s)" % LIB_PATH)
    # torch first: it loads its own copy of the HIP runtime by path, and this
    # library must bind to that copy (loaded first, the library would pull in
    # a second runtime whose streams and graphs are not torch's)
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


lib = _load()


def status_str(status: int) -> str:
    return lib.qmm_status_str(int(status)).decode()


def version() -> str:
    return lib.qmm_version().decode()


def block_elems(qtype: int) -> int:
    return lib.qmm_block_elems(qtype)


def block_bytes(qtype: int) -> int:
    return lib.qmm_block_bytes(qtype)


def row_bytes(qtype: int, k: int) -> int:
    return lib.qmm_row_bytes(qtype, k)


def _torch():
    import torch
    return torch


def _stream_ptr(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _check_w(w, qtype: int, n: int, k: int):
    torch = _torch()
    if w.dtype != torch.uint8 or not w.is_cuda:
        raise TypeError("weights must be a uint8 tensor on a HIP device")
    if not w.is_contiguous():
        raise ValueError("weights must be contiguous")
    rb = row_bytes(qtype, k)
    if (n > 0 and k > 0) and w.numel() != n * rb:
        raise ValueError("weight tensor has %d bytes, expected n * row_bytes = %d" % (w.numel(), n * rb))


def _out(out, shape, dtype, device):
    """The caller's output tensor, checked (the library writes exactly
    prod(shape) elements of dtype there), or a new one."""
    torch = _torch()
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if (out.dtype != dtype or tuple(out.shape) != tuple(shape) or not out.is_contiguous()
            or out.device != torch.device(device)):
        raise ValueError("out must be a contiguous %s tensor of shape %s on %s (got %s %s on %s)"
                         % (dtype, tuple(shape), device, out.dtype, tuple(out.shape), out.device))
    return out


def _call(status: int, what: str) -> None:
    if status != OK:
        raise QmmError(status, what)


def dequant(w, qtype: int, n: int, k: int, out=None):
    """fp32 [n, k] dequantized weights (bit-exact)."""
    torch = _torch()
    _check_w(w, qtype, n, k)
    out = _out(out, (n, k), torch.float32, w.device)
    _call(lib.qmm_dequant(qtype, w.data_ptr(), n, k, out.data_ptr(), _stream_ptr(w.device)), "qmm_dequant")
    return out


def dequant_f16(w, qtype: int, n: int, k: int, out=None):
    """fp16 [n, k] dequantized weights (the fp32 values rounded to nearest-even)."""
    torch = _torch()
    _check_w(w, qtype, n, k)
    out = _out(out, (n, k), torch.float16, w.device)
    _call(lib.qmm_dequant_f16(qtype, w.data_ptr(), n, k, out.data_ptr(), _stream_ptr(w.device)),
          "qmm_dequant_f16")
    return out


def embed(table, qtype: int, vocab: int, k: int, ids, dtype=None, out=None):
    """Embedding gather: row r = dequantized table row ids[r] (zeros for an id
    outside [0, vocab)).  ids: int32 device tensor [seq]; dtype float32
    (default, exact) or float16."""
    torch = _torch()
    _check_w(table, qtype, vocab, k)
    dtype = torch.float32 if dtype is None else dtype
    if ids.dtype != torch.int32 or not ids.is_cuda or ids.dim() != 1 or not ids.is_contiguous():
        raise ValueError("ids must be a contiguous int32 device tensor [seq]")
    seq = ids.shape[0]
    if dtype not in (torch.float32, torch.float16):
        raise ValueError("dtype must be torch.float32 or torch.float16")
    if ids.device != table.device:
        raise ValueError("ids and the table must be on the same device")
    out = _out(out, (seq, k), dtype, table.device)
    f = lib.qmm_embed if dtype == torch.float32 else lib.qmm_embed_f16
    _call(f(qtype, table.data_ptr(), vocab, k, ids.data_ptr(), seq, out.data_ptr(), _stream_ptr(table.device)),
          "qmm_embed")
    return out


def quantize(x, qtype: int, out=None):
    """Encode x (fp32 or fp16 device tensor [n, k], k a multiple of 32) into
    Q8_0 / Q4_0 blocks: uint8 [n, row_bytes]."""
    torch = _torch()
    if x.dim() == 1:
        x = x.unsqueeze(0)
    if not x.is_cuda or not x.is_contiguous() or x.dim() != 2:
        raise ValueError("x must be a contiguous 2-D device tensor")
    n, k = x.shape
    rb = row_bytes(qtype, k)
    if rb == 0 and k > 0:
        raise ValueError("k=%d is not a multiple of the block size of type %d" % (k, qtype))
    out = _out(out, (n, rb), torch.uint8, x.device)
    if x.dtype == torch.float32:
        f = lib.qmm_quantize
    elif x.dtype == torch.float16:
        f = lib.qmm_quantize_f16
    else:
        raise ValueError("x must be float32 or float16")
    _call(f(qtype, x.data_ptr(), n, k, out.data_ptr(), _stream_ptr(x.device)), "qmm_quantize")
    return out


def gemv(w, qtype: int, n: int, k: int, x, out=None):
    """y[b, j] = sum_i W[j, i] x[b, i]; x fp32 [B, k] (or [k]), 1 <= B <= 8."""
    torch = _torch()
    _check_w(w, qtype, n, k)
    squeeze = x.dim() == 1
    if squeeze:
        x = x.unsqueeze(0)
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous() or x.shape[1] != k:
        raise ValueError("x must be a contiguous fp32 device tensor [B, k]")
    B = x.shape[0]
    if x.device != w.device:
        raise ValueError("x and the weights must be on the same device")
    out = _out(out, (B, n), torch.float32, w.device)
    _call(lib.qmm_gemv(qtype, w.data_ptr(), n, k, x.data_ptr(), B, out.data_ptr(), _stream_ptr(w.device)),
          "qmm_gemv")
    return out[0] if squeeze else out


def gemv_multi(ws, qtype: int, ns, k: int, xs, outs=None):
    """Grouped GEMV: problem i computes W_i x_i (same type, k and batch) in
    as few launches as possible.  Returns the list of outputs."""
    torch = _torch()
    np_ = len(ws)
    if not (len(ns) == len(xs) == np_):
        raise ValueError("ws, ns and xs must have the same length")
    xs = [x.unsqueeze(0) if x.dim() == 1 else x for x in xs]
    B = xs[0].shape[0] if np_ else 0
    for w, n, x in zip(ws, ns, xs):
        _check_w(w, qtype, n, k)
        if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous() or tuple(x.shape) != (B, k):
            raise ValueError("each x must be a contiguous fp32 device tensor [B, k] with the same B")
    if outs is None:
        outs = [None] * np_
    if len(outs) != np_:
        raise ValueError("outs must have one tensor per problem")
    outs = [_out(o, (B, n), torch.float32, w.device) for o, w, n in zip(outs, ws, ns)]
    wp = (ctypes.c_void_p * max(np_, 1))(*[w.data_ptr() for w in ws])
    xp = (ctypes.c_void_p * max(np_, 1))(*[x.data_ptr() for x in xs])
    yp = (ctypes.c_void_p * max(np_, 1))(*[o.data_ptr() for o in outs])
    nn = (ctypes.c_int64 * max(np_, 1))(*ns)
    dev = ws[0].device if np_ else None
    _call(lib.qmm_gemv_multi(qtype, np_, wp, nn, k, xp, B, yp, _stream_ptr(dev) if np_ else None),
          "qmm_gemv_multi")
    return outs


class PassGemv(ctypes.Structure):
    """One GEMV of a decode pass (struct qmm_pass_gemv of include/qmm.h)."""
    _fields_ = [("w", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("n", ctypes.c_int64), ("k", ctypes.c_int64), ("type", ctypes.c_int32), ("stage", ctypes.c_int32)]


def pass_table(problems):
    """ctypes table of a decode pass from (w, qtype, n, k, x, y, stage) tuples
    of device tensors (w uint8, x fp32 of k elements, y fp32 of n)."""
    torch = _torch()
    tab = (PassGemv * max(1, len(problems)))()
    for i, (w, qtype, n, k, x, y, stage) in enumerate(problems):
        _check_w(w, qtype, n, k)
        for t, cnt in ((x, k), (y, n)):
            if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous() or t.numel() != cnt:
                raise ValueError("pass problem %d: x / y must be contiguous fp32 device tensors of k / n elements" % i)
        tab[i] = PassGemv(w.data_ptr(), x.data_ptr(), y.data_ptr(), n, k, qtype, stage)
    return tab


def gemv_pass(problems, table=None, stream=None):
    """Run a decode pass: problems = [(w, qtype, n, k, x, y, stage), ...] in
    nondecreasing stage order; each writes y = W x, and every problem of a
    stage completes before a later stage reads its x."""
    if table is None:
        table = pass_table(problems)
    n = len(problems)
    st = stream if stream is not None else (_stream_ptr(problems[0][0].device) if n else None)
    _call(lib.qmm_gemv_pass(n, ctypes.cast(table, ctypes.c_void_p), st), "qmm_gemv_pass")


def gemm_prefill(w, qtype: int, n: int, k: int, x, out=None):
    """Y[r, j] = sum_i X[r, i] W[j, i]; X fp16 [m, k] -> Y fp32 [m, n]."""
    torch = _torch()
    _check_w(w, qtype, n, k)
    if x.dtype != torch.float16 or not x.is_cuda or not x.is_contiguous() or x.shape[1] != k:
        raise ValueError("X must be a contiguous fp16 device tensor [m, k]")
    m = x.shape[0]
    if x.device != w.device:
        raise ValueError("X and the weights must be on the same device")
    out = _out(out, (m, n), torch.float32, w.device)
    _call(lib.qmm_gemm_prefill(qtype, w.data_ptr(), n, k, x.data_ptr(), m, out.data_ptr(),
                               _stream_ptr(w.device)), "qmm_gemm_prefill")
    return out
