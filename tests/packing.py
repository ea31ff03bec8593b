"""Test-side block *encoders* and simple quantizers (pure Python / numpy).

This is a third, independent implementation of each block layout, written in
the encoding direction, so that the oracle's decoders (C) can be checked
against it.  It shares nothing with the oracle or with the HIP library.

Layouts (workload definitions that accompany the pages; see the oracle's
header for the page citations):
  Q8_0: fp16 d | 32 int8 q                         w = d q
  Q4_0: fp16 d | 16 B; element i<16 low nibble of byte i, i>=16 high nibble of
        byte i-16                                   w = d (q - 8)
  Q4_K: fp16 d | fp16 dmin | 12 B scales | 128 B codes
        w = d sc_j q - dmin m_j, sub-block j = e // 32; code of element
        (j, l) in byte 32 (j // 2) + l, low nibble for even j (reading R5)
  Q6_K: 128 B ql | 64 B qh | 16 int8 sc | fp16 d     w = d sc[e // 16] (q - 32)
        element e: h = e // 128, r = e % 128, g = r // 32, l = r % 32;
        low 4 bits in ql[64 h + 32 (g % 2) + l] (low nibble if g < 2),
        high 2 bits at bit 2g of qh[32 h + l] (reading R8)
  Q5_0: fp16 d | 4 B high bits | 16 B nibbles as Q4_0; bit 4 of element i is
        bit i of the little-endian word              w = d (q - 16)
  Q5_K: fp16 d | fp16 dmin | 12 B scales | 32 B qh | 128 B codes as Q4_K;
        bit 4 of element (j, l) is bit j of qh[l]    w = d sc_j q - dmin m_j
        (both 5-bit layouts: GGUF convention, a reading; parity unpinned)
"""
from __future__ import annotations

import numpy as np

Q4_0, Q8_0, Q4_K, Q6_K, Q5_0, Q5_K = 0, 1, 2, 3, 4, 5
BE = {Q4_0: 32, Q8_0: 32, Q4_K: 256, Q6_K: 256, Q5_0: 32, Q5_K: 256}
BB = {Q4_0: 18, Q8_0: 34, Q4_K: 144, Q6_K: 210, Q5_0: 22, Q5_K: 176}


def f16(v) -> np.uint16:
    return np.array(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def _h(u16) -> bytes:
    return int(u16).to_bytes(2, "little")


def pack_q8_0(d16: int, q) -> bytes:
    q = np.asarray(q, dtype=np.int64)
    assert q.shape == (32,) and q.min() >= -128 and q.max() <= 127
    return _h(d16) + bytes(int(v) & 0xFF for v in q)


def pack_q4_0(d16: int, q) -> bytes:
    q = np.asarray(q, dtype=np.int64)
    assert q.shape == (32,) and q.min() >= 0 and q.max() <= 15
    return _h(d16) + bytes(int(q[i]) | (int(q[i + 16]) << 4) for i in range(16))


def pack_q4k_scales(sc, m) -> bytes:
    """8 six-bit scales and 8 six-bit mins -> 12 bytes (the packing rule given
    with the Q4_K workload, written in the encoding direction)."""
    sc = [int(v) for v in sc]
    m = [int(v) for v in m]
    assert all(0 <= v < 64 for v in sc + m)
    s = [0] * 12
    for j in range(4):
        s[j] = (sc[j] & 63) | ((sc[j + 4] >> 4) << 6)
        s[j + 4] = (m[j] & 63) | ((m[j + 4] >> 4) << 6)
        s[j + 8] = (sc[j + 4] & 15) | ((m[j + 4] & 15) << 4)
    return bytes(s)


def pack_q4_k(d16: int, dmin16: int, sc, m, q) -> bytes:
    q = np.asarray(q, dtype=np.int64)
    assert q.shape == (256,) and q.min() >= 0 and q.max() <= 15
    qs = bytearray(128)
    for j in range(8):
        for l in range(32):
            byte = 32 * (j // 2) + l
            if j % 2 == 0:
                qs[byte] |= int(q[32 * j + l])
            else:
                qs[byte] |= int(q[32 * j + l]) << 4
    return _h(d16) + _h(dmin16) + pack_q4k_scales(sc, m) + bytes(qs)


def pack_q6_k(d16: int, sc, q) -> bytes:
    q = np.asarray(q, dtype=np.int64)
    sc = np.asarray(sc, dtype=np.int64)
    assert q.shape == (256,) and q.min() >= 0 and q.max() <= 63
    assert sc.shape == (16,) and sc.min() >= -128 and sc.max() <= 127
    ql = bytearray(128)
    qh = bytearray(64)
    for e in range(256):
        h, r = divmod(e, 128)
        g, l = divmod(r, 32)
        lo, hi = int(q[e]) & 15, int(q[e]) >> 4
        ql[64 * h + 32 * (g % 2) + l] |= lo if g < 2 else (lo << 4)
        qh[32 * h + l] |= hi << (2 * g)
    return bytes(ql) + bytes(qh) + bytes(int(v) & 0xFF for v in sc) + _h(d16)


def pack_q5_0(d16: int, q) -> bytes:
    q = np.asarray(q, dtype=np.int64)
    assert q.shape == (32,) and q.min() >= 0 and q.max() <= 31
    hbits = sum((int(q[i]) >> 4) << i for i in range(32))
    lo = [int(v) & 15 for v in q]
    return _h(d16) + hbits.to_bytes(4, "little") + bytes(lo[i] | (lo[i + 16] << 4) for i in range(16))


def pack_q5_k(d16: int, dmin16: int, sc, m, q) -> bytes:
    q = np.asarray(q, dtype=np.int64)
    assert q.shape == (256,) and q.min() >= 0 and q.max() <= 31
    qh = bytearray(32)
    qs = bytearray(128)
    for j in range(8):
        for l in range(32):
            v = int(q[32 * j + l])
            qh[l] |= (v >> 4) << j
            byte = 32 * (j // 2) + l
            qs[byte] |= (v & 15) if j % 2 == 0 else ((v & 15) << 4)
    return _h(d16) + _h(dmin16) + pack_q4k_scales(sc, m) + bytes(qh) + bytes(qs)


# ---------------------------------------------------------------- readers ---

def read_fields(t: int, blk: bytes) -> dict:
    """Parse one block's fields (no arithmetic beyond bit extraction)."""
    b = np.frombuffer(blk, dtype=np.uint8)
    if t == Q8_0:
        return {"d": int(b[0]) | int(b[1]) << 8, "q": b[2:34].view(np.int8).astype(np.int64)}
    if t == Q4_0:
        qs = b[2:18].astype(np.int64)
        return {"d": int(b[0]) | int(b[1]) << 8, "q": np.concatenate([qs & 15, qs >> 4])}
    if t == Q4_K:
        s = b[4:16].astype(np.int64)
        sc = [0] * 8
        m = [0] * 8
        for j in range(4):
            sc[j] = s[j] & 63
            m[j] = s[j + 4] & 63
            sc[j + 4] = (s[j + 8] & 15) | ((s[j] >> 6) << 4)
            m[j + 4] = (s[j + 8] >> 4) | ((s[j + 4] >> 6) << 4)
        qs = b[16:144].astype(np.int64)
        q = np.zeros(256, dtype=np.int64)
        for j in range(8):
            grp = qs[32 * (j // 2): 32 * (j // 2) + 32]
            q[32 * j: 32 * j + 32] = (grp & 15) if j % 2 == 0 else (grp >> 4)
        return {"d": int(b[0]) | int(b[1]) << 8, "dmin": int(b[2]) | int(b[3]) << 8,
                "sc": np.array(sc), "m": np.array(m), "q": q}
    if t == Q6_K:
        ql = b[0:128].astype(np.int64)
        qh = b[128:192].astype(np.int64)
        q = np.zeros(256, dtype=np.int64)
        for e in range(256):
            h, r = divmod(e, 128)
            g, l = divmod(r, 32)
            lb = ql[64 * h + 32 * (g % 2) + l]
            lo = (lb & 15) if g < 2 else (lb >> 4)
            q[e] = lo | (((qh[32 * h + l] >> (2 * g)) & 3) << 4)
        return {"d": int(b[208]) | int(b[209]) << 8, "sc": b[192:208].view(np.int8).astype(np.int64), "q": q}
    if t == Q5_0:
        hb = int.from_bytes(bytes(b[2:6]), "little")
        qs = b[6:22].astype(np.int64)
        lo = np.concatenate([qs & 15, qs >> 4])
        hi = np.array([(hb >> i) & 1 for i in range(32)], dtype=np.int64)
        return {"d": int(b[0]) | int(b[1]) << 8, "q": lo | (hi << 4)}
    if t == Q5_K:
        f = read_fields(Q4_K, bytes(b[0:16]) + bytes(b[48:176]))
        qh = b[16:48].astype(np.int64)
        for j in range(8):
            f["q"][32 * j: 32 * j + 32] |= ((qh >> j) & 1) << 4
        return f
    raise ValueError(t)


# ------------------------------------------------------------ quantizers ---
# Simple reference quantizers (ours, not GGUF's).  Each guarantees that every
# element's code lies inside the representable range, so the reconstruction
# error is at most half a quantization step of the decoded scale.

def _f16_up(v: float) -> int:
    """Smallest fp16 >= v (v > 0), as bits."""
    h = np.float16(v)
    if float(h) < v:
        h = np.nextafter(h, np.float16(np.inf))
    return int(np.array(h, dtype=np.float16).view(np.uint16))


def _hval(u16: int) -> float:
    return float(np.array(u16, dtype=np.uint16).view(np.float16))


def quant_q8_0(w) -> tuple[bytes, np.ndarray]:
    """Returns (block, step) with step = d (error bound is step / 2)."""
    w = np.asarray(w, dtype=np.float64)
    d16 = _f16_up(max(np.abs(w).max(), 1e-4) / 127.0)
    d = _hval(d16)
    q = np.clip(np.rint(w / d), -127, 127).astype(np.int64)
    return pack_q8_0(d16, q), np.full(32, d)


def quant_q4_0(w) -> tuple[bytes, np.ndarray]:
    w = np.asarray(w, dtype=np.float64)
    d16 = _f16_up(max(np.abs(w).max(), 1e-4) / 7.0)
    d = _hval(d16)
    q = np.clip(np.rint(w / d) + 8, 0, 15).astype(np.int64)
    return pack_q4_0(d16, q), np.full(32, d)


def quant_q4_k(w) -> tuple[bytes, np.ndarray]:
    w = np.asarray(w, dtype=np.float64).reshape(8, 32)
    mn = np.minimum(w.min(axis=1), 0.0)
    mx = w.max(axis=1)
    off = -mn                                   # >= 0
    dmin16 = _f16_up(max(off.max(), 1e-4) / 63.0)
    dmin = _hval(dmin16)
    m = np.minimum(np.ceil(off / dmin), 63).astype(np.int64)  # dmin m >= off
    span = (mx - mn) + dmin                      # range to cover after the shift
    d16 = _f16_up(max(span.max(), 1e-4) / (15.0 * 63.0))
    d = _hval(d16)
    sc = np.clip(np.ceil(span / (15.0 * d)), 1, 63).astype(np.int64)
    q = np.zeros((8, 32), dtype=np.int64)
    step = np.zeros((8, 32))
    for j in range(8):
        q[j] = np.clip(np.rint((w[j] + dmin * m[j]) / (d * sc[j])), 0, 15)
        step[j] = d * sc[j]
    return pack_q4_k(d16, dmin16, sc, m, q.reshape(-1)), step.reshape(-1)


def quant_q6_k(w) -> tuple[bytes, np.ndarray]:
    w = np.asarray(w, dtype=np.float64).reshape(16, 16)
    amax = np.maximum(np.abs(w).max(axis=1), 1e-6)
    d16 = _f16_up(amax.max() / (31.0 * 127.0))
    d = _hval(d16)
    sc = np.clip(np.ceil(amax / (31.0 * d)), 1, 127).astype(np.int64)
    q = np.zeros((16, 16), dtype=np.int64)
    step = np.zeros((16, 16))
    for i in range(16):
        q[i] = np.clip(np.rint(w[i] / (d * sc[i])) + 32, 0, 63)
        step[i] = d * sc[i]
    return pack_q6_k(d16, sc, q.reshape(-1)), step.reshape(-1)


def quant_q5_0(w) -> tuple[bytes, np.ndarray]:
    w = np.asarray(w, dtype=np.float64)
    d16 = _f16_up(max(np.abs(w).max(), 1e-4) / 15.0)
    d = _hval(d16)
    q = np.clip(np.rint(w / d) + 16, 0, 31).astype(np.int64)
    return pack_q5_0(d16, q), np.full(32, d)


def quant_q5_k(w) -> tuple[bytes, np.ndarray]:
    w = np.asarray(w, dtype=np.float64).reshape(8, 32)
    mn = np.minimum(w.min(axis=1), 0.0)
    mx = w.max(axis=1)
    off = -mn
    dmin16 = _f16_up(max(off.max(), 1e-4) / 63.0)
    dmin = _hval(dmin16)
    m = np.minimum(np.ceil(off / dmin), 63).astype(np.int64)
    span = (mx - mn) + dmin
    d16 = _f16_up(max(span.max(), 1e-4) / (31.0 * 63.0))
    d = _hval(d16)
    sc = np.clip(np.ceil(span / (31.0 * d)), 1, 63).astype(np.int64)
    q = np.zeros((8, 32), dtype=np.int64)
    step = np.zeros((8, 32))
    for j in range(8):
        q[j] = np.clip(np.rint((w[j] + dmin * m[j]) / (d * sc[j])), 0, 31)
        step[j] = d * sc[j]
    return pack_q5_k(d16, dmin16, sc, m, q.reshape(-1)), step.reshape(-1)


QUANT = {Q8_0: quant_q8_0, Q4_0: quant_q4_0, Q4_K: quant_q4_k, Q6_K: quant_q6_k,
         Q5_0: quant_q5_0, Q5_K: quant_q5_k}
