"""Pins for the oracle's block decoders (CPU only).

Each test checks the oracle against something other than itself: a library
routine (numpy's binary16 conversion), hand-built blocks with closed-form
values (tests/golden), a bit-level statement of the Q4_K packing rule,
one-hot code placement, an independent encoder (tests/packing.py), and
quantize -> dequantize error bounds.
"""
import numpy as np
import pytest

import oracle
import packing as P
from golden_io import load

TYPES = [P.Q4_0, P.Q8_0, P.Q4_K, P.Q6_K, P.Q5_0, P.Q5_K]


# --- fp16 unpack (shimmy "Architecture", Quantization table: fp16 unpack) ---

def test_fp16_exhaustive_matches_numpy():
    h = np.arange(65536, dtype=np.uint16)
    got = oracle.half_to_float(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_fp16_special_values():
    cases = {0x0000: 0.0, 0x8000: -0.0, 0x0001: 2.0 ** -24, 0x03FF: 1023 * 2.0 ** -24,
             0x0400: 2.0 ** -14, 0x3C00: 1.0, 0xC000: -2.0, 0x7BFF: 65504.0,
             0x7C00: np.inf, 0xFC00: -np.inf, 0x3555: 0.333251953125}
    got = oracle.half_to_float(np.array(list(cases), dtype=np.uint16))
    for g, (h, v) in zip(got, cases.items()):
        assert g == v and np.signbit(g) == np.signbit(v), hex(h)
    assert np.isnan(oracle.half_to_float(np.array([0x7E00, 0xFD01], dtype=np.uint16))).all()


# --- sizes (dotLLM "GPU Inference", Weight Strategy: Q4_K ~4.5 bits/param) ---

def test_block_sizes_and_bits_per_weight():
    assert [oracle.block_elems(t) for t in TYPES] == [32, 32, 256, 256, 32, 256]
    assert [oracle.block_bytes(t) for t in TYPES] == [18, 34, 144, 210, 22, 176]
    assert oracle.block_bytes(P.Q5_K) * 8 / 256 == 5.5
    assert oracle.block_bytes(P.Q4_K) * 8 / 256 == 4.5
    assert oracle.row_bytes(P.Q4_K, 4096) == 2304
    assert oracle.row_bytes(P.Q6_K, 14336) == 11760
    assert oracle.row_bytes(P.Q8_0, 33) == 0          # not a block multiple
    assert oracle.block_elems(7) == 0


# --- hand-built goldens ------------------------------------------------------

def _signed_zero_equal(a, b):
    return np.array_equal(np.asarray(a, np.float64), np.asarray(b, np.float64))


@pytest.mark.parametrize("fname", ["q8_0.txt", "q4_0.txt", "q5_0.txt"])
def test_golden_simple_blocks(fname):
    for blk in load(fname):
        t = blk["type"]
        w = np.frombuffer(blk["bytes"], dtype=np.uint8)
        got = oracle.dequant(t, w, 1, 32)[0]
        assert _signed_zero_equal(got, blk["expect"]), blk["name"]
        y, a = oracle.gemv(t, w, 1, 32, np.ones(32, np.float32))
        assert y[0, 0] == blk["rowsum"], blk["name"]


def test_golden_q4_k():
    for blk in load("q4_k.txt"):
        w = np.frombuffer(blk["bytes"], dtype=np.uint8)
        got = oracle.dequant(P.Q4_K, w, 1, 256)[0]
        for e, v in blk["spot"].items():
            assert got[e] == v, (blk["name"], e)
        # scale/min fields as packed by hand
        for j in range(8):
            assert oracle.q4k_scale_min(blk["bytes"][4:16], j) == (blk["sc"][j], blk["m"][j])
        # every element from the closed form d*sc*q - dmin*m, d = 1, dmin = 0.5,
        # q = l % 16 for even sub-blocks and 15 - l % 16 for odd ones
        e = np.arange(256)
        j, l = e // 32, e % 32
        q = np.where(j % 2 == 0, l % 16, 15 - l % 16)
        exp = np.array(blk["sc"])[j] * q - 0.5 * np.array(blk["m"])[j]
        assert np.array_equal(got, exp.astype(np.float32)), blk["name"]


def test_golden_q5_k():
    for blk in load("q5_k.txt"):
        w = np.frombuffer(blk["bytes"], dtype=np.uint8)
        got = oracle.dequant(P.Q5_K, w, 1, 256)[0]
        for e, v in blk["spot"].items():
            assert got[e] == v, (blk["name"], e)
        for j in range(8):
            assert oracle.q4k_scale_min(blk["bytes"][4:16], j) == (blk["sc"][j], blk["m"][j])
    # block A element by element: q = l % 16 (even j), 31 - l % 16 (odd j)
    blk = load("q5_k.txt")[0]
    got = oracle.dequant(P.Q5_K, np.frombuffer(blk["bytes"], dtype=np.uint8), 1, 256)[0]
    e = np.arange(256)
    j, l = e // 32, e % 32
    q = np.where(j % 2 == 0, l % 16, 31 - l % 16)
    exp = np.array(blk["sc"])[j] * q - 0.5 * np.array(blk["m"])[j]
    assert np.array_equal(got, exp.astype(np.float32))


def test_golden_q6_k():
    for blk in load("q6_k.txt"):
        w = np.frombuffer(blk["bytes"], dtype=np.uint8)
        got = oracle.dequant(P.Q6_K, w, 1, 256)[0]
        for e, v in blk["spot"].items():
            assert got[e] == v, (blk["name"], e)
        e = np.arange(256)
        if "q_const" in blk:
            q = np.full(256, blk["q_const"])
        elif "q_by_g" in blk:
            q = np.array(blk["q_by_g"])[(e % 128) // 32]
        else:
            q = np.array(blk["q_by_h"])[e // 128]
        exp = (e // 16 - 8) * (q - 32)
        assert _signed_zero_equal(got, exp), blk["name"]


# --- Q4_K scale packing, stated bit by bit ----------------------------------
# The rule given with the Q4_K workload says where every bit of the 12 scale
# bytes goes.  Written as a table: bit b of byte i -> (field, index, bit).

def _q4k_bit_table():
    tab = {}
    for i in range(4):
        for b in range(6):
            tab[(i, b)] = ("sc", i, b)            # low 6 bits of bytes 0-3: sc0-3
            tab[(i + 4, b)] = ("m", i, b)          # low 6 bits of bytes 4-7: m0-3
        for b in (6, 7):
            tab[(i, b)] = ("sc", i + 4, b - 2)    # top 2 bits of bytes 0-3: sc4-7 bits 4,5
            tab[(i + 4, b)] = ("m", i + 4, b - 2)  # top 2 bits of bytes 4-7: m4-7 bits 4,5
        for b in range(4):
            tab[(i + 8, b)] = ("sc", i + 4, b)    # low nibble of bytes 8-11: sc4-7 bits 0-3
            tab[(i + 8, b + 4)] = ("m", i + 4, b)  # high nibble: m4-7 bits 0-3
    return tab


def test_q4k_scale_packing_one_hot_bits():
    tab = _q4k_bit_table()
    assert len(tab) == 96
    for (i, b), (field, j, bit) in tab.items():
        s = bytearray(12)
        s[i] = 1 << b
        for jj in range(8):
            sc, m = oracle.q4k_scale_min(bytes(s), jj)
            want_sc = (1 << bit) if (field == "sc" and jj == j) else 0
            want_m = (1 << bit) if (field == "m" and jj == j) else 0
            assert (sc, m) == (want_sc, want_m), (i, b, jj)


def test_q4k_scale_packing_bijection_random():
    rng = np.random.default_rng(7)
    for _ in range(300):
        sc = rng.integers(0, 64, 8)
        m = rng.integers(0, 64, 8)
        s = P.pack_q4k_scales(sc, m)
        assert [oracle.q4k_scale_min(s, j) for j in range(8)] == list(zip(sc, m))
    for _ in range(300):
        s = rng.integers(0, 256, 12, dtype=np.uint8).tobytes()
        fields = [oracle.q4k_scale_min(s, j) for j in range(8)]
        assert P.pack_q4k_scales([f[0] for f in fields], [f[1] for f in fields]) == s


# --- one-hot code placement ------------------------------------------------

def test_q8_0_one_hot_codes():
    for e in range(32):
        q = np.zeros(32, np.int64)
        q[e] = 3
        w = oracle.dequant(P.Q8_0, np.frombuffer(P.pack_q8_0(0x3C00, q), np.uint8), 1, 32)[0]
        assert np.array_equal(w, 3.0 * (np.arange(32) == e))


def test_q4_0_one_hot_codes():
    for e in range(32):
        q = np.full(32, 8, np.int64)   # code 8 -> weight 0
        q[e] = 13
        w = oracle.dequant(P.Q4_0, np.frombuffer(P.pack_q4_0(0x3C00, q), np.uint8), 1, 32)[0]
        assert np.array_equal(w, 5.0 * (np.arange(32) == e)), e


def test_q4_k_one_hot_codes():
    sc = [1] * 8
    m = [0] * 8
    for e in range(256):
        q = np.zeros(256, np.int64)
        q[e] = 9
        blk = P.pack_q4_k(0x3C00, 0x3C00, sc, m, q)
        w = oracle.dequant(P.Q4_K, np.frombuffer(blk, np.uint8), 1, 256)[0]
        assert np.array_equal(w, 9.0 * (np.arange(256) == e)), e
    # and one-hot bits in the raw code bytes land on exactly one element
    for byte in range(128):
        for nib in (0, 1):
            raw = bytearray(P.pack_q4_k(0x3C00, 0x3C00, sc, m, np.zeros(256, np.int64)))
            raw[16 + byte] = 1 << (4 * nib)
            w = oracle.dequant(P.Q4_K, np.frombuffer(bytes(raw), np.uint8), 1, 256)[0]
            nz = np.flatnonzero(w)
            assert nz.tolist() == [32 * (2 * (byte // 32) + nib) + byte % 32]


def test_q6_k_one_hot_codes():
    sc = np.ones(16, np.int64)
    base = np.full(256, 32, np.int64)   # code 32 -> weight 0
    for e in range(256):
        q = base.copy()
        q[e] = 32 + 17
        w = oracle.dequant(P.Q6_K, np.frombuffer(P.pack_q6_k(0x3C00, sc, q), np.uint8), 1, 256)[0]
        assert np.array_equal(w, 17.0 * (np.arange(256) == e)), e
    # every scale byte affects exactly its 16 elements
    for i in range(16):
        s = np.zeros(16, np.int64)
        s[i] = 5
        w = oracle.dequant(P.Q6_K, np.frombuffer(P.pack_q6_k(0x3C00, s, np.full(256, 33)), np.uint8), 1, 256)[0]
        assert np.array_equal(w, 5.0 * (np.arange(256) // 16 == i))


def test_q5_0_one_hot_codes_and_bits():
    for e in range(32):
        q = np.full(32, 16, np.int64)   # code 16 -> weight 0
        q[e] = 16 + 11 if e % 2 else 16 - 13   # both sides of the offset, high bit set / clear
        w = oracle.dequant(P.Q5_0, np.frombuffer(P.pack_q5_0(0x3C00, q), np.uint8), 1, 32)[0]
        assert np.array_equal(w, (11.0 if e % 2 else -13.0) * (np.arange(32) == e)), e
    # one-hot bits of the high-bit word move exactly one element by 16 d
    for bit in range(32):
        raw = bytearray(P.pack_q5_0(0x3C00, np.zeros(32, np.int64)))
        raw[2 + bit // 8] |= 1 << (bit % 8)
        w = oracle.dequant(P.Q5_0, np.frombuffer(bytes(raw), np.uint8), 1, 32)[0]
        assert np.array_equal(w, -16.0 + 16.0 * (np.arange(32) == bit)), bit


def test_q5_k_one_hot_codes_and_bits():
    sc = [1] * 8
    m = [0] * 8
    for e in range(0, 256, 3):
        q = np.zeros(256, np.int64)
        q[e] = 19          # low nibble 3, high bit set
        blk = P.pack_q5_k(0x3C00, 0x3C00, sc, m, q)
        w = oracle.dequant(P.Q5_K, np.frombuffer(blk, np.uint8), 1, 256)[0]
        assert np.array_equal(w, 19.0 * (np.arange(256) == e)), e
    # one-hot bits of the 32 qh bytes land on exactly one element (j = bit, l = byte)
    for byte in range(32):
        for bit in range(8):
            raw = bytearray(P.pack_q5_k(0x3C00, 0x3C00, sc, m, np.zeros(256, np.int64)))
            raw[16 + byte] = 1 << bit
            w = oracle.dequant(P.Q5_K, np.frombuffer(bytes(raw), np.uint8), 1, 256)[0]
            assert np.flatnonzero(w).tolist() == [32 * bit + byte] and w.max() == 16.0


# --- independent encoder vs decoder ----------------------------------------

@pytest.mark.parametrize("t", TYPES)
def test_encode_with_own_scales_round_trip(t):
    """Random blocks: read their fields with the test-side parser, re-encode
    them with the test-side packer -> identical bytes; and the oracle's value
    of every element equals the one implied by the parsed fields."""
    import qmm_inputs
    w = qmm_inputs.gen_weights(t, 4, 2 * P.BE[t], seed=11)
    vals = oracle.dequant_f64(t, w, 4, 2 * P.BE[t])
    raw = w.reshape(-1)
    for b in range(raw.size // P.BB[t]):
        blk = raw[b * P.BB[t]:(b + 1) * P.BB[t]].tobytes()
        f = P.read_fields(t, blk)
        h = lambda u: float(np.array(u, np.uint16).view(np.float16))
        if t == P.Q8_0:
            again = P.pack_q8_0(f["d"], f["q"])
            imp = h(f["d"]) * f["q"]
        elif t == P.Q4_0:
            again = P.pack_q4_0(f["d"], f["q"])
            imp = h(f["d"]) * (f["q"] - 8)
        elif t in (P.Q4_K, P.Q5_K):
            pack = P.pack_q4_k if t == P.Q4_K else P.pack_q5_k
            again = pack(f["d"], f["dmin"], f["sc"], f["m"], f["q"])
            j = np.arange(256) // 32
            imp = h(f["d"]) * f["sc"][j] * f["q"] - h(f["dmin"]) * f["m"][j]
        elif t == P.Q5_0:
            again = P.pack_q5_0(f["d"], f["q"])
            imp = h(f["d"]) * (f["q"] - 16)
        else:
            again = P.pack_q6_k(f["d"], f["sc"], f["q"])
            imp = h(f["d"]) * f["sc"][np.arange(256) // 16] * (f["q"] - 32)
        assert again == blk
        row, off = divmod(b, 2)
        got = vals[row, off * P.BE[t]:(off + 1) * P.BE[t]]
        assert np.array_equal(got, imp)


# --- quantize -> dequantize error bound --------------------------------------

@pytest.mark.parametrize("t", TYPES)
def test_quantize_dequantize_half_step(t):
    rng = np.random.default_rng(100 + t)
    for trial in range(20):
        scale = 10.0 ** rng.uniform(-3, 1)
        w = rng.standard_normal(P.BE[t]) * scale
        if trial % 4 == 1:
            w = np.abs(w)            # all positive (Q4_K: zero min offset)
        if trial % 4 == 2:
            w[rng.integers(0, w.size)] *= 20   # outlier
        blk, step = P.QUANT[t](w)
        got = oracle.dequant_f64(t, np.frombuffer(blk, np.uint8), 1, P.BE[t])[0]
        err = np.abs(got - w)
        assert np.all(err <= 0.5 * step * (1 + 1e-12) + 1e-12), (t, trial, (err / step).max())
        # fp32 path rounds the exact value once
        got32 = oracle.dequant(t, np.frombuffer(blk, np.uint8), 1, P.BE[t])[0]
        assert np.array_equal(got32, got.astype(np.float32))


def test_dequant_rejects_bad_shapes():
    w = np.zeros(34, np.uint8)
    with pytest.raises(ValueError):
        oracle.dequant(P.Q8_0, w, 1, 33)
    with pytest.raises(ValueError):
        oracle.dequant(9, w, 1, 32)
