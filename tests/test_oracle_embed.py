"""Pins for the oracle's fp16 rounding and embedding gather (CPU only).

fp16 rounding is checked against numpy's float32 -> float16 conversion (a
library routine that rounds to nearest-even) on every exponent with the
mantissa patterns that decide a rounding (exact, just below, at and just
above a tie), on the ties of the subnormal range, and on random bit
patterns, plus hand-derived values.  The gather is checked against the
separately pinned dequant, against a table whose rows decode to a closed
form, and for its invalid-id rule.
"""
import numpy as np
import pytest

import oracle
import packing as P
import qmm_inputs as I

TYPES = [P.Q4_0, P.Q8_0, P.Q4_K, P.Q6_K, P.Q5_0, P.Q5_K]


def _assert_half_bits_equal(got, ref):
    ref = np.asarray(ref, dtype=np.uint16)
    nan_ref = np.isnan(ref.view(np.float16))
    nan_got = np.isnan(got.view(np.float16))
    assert np.array_equal(nan_got, nan_ref)
    bad = np.nonzero(got[~nan_ref] != ref[~nan_ref])[0]
    assert bad.size == 0, [(hex(int(g)), hex(int(r))) for g, r in zip(got[~nan_ref][bad[:5]], ref[~nan_ref][bad[:5]])]


def test_half_rounding_matches_numpy_on_decision_patterns():
    rng = np.random.default_rng(7)
    hi = np.concatenate([[0, 1, 2, 0x1ff, 0x200, 0x3fe, 0x3ff], rng.integers(0, 1024, 16)]).astype(np.uint32)
    lo = np.array([0, 1, 0xfff, 0x1000, 0x1001, 0x1fff, int(rng.integers(0, 0x2000))], dtype=np.uint32)
    s, e, h, l = np.meshgrid(np.array([0, 1], np.uint32), np.arange(256, dtype=np.uint32), hi, lo, indexing="ij")
    bits = (s << 31) | (e << 23) | (h << 13) | l
    x = bits.reshape(-1).view(np.float32)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    _assert_half_bits_equal(oracle.to_half_bits(x), ref)


def test_half_rounding_matches_numpy_on_random_patterns():
    x = np.random.default_rng(8).integers(0, 2 ** 32, 1 << 21, dtype=np.uint64).astype(np.uint32).view(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    _assert_half_bits_equal(oracle.to_half_bits(x), ref)


def test_half_rounding_subnormal_ties_go_to_even():
    m = np.arange(1024, dtype=np.float64)
    tie = ((m + 0.5) * 2.0 ** -24).astype(np.float32)     # exact in fp32
    even = np.where(m % 2 == 0, m, m + 1).astype(np.uint16)
    assert np.array_equal(oracle.to_half_bits(tie), even)
    above = np.nextafter(tie, np.float32(1))
    below = np.nextafter(tie, np.float32(0))
    assert np.array_equal(oracle.to_half_bits(above), (m + 1).astype(np.uint16))
    assert np.array_equal(oracle.to_half_bits(below), m.astype(np.uint16))
    assert np.array_equal(oracle.to_half_bits(-tie), even | 0x8000)


def test_half_rounding_hand_values():
    # expected bit patterns derived by hand from the binary16 definition
    cases = [
        (1.0, 0x3C00), (-2.0, 0xC000), (0.0, 0x0000), (-0.0, 0x8000),
        (65504.0, 0x7BFF),                 # largest finite
        (65519.99, 0x7BFF),                # below the tie between 65504 and 65536
        (65520.0, 0x7C00),                 # the tie rounds to the even pattern: Inf
        (1e6, 0x7C00), (-1e6, 0xFC00),
        (2.0 ** -24, 0x0001),              # smallest subnormal
        (2.0 ** -25, 0x0000),              # tie between 0 and 2^-24 -> 0 (even)
        (1.5 * 2.0 ** -25, 0x0001),
        (2.0 ** -14, 0x0400),              # smallest normal
        (2.0 ** -14 - 2.0 ** -25, 0x0400), # tie between 1023 and 1024 quanta -> 1024
        (1.0 + 2.0 ** -11, 0x3C00),        # tie -> even fraction 0
        (1.0 + 3 * 2.0 ** -11, 0x3C02),    # tie -> even fraction 2
        (2047.0, 0x67FF), (2049.0, 0x6800),  # 2049 is a tie between 2048 and 2050
        (float("inf"), 0x7C00), (float("-inf"), 0xFC00),
    ]
    for v, bits in cases:
        assert oracle.double_to_half_bits(v) == bits, (v, hex(oracle.double_to_half_bits(v)), hex(bits))
    assert oracle.double_to_half_bits(float("nan")) & 0x7FFF > 0x7C00


# --- embedding gather (dotLLM "GPU Inference", Forward Pass step 2) ----------

@pytest.mark.parametrize("t", TYPES)
def test_embed_rows_are_dequant_rows(t):
    vocab, k = 37, 2 * I.BLOCK_ELEMS[t]
    table = I.gen_weights(t, vocab, k, seed=40 + t)
    ids = np.array([5, 0, 36, 5, 17, 36, 1, 2, 3, 29, 0], dtype=np.int32)
    got = oracle.embed(t, table, vocab, k, ids)
    ref = oracle.dequant(t, table, vocab, k)[ids]
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # the fp16 output is numpy's nearest-even rounding of the same values
    assert np.array_equal(oracle.embed(t, table, vocab, k, ids, f16=True), ref.astype(np.float16).view(np.uint16))


def test_embed_closed_form_rows():
    # row r of a Q8_0 table: d = 1, code i = ((r + i) mod 255) - 127
    vocab, k = 300, 64
    rows = []
    for r in range(vocab):
        q = [((r + i) % 255) - 127 for i in range(k)]
        rows.append(P.pack_q8_0(0x3C00, q[:32]) + P.pack_q8_0(0x3C00, q[32:]))
    table = np.frombuffer(b"".join(rows), dtype=np.uint8)
    ids = np.array([299, 0, 1, 254, 255, 128, 7, 7], dtype=np.int32)
    got = oracle.embed(P.Q8_0, table, vocab, k, ids)
    want = (ids[:, None] + np.arange(k)[None, :]) % 255 - 127
    assert np.array_equal(got, want.astype(np.float32))


def test_embed_invalid_ids_give_zero_rows():
    t, vocab, k = P.Q4_K, 9, 256
    table = I.gen_weights(t, vocab, k, seed=77)
    ids = np.array([-1, vocab, vocab + 100, -2 ** 31, 2 ** 31 - 1, 0, 8], dtype=np.int32)
    got = oracle.embed(t, table, vocab, k, ids)
    assert np.array_equal(got[:5].view(np.uint32), np.zeros((5, k), np.uint32))   # +0.0, not -0.0
    ref = oracle.dequant(t, table, vocab, k)
    assert np.array_equal(got[5], ref[0]) and np.array_equal(got[6], ref[8])
    # an empty table: every id is invalid
    assert np.array_equal(oracle.embed(t, np.zeros(0, np.uint8), 0, k, [0, 3]), np.zeros((2, k), np.float32))


def test_embed_empty_and_bad_shapes():
    table = I.gen_weights(P.Q8_0, 4, 32, seed=1)
    assert oracle.embed(P.Q8_0, table, 4, 32, np.zeros(0, np.int32)).shape == (0, 32)
    with pytest.raises(ValueError):
        oracle.embed(P.Q8_0, table, 4, 48, [0])
    with pytest.raises(ValueError):
        oracle.embed(9, table, 4, 32, [0])
