"""Pins for the oracle's Q8_0 / Q4_0 encoder (the KV-cache codec; CPU only).

Checked against things other than the encoder itself: blocks on an exact
grid whose bytes the independent packer (tests/packing.py) writes, rounding
decisions derived by hand, the error bound of a nearest-grid quantizer,
idempotence (encode . decode . encode == encode), sign and power-of-two
symmetries, and the decoder (the separately pinned dequant).
"""
import numpy as np
import pytest

import oracle
import packing as P

RNG = np.random.default_rng(2024)
BB = {P.Q8_0: 34, P.Q4_0: 18}     # bytes per block


def _blocks(q_bytes):
    return np.frombuffer(b"".join(q_bytes), dtype=np.uint8).reshape(len(q_bytes), -1)


def test_q8_0_exact_grid():
    rows, qs = [], []
    for s in range(6):
        q = RNG.integers(-127, 128, 32)
        q[RNG.integers(32)] = 127 if s % 2 else -127        # the block maximum
        rows.append(q * 2.0 ** -3)
        qs.append(P.pack_q8_0(0x3000, q))                   # d = 2^-3
    got = oracle.quantize(P.Q8_0, np.array(rows, np.float32).reshape(2, 96))
    assert np.array_equal(got.reshape(6, 34), _blocks(qs))


@pytest.mark.parametrize("sign", [1, -1])
def test_q4_0_exact_grid(sign):
    rows, qs = [], []
    for _ in range(4):
        q = RNG.integers(1, 16, 32)
        q[RNG.integers(32)] = 0                             # the element of largest magnitude
        rows.append(sign * (q - 8) * 0.25)                  # x = d (q - 8) with d = sign / 4
        qs.append(P.pack_q4_0(0x3400 if sign > 0 else 0xB400, q))
    got = oracle.quantize(P.Q4_0, np.array(rows, np.float32))
    assert np.array_equal(got, _blocks(qs))


def test_q8_0_rounding_by_hand():
    # amax = 127 -> d = 1, 1/d = 1: codes are x rounded half away from zero
    x = np.zeros(32, np.float32)
    x[:9] = [127, 2.5, -2.5, 0.5, -0.5, 1.49, 126.5, -0.49, 3.0]
    b = oracle.quantize(P.Q8_0, x)[0]
    assert b[0] == 0x00 and b[1] == 0x3C                    # fp16 1.0
    assert list(b[2:11].view(np.int8)) == [127, 3, -3, 1, -1, 1, 127, 0, 3]
    assert not b[11:].any()


def test_q4_0_rounding_by_hand():
    # first max -8 -> d = 1, 1/d = 1: code = min(15, trunc(x + 8.5))
    x = np.zeros(32, np.float32)
    x[[0, 1, 2, 3, 4, 5, 6, 7, 16, 17]] = [-8, 6.5, 7, 7.9, -7.5, -7.6, 0.4, 0.6, 8.0, -0.5]
    b = oracle.quantize(P.Q4_0, x)[0]
    assert b[0] == 0x00 and b[1] == 0x3C
    lo, hi = b[2:18] & 15, b[2:18] >> 4
    assert list(lo[:8]) == [0, 15, 15, 15, 1, 0, 8, 9] and list(lo[8:]) == [8] * 8
    assert list(hi[:2]) == [15, 8] and list(hi[2:]) == [8] * 14


def test_q4_0_first_of_equal_magnitudes_sets_the_sign():
    x = np.zeros(32, np.float32)
    x[5], x[20] = 3.0, -3.0
    b = oracle.quantize(P.Q4_0, x)[0]
    # d = 3 / -8 = -0.375 (fp16 0xB600); 1/d = -2.6666667: 3 -> trunc(0.4999999) = 0,
    # -3 -> trunc(16.5000001) = 16 -> 15, zeros -> 8
    assert b[0] == 0x00 and b[1] == 0xB6
    lo, hi = b[2:18] & 15, b[2:18] >> 4
    assert lo[5] == 0 and hi[4] == 15
    assert (np.delete(lo, 5) == 8).all() and (np.delete(hi, 4) == 8).all()
    x[5], x[20] = -3.0, 3.0
    assert oracle.quantize(P.Q4_0, x)[0][1] == 0x36      # d = +0.375


def test_zero_blocks():
    z = np.zeros((1, 32), np.float32)
    assert list(oracle.quantize(P.Q8_0, z)[0]) == [0] * 34
    # Q4_0: d = 0 / -8 = -0 (fp16 0x8000); every code 0 * 0 + 8.5 -> 8
    assert list(oracle.quantize(P.Q4_0, z)[0]) == [0x00, 0x80] + [0x88] * 16


def _inputs():
    r = np.random.default_rng(99)
    # scales stay in the fp16 normal range (d >= 2^-14), where the bound holds
    return [r.standard_normal((64, 256)).astype(np.float32),
            (r.standard_normal((16, 128)) * np.exp(r.uniform(-4, 6, (16, 1)))).astype(np.float32),
            r.integers(-40, 41, (16, 64)).astype(np.float32) / 4]          # many exact ties


@pytest.mark.parametrize("t", [P.Q8_0, P.Q4_0])
def test_decode_error_within_the_grid_bound(t):
    for x in _inputs():
        n, k = x.shape
        b = oracle.quantize(t, x)
        w = oracle.dequant(t, b, n, k).astype(np.float64)
        d16 = np.abs(oracle.half_to_float(b.reshape(-1, BB[t])[:, :2].copy().view(np.uint16).reshape(-1)))
        d16 = np.repeat(d16.astype(np.float64), 32).reshape(n, k)
        # nearest grid point of the fp32 scale (half a step; a full step at the
        # Q4_0 clamp of +8 to code 15), plus the fp16 rounding of the scale
        bound = (0.5 if t == P.Q8_0 else 1.0) * d16 * (1 + 2.0 ** -10) + (127 if t == P.Q8_0 else 8) * 2.0 ** -11 * d16
        assert np.all(np.abs(w - x) <= bound * (1 + 1e-6) + 1e-30)


@pytest.mark.parametrize("t", [P.Q8_0, P.Q4_0])
def test_idempotent(t):
    for x in _inputs():
        n, k = x.shape
        b = oracle.quantize(t, x)
        assert np.array_equal(oracle.quantize(t, oracle.dequant(t, b, n, k)), b)


def test_sign_and_power_of_two_symmetry():
    x = _inputs()[0]
    for t in (P.Q8_0, P.Q4_0):
        b = oracle.quantize(t, x).reshape(-1, BB[t])
        bn = oracle.quantize(t, -x).reshape(-1, BB[t])
        # the scale's fp16 sign bit: Q8_0 keeps it (+), Q4_0 flips it
        assert np.array_equal(bn[:, 0], b[:, 0])
        assert np.array_equal(bn[:, 1], b[:, 1] if t == P.Q8_0 else b[:, 1] ^ 0x80)
        codes, ncodes = b[:, 2:], bn[:, 2:]
        if t == P.Q8_0:
            assert np.array_equal(ncodes.view(np.int8), -codes.view(np.int8))
        else:
            assert np.array_equal(ncodes, codes)
        for s in (-4, 4):
            bs = oracle.quantize(t, x * np.float32(2.0 ** s)).reshape(-1, BB[t])
            assert np.array_equal(bs[:, 2:], codes)
            ds = oracle.half_to_float(bs[:, :2].copy().view(np.uint16).reshape(-1))
            d0 = oracle.half_to_float(b[:, :2].copy().view(np.uint16).reshape(-1))
            assert np.array_equal(ds, d0 * np.float32(2.0 ** s))


def test_f16_input_is_its_exact_value():
    x16 = RNG.standard_normal((8, 64)).astype(np.float16)
    for t in (P.Q8_0, P.Q4_0):
        assert np.array_equal(oracle.quantize(t, x16), oracle.quantize(t, x16.astype(np.float32)))


def test_rejects_other_types_and_shapes():
    with pytest.raises(ValueError):
        oracle.quantize(P.Q4_K, np.zeros((1, 256), np.float32))
    with pytest.raises(ValueError):
        oracle.quantize(P.Q8_0, np.zeros((1, 48), np.float32))
