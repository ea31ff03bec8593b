"""Weight matrices with exactly-zero weights, built with the independent
encoder (tests/packing.py), for the parity cases where the products cancel:

  Q8_0 code 0; Q4_0 code 8; Q5_0 code 16; Q6_K code 32 (with any scale);
  Q4_K / Q5_K: d = dmin and, per sub-block j, a code q0_j and a min
  m_j = sc_j * q0_j, so that d sc_j q0_j - dmin m_j = 0 exactly; the pairs
  (sc_j, q0_j) include codes that are not powers of two.

make_matrix(t, n, k, kind, rng) returns uint8 [n * row_bytes] where every
row follows one of the kinds:
  "zero"    every weight of the row is zero;
  "sparse"  every block zero except two random elements with random codes;
  "single"  zero except one element of the whole row;
  "dense"   random codes everywhere except one zero-weight element per block
            at a fixed position (zero_pos), the same for every row;
  "random"  random codes everywhere.
"""
from __future__ import annotations

import numpy as np

import packing as PK

Q4_0, Q8_0, Q4_K, Q6_K, Q5_0, Q5_K = PK.Q4_0, PK.Q8_0, PK.Q4_K, PK.Q6_K, PK.Q5_0, PK.Q5_K

# (sc_j, q0_j) per sub-block; m_j = sc_j * q0_j <= 63
PAIRS_4 = [(1, 8), (3, 5), (7, 9), (2, 15), (63, 1), (4, 13), (5, 11), (9, 7)]
PAIRS_5 = [(1, 8), (3, 5), (7, 9), (2, 15), (63, 1), (4, 13), (1, 31), (2, 31)]
ZERO_CODE = {Q8_0: 0, Q4_0: 8, Q5_0: 16, Q6_K: 32}
CODE_MAX = {Q8_0: 127, Q4_0: 15, Q5_0: 31, Q6_K: 63, Q4_K: 15, Q5_K: 31}


def _d16(rng, lo, hi) -> int:
    return int(PK.f16(rng.uniform(lo, hi)))


def zero_codes(t: int):
    """Per-element code that gives a zero weight (one block)."""
    be = PK.BE[t]
    if t in ZERO_CODE:
        return np.full(be, ZERO_CODE[t], np.int64)
    pairs = PAIRS_4 if t == Q4_K else PAIRS_5
    return np.repeat(np.array([q0 for (_, q0) in pairs], np.int64), 32)


def _random_codes(t, rng, zero):
    """Random codes, none equal to the zero code of its element."""
    lo = -127 if t == Q8_0 else 0
    v = rng.integers(lo, CODE_MAX[t] + 1, size=zero.shape)
    while True:
        same = v == zero
        if not same.any():
            return v
        v[same] = rng.integers(lo, CODE_MAX[t] + 1, size=int(same.sum()))


def block(t: int, rng, nonzero=(), all_random=False) -> bytes:
    """One block: zero weights except at the element indices in `nonzero`
    (random codes there), or random codes everywhere if all_random."""
    be = PK.BE[t]
    q = zero_codes(t)
    idx = np.arange(be) if all_random else np.asarray(list(nonzero), dtype=np.int64)
    if idx.size:
        q[idx] = _random_codes(t, rng, q[idx])
    if t == Q8_0:
        return PK.pack_q8_0(_d16(rng, 1e-3, 1e-2), q)
    if t == Q4_0:
        return PK.pack_q4_0(_d16(rng, 1e-3, 1e-2), q)
    if t == Q5_0:
        return PK.pack_q5_0(_d16(rng, 1e-3, 1e-2), q)
    if t == Q6_K:
        sc = rng.integers(-64, 64, size=16)
        sc[sc == 0] = 1
        return PK.pack_q6_k(_d16(rng, 1e-4, 1e-3), sc, q)
    pairs = PAIRS_4 if t == Q4_K else PAIRS_5
    sc = [s for (s, _) in pairs]
    m = [s * q0 for (s, q0) in pairs]
    d = _d16(rng, 1e-4, 1e-3)
    pack = PK.pack_q4_k if t == Q4_K else PK.pack_q5_k
    return pack(d, d, sc, m, q)


def make_matrix(t: int, n: int, k: int, kinds, rng, zero_pos: int = 5) -> np.ndarray:
    """Rows cycle through `kinds` (see the module docstring)."""
    be = PK.BE[t]
    nb = k // be
    rows = []
    for r in range(n):
        kind = kinds[r % len(kinds)]
        if kind == "single":
            hot = int(rng.integers(0, k))
        blocks = []
        for b in range(nb):
            if kind == "zero":
                blocks.append(block(t, rng))
            elif kind == "sparse":
                blocks.append(block(t, rng, nonzero=[int(v) for v in rng.choice(be, 2, replace=False)]))
            elif kind == "single":
                blocks.append(block(t, rng, nonzero=[hot - b * be] if hot // be == b else []))
            elif kind == "dense":
                blocks.append(block(t, rng, nonzero=[e for e in range(be) if e != zero_pos]))
            else:
                blocks.append(block(t, rng, all_random=True))
        rows.append(b"".join(blocks))
    return np.frombuffer(b"".join(rows), dtype=np.uint8).copy()
