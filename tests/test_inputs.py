"""Checks of the seeded synthetic input generator (CPU only).

The generator only draws field values; these tests read the fields back with
the test-side parser and check ranges / distributions, determinism, and the
workload byte totals against the figures the pages give.
"""
import numpy as np
import pytest

import qmm_inputs as G
import packing as P


def _fields(t, w):
    raw = w.reshape(-1)
    return [P.read_fields(t, raw[i:i + P.BB[t]].tobytes()) for i in range(0, raw.size, P.BB[t])]


def _h(u):
    return float(np.array(u, np.uint16).view(np.float16))


def test_deterministic_and_seed_sensitive():
    a = G.gen_weights(G.Q4_K, 8, 512, seed=5)
    b = G.gen_weights(G.Q4_K, 8, 512, seed=5)
    c = G.gen_weights(G.Q4_K, 8, 512, seed=6)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert a.shape == (8, 2 * 144)


@pytest.mark.parametrize("t,lo,hi", [(G.Q8_0, 1e-3, 1e-2), (G.Q4_0, 1e-3, 1e-2), (G.Q4_K, 1e-4, 1e-3), (G.Q6_K, 1e-4, 1e-3),
                                     (G.Q5_0, 1e-3, 1e-2), (G.Q5_K, 1e-4, 1e-3)])
def test_field_ranges(t, lo, hi):
    w = G.gen_weights(t, 64, 4 * G.BLOCK_ELEMS[t], seed=3)
    fs = _fields(t, w)
    d = np.array([_h(f["d"]) for f in fs])
    # fp16 rounding of the endpoints may step just outside [lo, hi]
    assert d.min() >= np.float16(lo) * (1 - 2 ** -10) and d.max() <= np.float16(hi) * (1 + 2 ** -10)
    q = np.concatenate([f["q"] for f in fs])
    if t == G.Q8_0:
        assert q.min() >= -127 and q.max() <= 127 and q.min() < -100 and q.max() > 100
    elif t == G.Q4_0 or t == G.Q4_K:
        assert q.min() == 0 and q.max() == 15
    elif t == G.Q5_0 or t == G.Q5_K:
        assert q.min() == 0 and q.max() == 31
    else:
        assert q.min() == 0 and q.max() == 63
        sc = np.concatenate([f["sc"] for f in fs])
        assert sc.min() == -64 and sc.max() == 63
    if t in (G.Q4_K, G.Q5_K):
        dmin = np.array([_h(f["dmin"]) for f in fs])
        assert dmin.min() >= np.float16(lo) * (1 - 2 ** -10) and dmin.max() <= np.float16(hi) * (1 + 2 ** -10)
        sc = np.concatenate([f["sc"] for f in fs])
        m = np.concatenate([f["m"] for f in fs])
        assert sc.min() == 0 and sc.max() == 63 and m.min() == 0 and m.max() == 63


def test_activation_distribution():
    x = G.gen_x(4096, 8, seed=9)
    assert x.dtype == np.float32 and x.shape == (8, 4096)
    assert abs(x.mean()) < 0.05 and abs(x.std() - 1) < 0.05
    X = G.gen_x_f16(512, 64, seed=9)
    assert X.dtype == np.float16 and abs(float(X.astype(np.float32).std()) - 1) < 0.05


def _total_bytes(cfg):
    return sum(n * G.row_bytes(t, k) for _, t, n, k, _ in G.workload(cfg))


def test_workload_shapes_and_byte_totals():
    assert len(G.workload(2)) == 154 and len(G.workload(3)) == 224 and len(G.workload(5)) == 225
    assert _total_bytes(1) == 4456448
    assert _total_bytes(2) == 544997376
    assert _total_bytes(3) == 3925868544
    # dotLLM "GPU Inference", VRAM Estimation: Llama 3 8B Q4_K_M weights ~4.9 GB
    tot5 = _total_bytes(5)
    assert tot5 == 4875853824 and abs(tot5 / 1e9 - 4.9) < 0.05
    head = [m for m in G.workload(5) if m[0] == "lm_head"][0]
    assert head[2] * G.row_bytes(head[1], head[3]) == 430940160
    seeds = [s for *_, s in G.workload(3)]
    assert len(set(seeds)) == len(seeds) and seeds[0] == 3000


def test_token_ids():
    ids = G.gen_ids(128256, 4096, seed=9500)
    assert ids.dtype == np.int32 and ids.min() >= 0 and ids.max() < 128256
    assert np.array_equal(ids, G.gen_ids(128256, 4096, seed=9500))
    assert len(np.unique(ids)) > 4000       # nearly all distinct rows
    embd = G.workload(9)
    # Llama 3.2 1B Q8_0 token table: 128256 x 2048 at 34 B per 32 weights
    assert embd[0][1:4] == (G.Q8_0, 128256, 2048) and 128256 * G.row_bytes(G.Q8_0, 2048) == 279085056
