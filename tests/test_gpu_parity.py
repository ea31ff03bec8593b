"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
the same seeded inputs.

Bars:
  dequant   bit-exact fp32 (+0 == -0);
  gemv      |y - ref| <= 2e-5 * sum|w x| per output element (exact 0 when the
            sum is 0);
  gemm      |Y - ref| <= 1e-3 * sum|w x| per output element, and X = one-hot
            rows reproduce fp16_RNE(w) exactly.
Sizes span several tiles / segments and ragged tails; the full workload shapes
are checked too (GEMM on sampled rows of M).
"""
import numpy as np
import pytest

import oracle
import packing as PK
import qmm_inputs as G

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import dequant_matmul_amd as q  # noqa: E402

DEV = "cuda:0"
TYPES = [G.Q4_0, G.Q8_0, G.Q4_K, G.Q6_K, G.Q5_0, G.Q5_K]
GEMV_TOL = 2e-5
GEMM_TOL = 1e-3


def say(*a):
    print(*a, flush=True)


def upload(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def check_tol(got, ref, absum, tol, what):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    bound = tol * absum
    zero = absum == 0
    assert np.all(got[zero] == 0), what + ": nonzero output where sum|w x| = 0"
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / np.where(bound > 0, bound, 1)), err.shape)
        raise AssertionError("%s: %d elements over tolerance, worst at %s: got %r ref %r bound %r"
                             % (what, int(bad.sum()), i, got[i], ref[i], bound[i]))
    return float((err[~zero] / absum[~zero]).max()) if (~zero).any() else 0.0


# ---------------------------------------------------------------- dequant ---

DEQ_SHAPES = [(1, None), (37, None), (130, 3), (64, 16)]   # (n, blocks per row; None = 1)


@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("shape", DEQ_SHAPES)
def test_dequant_bit_exact_small(t, shape):
    n, nb = shape
    k = G.BLOCK_ELEMS[t] * (nb or 1)
    say("dequant", G.NAMES[t], n, k)
    w = G.gen_weights(t, n, k, seed=100 + n + t)
    ref = oracle.dequant(t, w, n, k)
    got = q.dequant(upload(w), t, n, k).cpu().numpy()
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("t,n,k", [(G.Q8_0, 2048, 2048), (G.Q4_0, 5632, 2048), (G.Q4_K, 14336, 4096),
                                   (G.Q6_K, 4096, 14336)])
def test_dequant_bit_exact_workload_shapes(t, n, k):
    say("dequant full", G.NAMES[t], n, k)
    w = G.gen_weights(t, n, k, seed=7)
    ref = oracle.dequant(t, w, n, k)
    got = q.dequant(upload(w), t, n, k).cpu().numpy()
    assert np.array_equal(got, ref)


def test_dequant_extreme_scales():
    """fp16 scales over the whole finite range (incl. subnormals and negative
    values) still give bit-identical fp32 weights."""
    for t in TYPES:
        n, k = 16, 4 * G.BLOCK_ELEMS[t]
        w = G.gen_weights(t, n, k, seed=3, d_range=(-6e4, 6e4))
        w2 = G.gen_weights(t, n, k, seed=4, d_range=(-1e-6, 1e-6))   # fp16 subnormals
        for ww in (w, w2):
            ref = oracle.dequant(t, ww, n, k)
            got = q.dequant(upload(ww), t, n, k).cpu().numpy()
            assert np.array_equal(got, ref), G.NAMES[t]


# ------------------------------------------------------------------- gemv ---

GEMV_SHAPES = [(1, 1), (37, 3), (130, 9), (259, 17), (64, 40)]   # (n, blocks per row)


@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("batch", [1, 2, 3, 4, 8])
def test_gemv_small_and_ragged(t, batch):
    worst = 0.0
    for n, nb in GEMV_SHAPES:
        k = G.BLOCK_ELEMS[t] * nb
        say("gemv", G.NAMES[t], "n", n, "k", k, "batch", batch)
        w = G.gen_weights(t, n, k, seed=200 + nb)
        x = G.gen_x(k, batch, seed=300 + nb)
        ref, absum = oracle.gemv(t, w, n, k, x)
        got = q.gemv(upload(w), t, n, k, upload(x)).cpu().numpy()
        worst = max(worst, check_tol(got, ref, absum, GEMV_TOL, "gemv %s n=%d k=%d B=%d" % (G.NAMES[t], n, k, batch)))
    say("  worst relative error", worst)


@pytest.mark.parametrize("t,n,k", [(G.Q8_0, 2048, 2048), (G.Q4_0, 2048, 5632), (G.Q4_0, 256, 2048),
                                   (G.Q4_0, 2048, 2048), (G.Q4_0, 5632, 2048), (G.Q4_0, 4099, 1952),
                                   (G.Q4_0, 1023, 96), (G.Q5_0, 5632, 2048), (G.Q5_0, 300, 2048),
                                   (G.Q4_K, 14336, 4096), (G.Q4_K, 4096, 14336), (G.Q4_K, 1024, 4096),
                                   (G.Q4_K, 1000, 3840), (G.Q6_K, 4096, 14336),
                                   (G.Q6_K, 1024, 4096), (G.Q5_0, 4096, 4096), (G.Q5_K, 14336, 4096),
                                   (G.Q5_K, 4096, 14336)])
@pytest.mark.parametrize("batch", [1, 8])
def test_gemv_workload_shapes(t, n, k, batch):
    say("gemv full", G.NAMES[t], n, k, batch)
    w = G.gen_weights(t, n, k, seed=11)
    x = G.gen_x(k, batch, seed=12)
    ref, absum = oracle.gemv(t, w, n, k, x)
    got = q.gemv(upload(w), t, n, k, upload(x)).cpu().numpy()
    say("  worst relative error", check_tol(got, ref, absum, GEMV_TOL, "gemv %s %dx%d" % (G.NAMES[t], n, k)))


@pytest.mark.parametrize("t,n,k", [(G.Q8_0, 4099, 2048), (G.Q4_0, 7433, 2048), (G.Q5_0, 6007, 2048),
                                   (G.Q4_K, 3641, 4096), (G.Q5_K, 2981, 4096), (G.Q6_K, 2501, 4096),
                                   (G.Q6_K, 1001, 10240)])
def test_gemv_batch1_large_ragged(t, n, k):
    """Batch 1 just past 8 MiB of weights (the non-temporal loads through a
    buffer resource per row), odd row counts (waves with one item fewer
    than others), and a Q6_K row of 40 super-blocks on the split-k kernel."""
    assert n * G.row_bytes(t, k) >= 8 << 20
    say("gemv large ragged", G.NAMES[t], n, k)
    w = G.gen_weights(t, n, k, seed=61)
    x = G.gen_x(k, 1, seed=62)
    ref, absum = oracle.gemv(t, w, n, k, x)
    got = q.gemv(upload(w), t, n, k, upload(x)).cpu().numpy()
    say("  worst relative error", check_tol(got, ref, absum, GEMV_TOL, "gemv %s %dx%d" % (G.NAMES[t], n, k)))


@pytest.mark.parametrize("t", TYPES)
def test_gemv_and_gemm_wide_k(t):
    """k past the widest x staging of the batch-1 kernels (16384), with a
    partial last segment: batch 1 takes the generic segment-by-segment
    kernel, batches 3 and 8 their usual paths over many segments; the GEMM
    runs 161 K steps."""
    k = 20480 if G.BLOCK_ELEMS[t] == 256 else 16416
    n = 133
    w = G.gen_weights(t, n, k, seed=900 + t)
    wd = upload(w)
    for batch in (1, 3, 8):
        say("gemv wide k", G.NAMES[t], n, k, batch)
        x = G.gen_x(k, batch, seed=910 + batch)
        ref, absum = oracle.gemv(t, w, n, k, x)
        got = q.gemv(wd, t, n, k, upload(x)).cpu().numpy()
        check_tol(got, ref, absum, GEMV_TOL, "gemv wide k %s B=%d" % (G.NAMES[t], batch))
    say("gemm wide k", G.NAMES[t], 70, n, k)
    X = G.gen_x_f16(70, k, seed=920)
    ref, absum = oracle.gemm(t, w, n, k, X)
    got = q.gemm_prefill(wd, t, n, k, upload(X)).cpu().numpy()
    check_tol(got, ref, absum, GEMM_TOL, "gemm wide k %s" % G.NAMES[t])


@pytest.mark.parametrize("batch", [1, 2, 4, 8])
def test_gemv_lm_head(batch):
    """The largest matrix of the workloads: the 128256 x 4096 Q6_K LM head of
    the Q4_K_M-style mix (431 MB), every output against the oracle."""
    t, n, k = G.Q6_K, 128256, 4096
    say("gemv lm head", n, k, batch)
    w = G.gen_weights(t, n, k, seed=5024)
    x = G.gen_x(k, batch, seed=5524)
    ref, absum = oracle.gemv(t, w, n, k, x)
    got = q.gemv(upload(w), t, n, k, upload(x)).cpu().numpy()
    say("  worst relative error", check_tol(got, ref, absum, GEMV_TOL, "lm head B=%d" % batch))


@pytest.mark.parametrize("t", TYPES)
def test_gemv_special_inputs(t):
    n, k = 70, 8 * G.BLOCK_ELEMS[t]
    w = G.gen_weights(t, n, k, seed=5)
    W = oracle.dequant(t, w, n, k)
    wd = upload(w)
    # one-hot x selects a column (exactly: a single nonzero product)
    for col in (0, 17, k // 2 + 3, k - 1):
        x = np.zeros((1, k), np.float32)
        x[0, col] = 1.0
        got = q.gemv(wd, t, n, k, upload(x)).cpu().numpy()[0]
        assert np.array_equal(got, W[:, col]), col
    # zero x -> exactly zero
    got = q.gemv(wd, t, n, k, upload(np.zeros((3, k), np.float32))).cpu().numpy()
    assert not got.any()
    # each batch column equals the batch-1 call
    x = G.gen_x(k, 8, seed=6)
    y8 = q.gemv(wd, t, n, k, upload(x)).cpu().numpy()
    for b in (0, 3, 7):
        y1 = q.gemv(wd, t, n, k, upload(x[b:b + 1])).cpu().numpy()
        ref, absum = oracle.gemv(t, w, n, k, x[b:b + 1])
        check_tol(y1, ref, absum, GEMV_TOL, "batch-1")
        check_tol(y8[b:b + 1], ref, absum, GEMV_TOL, "batch-8 column")


@pytest.mark.parametrize("t", TYPES)
def test_gemv_batch_one_hot_exact(t):
    """Batch 8 with one-hot rows: every output is a single product w * 1,
    so each row of y must equal a column of the exact dequantized weights."""
    n, k = 70, 8 * G.BLOCK_ELEMS[t]
    w = G.gen_weights(t, n, k, seed=15)
    W = oracle.dequant(t, w, n, k)
    cols = [0, 5, 31, 32, k // 2 + 3, k - 256 + 17, k - 2, k - 1]
    x = np.zeros((8, k), np.float32)
    for b, c in enumerate(cols):
        x[b, c] = 1.0
    got = q.gemv(upload(w), t, n, k, upload(x)).cpu().numpy()
    for b, c in enumerate(cols):
        assert np.array_equal(got[b], W[:, c]), (G.NAMES[t], b, c)


@pytest.mark.parametrize("t", [G.Q4_K, G.Q6_K])
def test_gemv_batch_dynamic_range(t):
    """Activation rows of very different magnitudes, tiny elements next to
    large ones in the same block, and an all-zero block: batch > 1 splits x
    into two fp16 parts per 256-element block after a power-of-two scaling,
    which must keep the 2e-5 bound over the whole fp32 range."""
    n, k = 45, 6 * 256
    w = G.gen_weights(t, n, k, seed=21)
    x = G.gen_x(k, 7, seed=22).astype(np.float64)
    mags = [1e-30, 1e-6, 1e-2, 1.0, 3e3, 1e20, 1e-38]
    x *= np.array(mags)[:, None]
    x[:, ::3] *= 1e-9          # tiny elements inside every block
    x[2, 256:512] = 0.0        # one empty block
    x[4, 1000] = 6e4 * 1e4     # one element far above the rest of its block
    x = x.astype(np.float32)
    ref, absum = oracle.gemv(t, w, n, k, x)
    got = q.gemv(upload(w), t, n, k, upload(x)).cpu().numpy()
    say("  worst relative error", check_tol(got, ref, absum, GEMV_TOL, "dynamic range %s" % G.NAMES[t]))


def _edge_field_rows(t, n, nb, seed):
    """K-quant rows whose fields sit at the edges of their ranges.  Q6_K: int8
    scales -128, 127 and odd values past 64 (where (q - 32) * scale needs 12
    bits), codes 0, 63 and 32, d from fp16 subnormal to 6e4.  Q4_K: 6-bit
    scales and mins 0, 1, 62, 63, codes 0 and 15, and d, dmin equal, 2^29
    apart either way round, of opposite signs, or fp16 subnormal."""
    rng = np.random.default_rng(seed)
    rows = []
    for r in range(n):
        blks = []
        for _ in range(nb):
            if t == G.Q6_K:
                sc = rng.choice([-128, 127, -127, 125, 65, -65, 99, -1, 0, 1], size=16)
                q6 = rng.integers(0, 64, size=256) if r % 3 == 0 else rng.choice([0, 63, 1, 62, 32, 31, 33], size=256)
                d = [3e-4, -7e-4, 6e4, 1e-7][r % 4]
                blks.append(PK.pack_q6_k(int(PK.f16(d)), sc, q6))
            else:
                sc = rng.choice([0, 1, 62, 63, 33], size=8)
                m = rng.choice([0, 1, 62, 63, 17], size=8)
                q4 = rng.choice([0, 15, 1, 14], size=256)
                d, dmin = [(1e-3, 1e-3), (6e4, 1e-4), (1e-4, 6e4), (-5e3, 2e-2), (3e-6, -2e-5)][r % 5]
                blks.append(PK.pack_q4_k(int(PK.f16(d)), int(PK.f16(dmin)), sc, m, q4))
        rows.append(b"".join(blks))
    return np.frombuffer(b"".join(rows), np.uint8).reshape(n, -1).copy()


@pytest.mark.parametrize("t", [G.Q4_K, G.Q6_K])
@pytest.mark.parametrize("nb", [5, 16, 18])
def test_kquant_edge_fields(t, nb):
    """Dequant bit-exact, every GEMV path within 2e-5, and the GEMM within
    1e-3 on the rows whose weights fit fp16, for blocks at the edges of the
    format (full-range Q6_K scales are what real Q6_K files hold)."""
    n, k = 40, 256 * nb
    w = _edge_field_rows(t, n, nb, seed=77 + t + nb)
    say("edge fields", G.NAMES[t], n, k)
    W = oracle.dequant(t, w, n, k)
    assert np.array_equal(q.dequant(upload(w), t, n, k).cpu().numpy(), W)
    for batch in (1, 2, 5, 8):
        x = G.gen_x(k, batch, seed=78 + batch)
        ref, absum = oracle.gemv(t, w, n, k, x)
        got = q.gemv(upload(w), t, n, k, upload(x)).cpu().numpy()
        say("  B", batch, "worst relative error",
            check_tol(got, ref, absum, GEMV_TOL, "edge fields %s B=%d" % (G.NAMES[t], batch)))
    fits = np.abs(W).max(axis=1) < 6e4
    X = G.gen_x_f16(33, k, seed=79)
    ref, absum = oracle.gemm(t, w, n, k, X)
    got = q.gemm_prefill(upload(w), t, n, k, upload(X)).cpu().numpy()
    check_tol(got[:, fits], ref[:, fits], absum[:, fits], GEMM_TOL, "edge fields gemm %s" % G.NAMES[t])


@pytest.mark.parametrize("t,n,k,batch", [(G.Q4_K, 33000, 4608, 5), (G.Q6_K, 40000, 1024, 8),
                                         (G.Q6_K, 2100, 4864, 3), (G.Q4_K, 66000, 512, 2),
                                         (G.Q6_K, 70001, 4608, 2)])
def test_gemv_batch_many_tiles(t, n, k, batch):
    """More 16-row tiles than 8 per compute unit (several reduction rounds
    per workgroup), K runs longer than two blocks per wave, waves with no
    block (k = 1024), an odd super-block count per row (Q6_K rows then
    alternate their 4-byte alignment), and batch 2 past 65536 rows (the
    matrix-core kernel; shorter matrices take the vector kernel at B = 2)."""
    say("gemv many tiles", G.NAMES[t], n, k, batch)
    w = G.gen_weights(t, n, k, seed=31)
    x = G.gen_x(k, batch, seed=32)
    ref, absum = oracle.gemv(t, w, n, k, x)
    got = q.gemv(upload(w), t, n, k, upload(x)).cpu().numpy()
    say("  worst relative error", check_tol(got, ref, absum, GEMV_TOL, "gemv %s %dx%d B%d" % (G.NAMES[t], n, k, batch)))


@pytest.mark.parametrize("batch", [3, 8])
def test_gemv_q6k_staged_tiles(batch):
    """Q6_K at k = 4096 with at least four 16-row tiles per workgroup: the
    batch kernel stages whole tiles through LDS.  Rows of random blocks, and
    rows of edge-field blocks (full-range int8 scales), over a ragged last
    tile (16390 rows)."""
    t, n, k = G.Q6_K, 16390, 4096
    say("gemv q6k staged", n, k, batch)
    x = G.gen_x(k, batch, seed=41 + batch)
    w = G.gen_weights(t, n, k, seed=40)
    ref, absum = oracle.gemv(t, w, n, k, x)
    got = q.gemv(upload(w), t, n, k, upload(x)).cpu().numpy()
    say("  random, worst relative error", check_tol(got, ref, absum, GEMV_TOL, "staged random B=%d" % batch))
    base = _edge_field_rows(t, 40, 16, seed=42)
    we = np.ascontiguousarray(np.tile(base, ((n + 39) // 40, 1))[:n])
    ref, absum = oracle.gemv(t, we, n, k, x)
    got = q.gemv(upload(we), t, n, k, upload(x)).cpu().numpy()
    say("  edge fields, worst relative error", check_tol(got, ref, absum, GEMV_TOL, "staged edge B=%d" % batch))


def test_gemv_unaligned_rows():
    """Row sizes that are not a multiple of 16 bytes take the 2-byte staging
    path."""
    for t, nb in ((G.Q8_0, 3), (G.Q4_0, 5), (G.Q6_K, 3), (G.Q5_0, 3)):
        k = G.BLOCK_ELEMS[t] * nb
        assert G.row_bytes(t, k) % 16 != 0
        for batch in (1, 5):
            w = G.gen_weights(t, 45, k, seed=9)
            x = G.gen_x(k, batch, seed=10)
            ref, absum = oracle.gemv(t, w, 45, k, x)
            got = q.gemv(upload(w), t, 45, k, upload(x)).cpu().numpy()
            check_tol(got, ref, absum, GEMV_TOL, "unaligned %s" % G.NAMES[t])


def test_gemv_empty_and_k0():
    w = upload(np.zeros(16, np.uint8))
    y = q.gemv(w[:0], G.Q8_0, 0, 32, upload(np.zeros((1, 32), np.float32)))
    assert y.shape == (1, 0)
    y = torch.full((2, 5), 7.0, device=DEV)
    q.gemv(w[:0], G.Q8_0, 5, 0, torch.zeros((2, 0), device=DEV), out=y)
    assert not y.cpu().numpy().any()


# ------------------------------------------------------------------- gemm ---

GEMM_SHAPES = [(1, 1, 1), (7, 50, 3), (130, 200, 9), (257, 129, 5)]   # (m, n, blocks per row)


@pytest.mark.parametrize("t", TYPES)
def test_gemm_small_and_ragged(t):
    worst = 0.0
    for m, n, nb in GEMM_SHAPES:
        k = G.BLOCK_ELEMS[t] * nb
        say("gemm", G.NAMES[t], m, n, k)
        w = G.gen_weights(t, n, k, seed=400 + nb)
        X = G.gen_x_f16(m, k, seed=500 + nb)
        ref, absum = oracle.gemm(t, w, n, k, X)
        got = q.gemm_prefill(upload(w), t, n, k, upload(X)).cpu().numpy()
        worst = max(worst, check_tol(got, ref, absum, GEMM_TOL, "gemm %s %dx%dx%d" % (G.NAMES[t], m, n, k)))
    say("  worst relative error", worst)


@pytest.mark.parametrize("t", TYPES)
def test_gemm_one_hot_rows_give_fp16_weights(t):
    """Row r of X = e_{c_r} makes row r of Y equal to column c_r of W rounded
    to fp16 (round to nearest even), exactly: pins the rounding mode and the
    operand orientation."""
    n, k = 150, 5 * G.BLOCK_ELEMS[t]
    w = G.gen_weights(t, n, k, seed=8)
    W16 = oracle.dequant(t, w, n, k).astype(np.float16).astype(np.float32)
    cols = [0, 1, 31, 32, k // 2, k - 1, 129 % k]
    X = np.zeros((len(cols), k), np.float16)
    for r, c in enumerate(cols):
        X[r, c] = 1.0
    got = q.gemm_prefill(upload(w), t, n, k, upload(X)).cpu().numpy()
    for r, c in enumerate(cols):
        assert np.array_equal(got[r], W16[:, c]), (r, c)


def _tiny_scales(t, w, n, k, rng):
    """Overwrite every fp16 scale field (d, and dmin for Q4_K / Q5_K) with a random
    subnormal fp16 (bits 0x0001..0x03ff), so that many dequantized weights are
    fp16 subnormals or need rounding near the subnormal range."""
    w = w.copy().reshape(n, -1)
    bb, be = G.BLOCK_BYTES[t], G.BLOCK_ELEMS[t]
    nb = k // be
    offs = {G.Q8_0: [0], G.Q4_0: [0], G.Q4_K: [0, 2], G.Q6_K: [208], G.Q5_0: [0], G.Q5_K: [0, 2]}[t]
    for b in range(nb):
        for o in offs:
            bits = rng.integers(1, 0x400, size=n).astype(np.uint16)
            w[:, b * bb + o] = (bits & 0xff).astype(np.uint8)
            w[:, b * bb + o + 1] = (bits >> 8).astype(np.uint8)
    return w.reshape(-1)


@pytest.mark.parametrize("t", TYPES)
def test_gemm_one_hot_subnormal_scales(t):
    """One-hot rows with subnormal fp16 scales: the weights entering the MFMA
    are still exactly fp16_RNE of the fp32 dequantized values (no flush to
    zero of subnormal inputs or results anywhere in the decode)."""
    n, k = 140, 4 * G.BLOCK_ELEMS[t]
    w = _tiny_scales(t, G.gen_weights(t, n, k, seed=9), n, k, np.random.default_rng(19))
    W16 = oracle.dequant(t, w, n, k).astype(np.float16).astype(np.float32)
    assert np.any((W16 != 0) & (np.abs(W16) < 2.0 ** -14)), "no subnormal weights in the case"
    cols = list(range(0, k, max(1, k // 37)))[:40] + [k - 1]
    X = np.zeros((len(cols), k), np.float16)
    for r, c in enumerate(cols):
        X[r, c] = 1.0
    got = q.gemm_prefill(upload(w), t, n, k, upload(X)).cpu().numpy()
    for r, c in enumerate(cols):
        assert np.array_equal(got[r], W16[:, c]), (r, c)


# every 8th row of M plus the edges: at least one row of every 16-row wave
# slice of every M tile, whatever the tile shape
GEMM_ROWS = sorted(set(range(0, 512, 8)) | set(range(7, 512, 16)) | {1, 511})


@pytest.mark.parametrize("t,n", [(G.Q8_0, 14336), (G.Q8_0, 4096), (G.Q4_K, 14336), (G.Q4_K, 4096),
                                 (G.Q4_0, 4096), (G.Q6_K, 4096), (G.Q5_0, 4096), (G.Q5_K, 14336),
                                 (G.Q6_K, 14336), (G.Q4_K, 14296), (G.Q8_0, 14200),   # ragged n
                                 (G.Q4_0, 14336), (G.Q5_0, 14336), (G.Q5_K, 4096)]
                         + [(t, 16384) for t in TYPES])
def test_gemm_prefill_workload_shapes(t, n):
    m, k = G.PREFILL_M, 4096
    say("gemm full", G.NAMES[t], m, n, k)
    w = G.gen_weights(t, n, k, seed=13)
    X = G.gen_x_f16(m, k, seed=14)
    got = q.gemm_prefill(upload(w), t, n, k, upload(X)).cpu().numpy()
    ref, absum = oracle.gemm(t, w, n, k, X, rows=GEMM_ROWS)
    say("  worst relative error", check_tol(got[GEMM_ROWS], ref, absum, GEMM_TOL, "gemm full"))


@pytest.mark.parametrize("t", [G.Q4_K, G.Q6_K])
@pytest.mark.parametrize("mb", [1, 4, 8])
def test_gemm_skinny_matches_oracle(t, mb):
    """M = batch (the skinny-GEMM side of the decode crossover)."""
    n, k = 1000, 4096
    w = G.gen_weights(t, n, k, seed=15)
    X = G.gen_x_f16(mb, k, seed=16)
    ref, absum = oracle.gemm(t, w, n, k, X)
    got = q.gemm_prefill(upload(w), t, n, k, upload(X)).cpu().numpy()
    check_tol(got, ref, absum, GEMM_TOL, "skinny")


def test_gemm_k0_writes_zeros():
    y = torch.full((3, 4), 5.0, device=DEV)
    w = upload(np.zeros(16, np.uint8))
    q.gemm_prefill(w[:0], G.Q4_K, 4, 0, torch.zeros((3, 0), dtype=torch.float16, device=DEV), out=y)
    assert not y.cpu().numpy().any()


def test_native_library_loaded():
    import os
    maps = open("/proc/self/maps").read()
    assert os.path.realpath(q.LIB_PATH) in maps


# ------------------------------------------------------------ gemv_multi ---

# [700, 0] and [37] * 7 + [0]: a trailing empty problem (its weight tensor
# is empty, a null pointer) while waves outnumber the row groups
@pytest.mark.parametrize("t,k,ns", [(G.Q4_K, 4096, [4096, 1024, 1024]), (G.Q4_0, 2048, [5632, 5632]),
                                    (G.Q6_K, 4096, [1024, 3, 0, 700]), (G.Q8_0, 2048, [37] * 9),
                                    (G.Q4_K, 14336, [300, 200]), (G.Q4_0, 2048, [700, 0]),
                                    (G.Q8_0, 2048, [37] * 7 + [0])])
@pytest.mark.parametrize("batch", [1, 4])
def test_gemv_multi_matches_single_calls(t, k, ns, batch):
    """One grouped call gives bit-identical results to one qmm_gemv call per
    problem, and each matches the oracle."""
    say("gemv_multi", G.NAMES[t], k, ns, batch)
    ws = [G.gen_weights(t, n, k, seed=600 + i) for i, n in enumerate(ns)]
    xs = [G.gen_x(k, batch, seed=700 + i) for i in range(len(ns))]
    wd = [upload(w) for w in ws]
    xd = [upload(x) for x in xs]
    ys = q.gemv_multi(wd, t, ns, k, xd)
    for w, n, x, y, a, b in zip(ws, ns, xs, ys, wd, xd):
        single = q.gemv(a, t, n, k, b).cpu().numpy()
        got = y.cpu().numpy()
        assert np.array_equal(got, single)
        if n:
            ref, absum = oracle.gemv(t, w, n, k, x)
            check_tol(got, ref, absum, GEMV_TOL, "gemv_multi")


@pytest.mark.parametrize("t,k,ns", [(G.Q4_0, 2048, [2048, 256, 256]), (G.Q4_0, 2048, [5632, 5632]),
                                    (G.Q4_K, 4096, [4096, 1024, 1024]), (G.Q4_K, 4096, [14336, 14336]),
                                    (G.Q6_K, 4096, [1024, 3, 0, 700]), (G.Q8_0, 1984, [37] * 9),
                                    (G.Q5_0, 2048, [4100, 7]), (G.Q5_K, 3840, [0, 515, 1]),
                                    (G.Q4_K, 4096, [700, 0]), (G.Q4_0, 2048, [37] * 7 + [0]),
                                    (G.Q6_K, 4096, [16384, 16390]),
                                    # eight problems (a full table), ragged and tiny ones among them
                                    (G.Q4_K, 4096, [1, 17, 300, 2, 16, 15, 33, 1000]),
                                    (G.Q6_K, 4096, [5, 40, 1, 16, 700, 2, 31, 64])])
@pytest.mark.parametrize("batch", [1, 3, 8])
def test_gemv_multi_shared_x_matches_single_calls(t, k, ns, batch):
    """A grouped call whose problems all read one x (q / k / v, gate / up)
    stages x once per workgroup (at batch 3..8 of the K-quants: one
    matrix-core launch over the tiles of every problem, a workgroup's tiles
    crossing from one problem into the next); results stay bit-identical to
    one qmm_gemv call per problem, and each matches the oracle."""
    say("gemv_multi shared x", G.NAMES[t], k, ns, batch)
    ws = [G.gen_weights(t, n, k, seed=800 + i) for i, n in enumerate(ns)]
    x = G.gen_x(k, batch, seed=900)
    wd = [upload(w) for w in ws]
    xd = upload(x)
    ys = q.gemv_multi(wd, t, ns, k, [xd] * len(ns))
    for w, n, y, a in zip(ws, ns, ys, wd):
        single = q.gemv(a, t, n, k, xd).cpu().numpy()
        got = y.cpu().numpy()
        assert np.array_equal(got, single)
        if n:
            ref, absum = oracle.gemv(t, w, n, k, x)
            check_tol(got, ref, absum, GEMV_TOL, "gemv_multi shared x")


# ------------------------------------------------------ zero-weight rows ---

import zero_rows as Z  # noqa: E402

ZERO_KINDS = ["zero", "sparse", "single", "dense", "random"]


@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("batch", [1, 2, 5, 8])
def test_gemv_zero_weight_rows(t, batch):
    """Rows of exactly zero weights, mostly zero weights, one nonzero weight,
    or one zero weight per block (tests/zero_rows.py): Q8_0 code 0, Q4_0 code
    8, Q5_0 code 16, Q6_K code 32, Q4_K / Q5_K with d sc q = dmin m.  Every
    product uses the element's own weight, so zero rows give exactly 0 and
    every output meets 2e-5 relative to sum |w x| of its own row (no
    cancellation after a rounding).  Shapes cover the one-segment, the
    multi-segment and the batch kernels."""
    be = G.BLOCK_ELEMS[t]
    shapes = [(70, 8 * be)] + ([(45, 4096), (37, 14336)] if be == 256 else [(45, 2048), (37, 5632)])
    for n, k in shapes:
        say("gemv zero rows", G.NAMES[t], n, k, batch)
        w = Z.make_matrix(t, n, k, ZERO_KINDS, np.random.default_rng(1000 * t + k + batch))
        x = G.gen_x(k, batch, seed=40 + k)
        ref, absum = oracle.gemv(t, w, n, k, x)
        assert (absum[:, 0::5] == 0).all()       # the all-zero rows
        got = q.gemv(upload(w), t, n, k, upload(x)).cpu().numpy()
        check_tol(got, ref, absum, GEMV_TOL, "zero rows %s n=%d k=%d B=%d" % (G.NAMES[t], n, k, batch))


@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("batch", [1, 4, 8])
@pytest.mark.parametrize("ratio", [1e-8, 1e-10])
def test_gemv_large_x_on_zero_weight(t, batch, ratio):
    """In every block the largest |x| sits on a weight that is zero in every
    row, and the other elements (~ N(0, 1)) are about `ratio` times smaller:
    sum |w x| comes from the small elements alone.  The batch path splits x
    into two fp16 parts after scaling each 256-element block to its largest
    |x|; elements down to about 2^-34 of that largest keep the 2e-5 bound."""
    be = G.BLOCK_ELEMS[t]
    n, k = 40, 4 * 256
    w = Z.make_matrix(t, n, k, ["dense"], np.random.default_rng(77 + t), zero_pos=5)
    x = G.gen_x(k, batch, seed=78).astype(np.float64)
    x[:, 5::be] = np.where(x[:, 5::be] < 0, -1.0, 1.0) / ratio
    x = x.astype(np.float32)
    say("gemv large x on zero weight", G.NAMES[t], batch, ratio)
    ref, absum = oracle.gemv(t, w, n, k, x)
    got = q.gemv(upload(w), t, n, k, upload(x)).cpu().numpy()
    say("  worst relative error", check_tol(got, ref, absum, GEMV_TOL, "large x on zero weight"))


@pytest.mark.parametrize("t", [G.Q4_K, G.Q5_K])
@pytest.mark.parametrize("batch", [1, 3, 8])
def test_gemv_k_quant_scale_ratio(t, batch):
    """d and dmin far apart (one of them 2^-12 times the other, which puts it
    among the fp16 subnormals for these ranges), and dmin = 0: the
    per-element weights d sc q - dmin m then need all 24 bits of fp32, which
    the batch path carries as two fp16 parts per weight."""
    n, k = 48, 6 * 256
    bb = G.BLOCK_BYTES[t]
    x = G.gen_x(k, batch, seed=92)

    def put(w, b, off, v):
        w[:, b * bb + off:b * bb + off + 2] = np.frombuffer(v.astype(np.float16).tobytes(), np.uint8).reshape(-1, 2)

    for mode in ("dmin_small", "d_small", "dmin_zero"):
        w = G.gen_weights(t, n, k, seed=93).reshape(n, -1).copy()
        for b in range(k // 256):
            d = np.frombuffer(w[:, b * bb:b * bb + 2].tobytes(), np.float16).astype(np.float64)
            if mode == "dmin_small":
                put(w, b, 2, d * 2.0 ** -12)
            elif mode == "d_small":
                put(w, b, 2, d)
                put(w, b, 0, d * 2.0 ** -12)
            else:
                put(w, b, 2, np.zeros_like(d))
        w = w.reshape(-1)
        say("gemv K-quant scale ratio", G.NAMES[t], batch, mode)
        ref, absum = oracle.gemv(t, w, n, k, x)
        got = q.gemv(upload(w), t, n, k, upload(x)).cpu().numpy()
        check_tol(got, ref, absum, GEMV_TOL, "scale ratio %s %s" % (G.NAMES[t], mode))


@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("nseg", [2, 3, 4, 5, 6, 7, 8])
def test_gemv_split_segments(t, nseg):
    """Batch 1 with k spanning 2..8 segments of 64 lane-units (the waves of a
    workgroup split k by segment, the partial sums meet in LDS), a partial
    last segment and a ragged row count over several workgroups; then the
    same call again gives the same bits."""
    be = G.BLOCK_ELEMS[t]
    sege = 64 * (64 if be == 256 else 32)
    k = nseg * sege - 3 * be
    n = 700
    say("gemv split segments", G.NAMES[t], n, k, nseg)
    w = G.gen_weights(t, n, k, seed=1100 + nseg)
    x = G.gen_x(k, 1, seed=1200 + nseg)
    ref, absum = oracle.gemv(t, w, n, k, x)
    wd, xd = upload(w), upload(x)
    got = q.gemv(wd, t, n, k, xd).cpu().numpy()
    check_tol(got, ref, absum, GEMV_TOL, "split segments %s k=%d" % (G.NAMES[t], k))
    assert np.array_equal(q.gemv(wd, t, n, k, xd).cpu().numpy(), got)
