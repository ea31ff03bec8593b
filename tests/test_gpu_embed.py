"""GPU parity of the FP16 dequant and the quantized embedding gather: the
HIP library (through its C ABI) against the CPU oracle on the same seeded
inputs.  Bar: bit-exact (fp32 values, or fp16 bit patterns; +0 == -0).
Sizes span several workgroups and ragged tails; the embedding tables of the
Llama 3.2 1B (Q8_0) and Llama-3-8B (Q4_K) shapes are checked in full for a
512-token prefill chunk and a single decode token.
"""
import ctypes

import numpy as np
import pytest

import oracle
import qmm_inputs as G

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import dequant_matmul_amd as q  # noqa: E402

DEV = "cuda:0"
TYPES = [G.Q4_0, G.Q8_0, G.Q4_K, G.Q6_K, G.Q5_0, G.Q5_K]
I32_MIN, I32_MAX = -2 ** 31, 2 ** 31 - 1


def say(*a):
    print(*a, flush=True)


def upload(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def half_bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def assert_half_equal(got, ref, what):
    """fp16 bit patterns equal, with -0 == +0."""
    g = np.where(got == 0x8000, 0, got)
    r = np.where(ref == 0x8000, 0, ref)
    bad = np.nonzero(g != r)
    assert bad[0].size == 0, "%s: %d mismatches, first at %s: got %#06x ref %#06x" % (
        what, bad[0].size, tuple(b[0] for b in bad), got[tuple(b[0] for b in bad)], ref[tuple(b[0] for b in bad)])


# -------------------------------------------------------------- dequant f16 ---

@pytest.mark.parametrize("t", TYPES)
def test_dequant_f16_bit_exact(t):
    for n, nb, dr in [(1, 1, None), (37, 3, None), (130, 5, None), (16, 4, (-6e4, 6e4)), (16, 4, (-1e-6, 1e-6))]:
        k = G.BLOCK_ELEMS[t] * nb
        say("dequant_f16", G.NAMES[t], n, k, dr)
        w = G.gen_weights(t, n, k, seed=500 + n + t, d_range=dr)
        ref = oracle.dequant_f16(t, w, n, k)
        got = half_bits(q.dequant_f16(upload(w), t, n, k))
        assert_half_equal(got, ref, "dequant_f16 %s n=%d k=%d" % (G.NAMES[t], n, k))
        if dr == (-6e4, 6e4):
            assert (np.abs(oracle.dequant(t, w, n, k)) >= 65520).any()   # the case reaches fp16 overflow


def test_dequant_f16_workload_shape():
    t, n, k = G.Q4_K, 14336, 4096
    say("dequant_f16 full", G.NAMES[t], n, k)
    w = G.gen_weights(t, n, k, seed=7)
    assert_half_equal(half_bits(q.dequant_f16(upload(w), t, n, k)), oracle.dequant_f16(t, w, n, k), "dequant_f16")


# ------------------------------------------------------------------ embed ---

def _ids(vocab, seq, seed):
    ids = G.gen_ids(max(vocab, 1), seq, seed)
    if seq >= 8:
        # repeats and every kind of invalid id
        ids[:8] = [0, vocab - 1, vocab, -1, I32_MIN, I32_MAX, ids[9 % seq], vocab + 7]
    return ids


@pytest.mark.parametrize("t", TYPES)
@pytest.mark.parametrize("seq", [1, 9, 300])
def test_embed_bit_exact_small(t, seq):
    vocab, nb = 37, 3
    k = G.BLOCK_ELEMS[t] * nb
    say("embed", G.NAMES[t], "vocab", vocab, "k", k, "seq", seq)
    table = G.gen_weights(t, vocab, k, seed=600 + t)
    ids = _ids(vocab, seq, seed=700 + seq)
    tt, it = upload(table), upload(ids)
    ref = oracle.embed(t, table, vocab, k, ids)
    got = q.embed(tt, t, vocab, k, it).cpu().numpy()
    assert np.array_equal(got, ref)
    bad_ids = (ids < 0) | (ids >= vocab)
    assert not np.signbit(got[bad_ids]).any()             # +0 rows
    got16 = half_bits(q.embed(tt, t, vocab, k, it, dtype=torch.float16))
    assert_half_equal(got16, oracle.embed(t, table, vocab, k, ids, f16=True), "embed_f16")


@pytest.mark.parametrize("name,seq", [("embd_q8_0", 512), ("embd_q8_0", 1), ("embd_q4_k", 512)])
def test_embed_full_tables(name, seq):
    _, t, vocab, k, seed = [m for m in G.workload(9) if m[0] == name][0]
    say("embed full", name, vocab, k, "seq", seq)
    table = G.gen_weights(t, vocab, k, seed=seed)
    ids = G.gen_ids(vocab, seq, seed=G.x_seed(9, seq))
    if seq > 2:
        ids[:2] = [0, vocab - 1]          # first and last rows of the table
    tt, it = upload(table), upload(ids)
    ref = oracle.embed(t, table, vocab, k, ids)
    assert np.array_equal(q.embed(tt, t, vocab, k, it).cpu().numpy(), ref)
    assert_half_equal(half_bits(q.embed(tt, t, vocab, k, it, dtype=torch.float16)),
                      oracle.to_half_bits(ref), "embed_f16 " + name)


def test_embed_empty_table_and_offset_ids():
    t, k = G.Q8_0, 64
    # vocab 0: every id is invalid, the table is never read
    out = q.embed(torch.empty(0, dtype=torch.uint8, device=DEV), t, 0, k, upload(np.array([0, 5], np.int32)))
    assert torch.equal(out.cpu(), torch.zeros(2, k))
    # seq 0: nothing to do
    table = G.gen_weights(t, 10, k, seed=1)
    assert q.embed(upload(table), t, 10, k, torch.empty(0, dtype=torch.int32, device=DEV)).shape == (0, k)
    # ids at a 4-byte (not 16-byte) offset are accepted
    ids = np.array([3, 1, 4, 1, 5, 9, 2, 6], np.int32)
    it = upload(ids)[1:]
    assert it.data_ptr() % 16 == 4
    got = q.embed(upload(table), t, 10, k, it).cpu().numpy()
    assert np.array_equal(got, oracle.embed(t, table, 10, k, ids[1:]))


def test_embed_rejects_misaligned_ids_without_launching():
    t, k = G.Q8_0, 32
    table = upload(G.gen_weights(t, 4, k, seed=2))
    raw = torch.zeros(16, dtype=torch.uint8, device=DEV)
    out = torch.full((1, k), 7.0, device=DEV)
    st = q.lib.qmm_embed(t, table.data_ptr(), 4, k, raw.data_ptr() + 2, 1, out.data_ptr(),
                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == q.ERR_ALIGN
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), torch.full((1, k), 7.0))      # untouched


def test_binding_checks_output_tensors():
    """A caller's out= tensor of the wrong dtype, shape or layout is refused
    before anything is launched (the library writes exactly the requested
    elements there)."""
    t, n, k = G.Q8_0, 8, 64
    w = upload(G.gen_weights(t, n, k, seed=3))
    ids = upload(np.array([1, 2], np.int32))
    x = upload(G.gen_x(k, 2, seed=4))
    X = upload(G.gen_x_f16(3, k, seed=5))
    bad = [
        lambda: q.embed(w, t, n, k, ids, out=torch.empty((2, k), dtype=torch.float16, device=DEV)),
        lambda: q.embed(w, t, n, k, ids, dtype=torch.float16, out=torch.empty((2, k), device=DEV)),
        lambda: q.embed(w, t, n, k, ids, out=torch.empty((3, k), device=DEV)),
        lambda: q.dequant(w, t, n, k, out=torch.empty((n, k - 32), device=DEV)),
        lambda: q.dequant_f16(w, t, n, k, out=torch.empty((n, k), device=DEV)),
        lambda: q.gemv(w, t, n, k, x, out=torch.empty((n, 2), device=DEV).t()),
        lambda: q.gemm_prefill(w, t, n, k, X, out=torch.empty((3, n), dtype=torch.float16, device=DEV)),
        lambda: q.quantize(X.float(), t, out=torch.empty((3, 60), dtype=torch.uint8, device=DEV)),
        lambda: q.gemv_multi([w], t, [n], k, [x], outs=[torch.empty((2, n - 1), device=DEV)]),
    ]
    for i, f in enumerate(bad):
        with pytest.raises(ValueError):
            f()
    # matching tensors are used in place
    o = torch.empty((2, k), device=DEV)
    assert q.embed(w, t, n, k, ids, out=o).data_ptr() == o.data_ptr()
