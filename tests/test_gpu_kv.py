"""GPU parity of the Q8_0 / Q4_0 encoder (the KV-cache codec): the HIP
library (through its C ABI) against the CPU oracle on the same seeded
inputs.  Bar: the encoded bytes are identical (the codes are integers
decided in fp32 on both sides, the scale is fp16 of the same fp32 value).
Inputs: fp16 and fp32 values ~ N(0, 1), blocks on exact ties of the
rounding rule, a wide dynamic range (fp16 scale underflow to subnormal and
zero), zero blocks, equal-magnitude opposite-sign maxima; shapes from one
block to several workgroups with a partial last group, and one layer's K
rows of Llama-3-8B over an 8192-token context.
"""
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
ENC = [G.Q8_0, G.Q4_0]


def say(*a):
    print(*a, flush=True)


def upload(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def check(t, x, what):
    ref = oracle.quantize(t, x)
    got = q.quantize(upload(x), t).cpu().numpy()
    assert got.shape == ref.shape
    bad = np.nonzero(got != ref)
    assert bad[0].size == 0, "%s %s: %d bytes differ, first at %s (got %d, ref %d)" % (
        G.NAMES[t], what, bad[0].size, (bad[0][0], bad[1][0]), got[bad[0][0], bad[1][0]], ref[bad[0][0], bad[1][0]])


def tie_blocks(t, nblk, e, rng):
    """Blocks on the rounding grid: the block maximum makes d = 2^e and
    1/d = 2^-e exactly, and every other value is a half-integer multiple of
    2^e, i.e. an exact tie of the code rounding."""
    lim = 126 if t == G.Q8_0 else 8
    m = rng.integers(-lim, lim, (nblk, 32)) + 0.5
    if t == G.Q4_0:
        m = np.clip(m, -7.5, 7.5)
    x = m * 2.0 ** e
    j = rng.integers(0, 32, nblk)
    sign = rng.choice([-1.0, 1.0], nblk)
    x[np.arange(nblk), j] = (127.0 if t == G.Q8_0 else 8.0) * 2.0 ** e * sign
    return x


@pytest.mark.parametrize("t", ENC)
@pytest.mark.parametrize("dt", [np.float16, np.float32])
def test_quantize_bit_exact(t, dt):
    rng = np.random.default_rng(31 + t)
    for n, k in [(1, 32), (37, 96), (300, 1024), (5, 4096)]:
        say("quantize", G.NAMES[t], dt.__name__, n, k)
        check(t, rng.standard_normal((n, k)).astype(dt), "normal %dx%d" % (n, k))
    for e in (-4, 0, 3):
        check(t, tie_blocks(t, 130, e, rng).reshape(65, 64).astype(dt), "ties 2^%d" % e)
    wide = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-12 if dt == np.float32 else -8,
                                                                 8 if dt == np.float32 else 6, (64, 1)))
    check(t, wide.astype(dt), "wide range")
    z = rng.standard_normal((4, 128)).astype(dt)
    z[0] = 0
    z[1, :32] = -0.0
    z[2, 32:64] = 0
    z[2, 40] = 1e-3
    z[3, :32] = 0
    z[3, 5], z[3, 20] = 3, -3          # the first of equal magnitudes decides the Q4_0 sign
    z[3, 32:64] = 0
    z[3, 40], z[3, 33] = -2, 2
    check(t, z, "zeros and ties of magnitude")


@pytest.mark.parametrize("t", ENC)
def test_quantize_kv_context(t):
    _, tt, n, k, seed = [m for m in G.workload(10) if m[1] == t][0]
    say("quantize kv", G.NAMES[t], n, k)
    x = G.gen_x_f16(n, k, seed)
    check(t, x, "kv %dx%d" % (n, k))
    # decoding the GPU bytes back to fp16 (the attention scratch) is the
    # exact fp16 of the oracle's decode of the same bytes
    b = q.quantize(upload(x), t)
    back = q.dequant_f16(b, t, n, k).cpu().view(torch.int16).numpy().view(np.uint16)
    ref = oracle.dequant_f16(t, b.cpu().numpy(), n, k)
    assert np.array_equal(np.where(back == 0x8000, 0, back), np.where(ref == 0x8000, 0, ref))


def test_quantize_rejects_without_launching():
    x = upload(np.ones((4, 64), np.float16))
    out = torch.full((4, 68), 7, dtype=torch.uint8, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    assert q.lib.qmm_quantize_f16(q.Q4_K, x.data_ptr(), 4, 64, out.data_ptr(), s) == q.ERR_TYPE
    assert q.lib.qmm_quantize_f16(q.Q8_0, x.data_ptr() + 2, 4, 64, out.data_ptr(), s) == q.ERR_ALIGN
    torch.cuda.synchronize()
    assert (out.cpu() == 7).all()
    with pytest.raises(ValueError):
        q.quantize(x.t(), q.Q8_0)
