"""Every entry point captured in one HIP graph and replayed several times,
with new inputs copied into the captured buffers and eager work and host
synchronizations between the replays: each replay equals eager calls on the
same inputs (bit for bit for the deterministic kernels; the split-K GEMM,
whose fp32 atomics add in a varying order, within its tolerance of the
oracle).  The split-K path clears y with a fill kernel, not a memset node.
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


def up(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def test_graph_replays_match_eager():
    rng = np.random.default_rng(77)
    # inputs (captured buffers) and their per-replay contents
    w40 = up(G.gen_weights(G.Q4_0, 2048, 5632, 1))          # wide-k batch-1 GEMV
    w4k = up(G.gen_weights(G.Q4_K, 1024, 4096, 2))          # batch-8 MFMA GEMV, GEMM
    w6k = up(G.gen_weights(G.Q6_K, 700, 4096, 3))           # grouped GEMV
    tab = up(G.gen_weights(G.Q8_0, 5000, 2048, 4))          # embedding table
    x1 = torch.empty((1, 5632), device=DEV)
    x8 = torch.empty((8, 4096), device=DEV)
    xg = [torch.empty((1, 4096), device=DEV) for _ in range(2)]
    X = torch.empty((512, 4096), dtype=torch.float16, device=DEV)   # 512 x 1024 x 4096: split K
    ids = torch.empty(64, dtype=torch.int32, device=DEV)
    kv = torch.empty((300, 1024), dtype=torch.float16, device=DEV)

    def fill(r):
        x1.copy_(up(G.gen_x(5632, 1, 100 + r)))
        x8.copy_(up(G.gen_x(4096, 8, 200 + r)))
        for i, t in enumerate(xg):
            t.copy_(up(G.gen_x(4096, 1, 300 + 10 * r + i)))
        X.copy_(up(G.gen_x_f16(512, 4096, 400 + r)))
        ids.copy_(up(rng.integers(-3, 5003, 64).astype(np.int32)))
        kv.copy_(up(G.gen_x_f16(300, 1024, 500 + r)))

    outs = {
        "gemv1": torch.empty((1, 2048), device=DEV), "gemv8": torch.empty((8, 1024), device=DEV),
        "multi": [torch.empty((1, 700), device=DEV), torch.empty((1, 700), device=DEV)],
        "gemm": torch.empty((512, 1024), device=DEV), "deq": torch.empty((1024, 4096), dtype=torch.float16, device=DEV),
        "emb": torch.empty((64, 2048), device=DEV), "kvq": torch.empty((300, 1088), dtype=torch.uint8, device=DEV),
    }

    def run(o):
        q.gemv(w40, G.Q4_0, 2048, 5632, x1, out=o["gemv1"])
        q.gemv(w4k, G.Q4_K, 1024, 4096, x8, out=o["gemv8"])
        q.gemv_multi([w6k, w6k], G.Q6_K, [700, 700], 4096, xg, outs=o["multi"])
        q.gemm_prefill(w4k, G.Q4_K, 1024, 4096, X, out=o["gemm"])
        q.dequant_f16(w4k, G.Q4_K, 1024, 4096, out=o["deq"])
        q.embed(tab, G.Q8_0, 5000, 2048, ids, out=o["emb"])
        q.quantize(kv, G.Q8_0, out=o["kvq"])

    fill(0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(outs)                       # warm up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(outs)

    for r in range(4):
        fill(r)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {k: ([t.clone() for t in v] if isinstance(v, list) else v.clone()) for k, v in outs.items()}
        # eager work between the replays, then the same calls eagerly
        eager = {k: ([torch.full_like(t, 7) for t in v] if isinstance(v, list) else torch.full_like(v, 7))
                 for k, v in outs.items()}
        run(eager)
        torch.cuda.synchronize()
        for k in outs:
            if k == "gemm":
                continue
            a = got[k] if isinstance(got[k], list) else [got[k]]
            b = eager[k] if isinstance(eager[k], list) else [eager[k]]
            for u, v in zip(a, b):
                assert torch.equal(u, v), (r, k)
        rows = [0, 1, 255, 256, 511]
        Xh = X.cpu().numpy()
        ref, absum = oracle.gemm(G.Q4_K, w4k.cpu().numpy(), 1024, 4096, Xh, rows=rows)
        err = np.abs(got["gemm"].cpu().numpy()[rows] - ref)
        assert np.all(err <= 1e-3 * absum), r
        print("replay", r, "ok", flush=True)


def test_concurrent_host_threads():
    """Four host threads, each on its own stream, call the GEMV and the GEMM
    at the same time (the launch parameters they share are read from
    per-device atomic caches); every result matches the single-threaded
    one."""
    import threading
    jobs = []
    for i in range(4):
        t = [G.Q4_0, G.Q4_K, G.Q6_K, G.Q8_0][i]
        n, k = 1000 + 37 * i, 4096
        w = up(G.gen_weights(t, n, k, 60 + i))
        x = up(G.gen_x(k, 1 + 2 * i, 70 + i))
        X = up(G.gen_x_f16(33, k, 80 + i))
        jobs.append((t, n, k, w, x, X))
    ref = [(q.gemv(w, t, n, k, x).clone(), q.gemm_prefill(w, t, n, k, X).clone()) for t, n, k, w, x, X in jobs]
    torch.cuda.synchronize()
    results = [None] * 4
    errors = []
    barrier = threading.Barrier(4)

    def work(i):
        try:
            t, n, k, w, x, X = jobs[i]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                barrier.wait()
                outs = [(q.gemv(w, t, n, k, x), q.gemm_prefill(w, t, n, k, X)) for _ in range(10)]
            s.synchronize()
            results[i] = outs
        except Exception as e:          # reported below
            errors.append(e)

    th = [threading.Thread(target=work, args=(i,)) for i in range(4)]
    for h in th:
        h.start()
    for h in th:
        h.join()
    assert not errors, errors
    for i, outs in enumerate(results):
        for y, Y in outs:
            assert torch.equal(y, ref[i][0]), i
            # shapes whose GEMM splits K add in a varying order: compare closely
            assert torch.allclose(Y, ref[i][1], rtol=0, atol=1e-4 * float(ref[i][1].abs().max())), i
