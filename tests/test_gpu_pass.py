"""GPU parity of the decode pass (qmm_gemv_pass): every GEMV of a pass
against the CPU oracle, 2e-5 per output relative to sum |w x|, on chained
stages where a stage reads the outputs of the stage before it (so a stage
that read its x too early would read the NaN the outputs start as), with
mixed block types in one stage launch."""
import numpy as np
import pytest

import oracle
import qmm_inputs as G
import zero_rows as Z

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import dequant_matmul_amd as q  # noqa: E402

DEV = "cuda:0"
TOL = 2e-5
TYPES = [G.Q4_0, G.Q8_0, G.Q4_K, G.Q6_K, G.Q5_0, G.Q5_K]


def say(*a):
    print(*a, flush=True)


def upload(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def check(got, ref, absum, what):
    got = np.asarray(got, np.float64).reshape(ref.shape)
    err = np.abs(got - ref)
    zero = absum == 0
    assert np.all(got[zero] == 0), what + ": nonzero output where sum|w x| = 0"
    bad = err > TOL * absum
    assert not bad.any(), "%s: %d outputs over tolerance (worst %r)" % (
        what, int(bad.sum()), float((err / np.where(absum > 0, absum, 1)).max()))


def nan_out(n):
    return torch.full((n,), float("nan"), dtype=torch.float32, device=DEV)


class Net:
    """A chain of stages: each problem is (name, type, n, k, x_source, stage);
    x_source is an input vector name or the name of an earlier problem."""

    def __init__(self, spec, inputs, seed=0):
        self.spec = spec
        self.host_w = {}
        self.w = {}
        self.y = {}
        self.x = {nm: upload(v) for nm, v in inputs.items()}
        for i, (name, t, n, k, src, stage) in enumerate(spec):
            self.host_w[name] = G.gen_weights(t, n, k, seed=seed + 31 * i)
            self.w[name] = upload(self.host_w[name])
            self.y[name] = nan_out(n)

    def src(self, s):
        return self.y[s] if s in self.y else self.x[s]

    def problems(self):
        return [(self.w[nm], t, n, k, self.src(src), self.y[nm], st) for (nm, t, n, k, src, st) in self.spec]

    def run(self):
        q.gemv_pass(self.problems())
        torch.cuda.synchronize()

    def verify(self, what):
        for (nm, t, n, k, src, st) in self.spec:
            xin = self.src(src).cpu().numpy().reshape(1, k)
            assert np.isfinite(xin).all(), "%s: input of %s not finite" % (what, nm)
            ref, absum = oracle.gemv(t, self.host_w[nm], n, k, xin)
            check(self.y[nm].cpu().numpy(), ref[0], absum[0], "%s %s" % (what, nm))


def decoder_spec(layers, H, F, KV, V, types):
    """A decoder-shaped chain: q|k|v read h, o reads q's output, gate|up read
    o's, down reads gate's, the next layer reads down's, the head reads the
    last down.  types: (t_q, t_k, t_v, t_o, t_gate, t_up, t_down, t_head)."""
    tq, tk, tv, to, tg, tu, td, th = types
    spec, h, st = [], "h", 0
    for L in range(layers):
        spec += [("q%d" % L, tq, H, H, h, st), ("k%d" % L, tk, KV, H, h, st), ("v%d" % L, tv, KV, H, h, st)]
        spec += [("o%d" % L, to, H, H, "q%d" % L, st + 1)]
        spec += [("gate%d" % L, tg, F, H, "o%d" % L, st + 2), ("up%d" % L, tu, F, H, "o%d" % L, st + 2)]
        spec += [("down%d" % L, td, H, F, "gate%d" % L, st + 3)]
        h, st = "down%d" % L, st + 4
    spec += [("head", th, V, H, h, st)]
    return spec


@pytest.mark.parametrize("types", [
    (G.Q4_K, G.Q4_K, G.Q6_K, G.Q4_K, G.Q4_K, G.Q4_K, G.Q6_K, G.Q6_K),     # Q4_K_M-style mix
    (G.Q5_K, G.Q6_K, G.Q4_K, G.Q5_K, G.Q6_K, G.Q5_K, G.Q4_K, G.Q5_K),
])
def test_pass_decoder_chain_k_quants(types):
    """Three decoder layers (hidden 2048, ffn 6144 -- the down projection
    spans two row segments; Q6_K rows are 16-byte multiples from k = 2048)
    and a head, every stage reading the previous stage's output."""
    spec = decoder_spec(3, 2048, 6144, 256, 3000, types)
    net = Net(spec, {"h": G.gen_x(2048, 1, seed=5)[0]}, seed=100)
    say("pass decoder chain", [G.NAMES[t] for t in types], len(spec), "GEMVs")
    net.run()
    net.verify("chain")


@pytest.mark.parametrize("t", [G.Q4_0, G.Q8_0, G.Q5_0])
def test_pass_decoder_chain_32_element_types(t):
    """The same chain in one 32-element type (TinyLlama-like: hidden 2048,
    ffn 5632 -- two-plus row segments for the down projection)."""
    spec = decoder_spec(2, 2048, 5632, 256, 2000, (t,) * 8)
    net = Net(spec, {"h": G.gen_x(2048, 1, seed=6)[0]}, seed=200 + t)
    say("pass decoder chain", G.NAMES[t], len(spec), "GEMVs")
    net.run()
    net.verify("chain %s" % G.NAMES[t])


def test_pass_many_problems_several_launches():
    """40 stages of up to five problems of mixed types reading one x (so a
    stage launch carries up to three block types of the same lane-unit size,
    and the other types get launches of their own); every odd stage reads
    an output of the stage before (even stages read the input again, which
    keeps the values' growth bounded)."""
    spec, prev = [], "h"
    rng = np.random.default_rng(3)
    H = 2048
    for s in range(40):
        names = []
        for j in range(1 + s % 5):
            t = TYPES[(s + j) % 6]
            nm = "p%d_%d" % (s, j)
            spec.append((nm, t, H, H, prev if s % 2 else "h", s))
            names.append(nm)
        prev = names[int(rng.integers(0, len(names)))]
    net = Net(spec, {"h": G.gen_x(H, 1, seed=9)[0]}, seed=300)
    say("pass", len(spec), "GEMVs in 40 stages")
    net.run()
    net.verify("many")


@pytest.mark.parametrize("t", TYPES)
def test_pass_zero_weight_rows_and_independent_stage(t):
    """Zero / sparse / single-weight rows (tests/zero_rows.py) in a pass of
    independent GEMVs (distinct x per problem, as the weight-stream
    workloads draw them; the widest in a stage of its own, since the x of a
    stage share 16384 elements of LDS) and ragged row counts."""
    be = G.BLOCK_ELEMS[t]
    ks = [8 * be, 4096 if be == 256 else 2048, 14336 if be == 256 else 5632]
    probs, host = [], []
    for i, k in enumerate(ks):
        n = 37 + 50 * i
        w = Z.make_matrix(t, n, k, ["zero", "sparse", "single", "dense", "random"],
                          np.random.default_rng(7 * t + i))
        x = G.gen_x(k, 1, seed=60 + i)
        wd, xd, yd = upload(w), upload(x[0]), nan_out(n)
        probs.append((wd, t, n, k, xd, yd, i // 2))
        host.append((w, n, k, x, yd))
    q.gemv_pass(probs)
    torch.cuda.synchronize()
    for (w, n, k, x, yd) in host:
        ref, absum = oracle.gemv(t, w, n, k, x)
        check(yd.cpu().numpy(), ref[0], absum[0], "zero rows %s k=%d" % (G.NAMES[t], k))


def test_pass_matches_across_graph_replays():
    """The pass captured in a HIP graph gives the eager results on every
    replay, with eager work between the replays."""
    spec = decoder_spec(1, 2048, 6144, 256, 1000,
                        (G.Q4_K, G.Q4_K, G.Q6_K, G.Q4_K, G.Q4_K, G.Q4_K, G.Q6_K, G.Q6_K))
    net = Net(spec, {"h": G.gen_x(2048, 1, seed=8)[0]}, seed=400)
    probs = net.problems()
    table = q.pass_table(probs)
    q.gemv_pass(probs, table=table)
    torch.cuda.synchronize()
    eager = {nm: y.clone() for nm, y in net.y.items()}
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        q.gemv_pass(probs, table=table, stream=s.cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        q.gemv_pass(probs, table=table, stream=torch.cuda.current_stream().cuda_stream)
    for rep in range(4):
        for y in net.y.values():
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for nm, y in net.y.items():
            assert torch.equal(y, eager[nm]), (rep, nm)
        q.gemv(net.w["q0"], G.Q4_K, 2048, 2048, net.x["h"].view(1, -1))   # eager work between replays
        torch.cuda.synchronize()


def test_pass_stage_launch_matches_single_calls():
    """A mixed-type stage launch (two K-quant types sharing x) gives the same
    bits as one qmm_gemv call per problem: the same decode and summation
    order, only the waves are shared out differently."""
    k = 4096
    x = upload(G.gen_x(k, 1, seed=11)[0])
    specs = [(G.Q4_K, 4096), (G.Q4_K, 1024), (G.Q6_K, 1024), (G.Q5_K, 700)]
    probs, ws = [], []
    for i, (t, n) in enumerate(specs):
        w = upload(G.gen_weights(t, n, k, seed=12 + i))
        probs.append((w, t, n, k, x, nan_out(n), 0))
        ws.append(w)
    q.gemv_pass(probs)
    torch.cuda.synchronize()
    for (w, t, n, k_, xx, y, st) in probs:
        single = q.gemv(w, t, n, k, x.view(1, -1)).view(-1)
        assert torch.equal(y, single), G.NAMES[t]


def test_pass_stage_group_edges():
    """Stage launches at the edges of their wave-slot split: a group of the
    full eight problems with one- and three-row problems between large ones,
    a group of two rows (fewer rows than its byte share of the slots, so it
    is capped and the slots past the groups fall into the last group), and
    a one-row problem last; the same for the 32-element types.  Each output
    is checked against the oracle and against one qmm_gemv call of its own
    (same decode and summation order, so the same bits)."""
    spec = []
    k_groups = [(G.Q4_K, [1, 3, 700, 5, 2048, 17, 1, 900]), (G.Q6_K, [2]), (G.Q5_K, [1000, 1])]
    e_groups = [(G.Q8_0, [1]), (G.Q4_0, [5000, 3]), (G.Q5_0, [64, 7])]
    for st, (k, src, groups) in enumerate([(4096, "h4", k_groups), (2048, "h2", e_groups)]):
        for t, ns in groups:
            for j, n in enumerate(ns):
                spec.append(("%s_%d_%d" % (G.NAMES[t], st, j), t, n, k, src, st))
    net = Net(spec, {"h4": G.gen_x(4096, 1, seed=21)[0], "h2": G.gen_x(2048, 1, seed=22)[0]}, seed=300)
    say("pass stage group edges", len(spec), "GEMVs")
    net.run()
    net.verify("stage edges")
    for (nm, t, n, k, src, st) in spec:
        single = q.gemv(net.w[nm], t, n, k, net.x[src].view(1, -1)).view(-1)
        assert torch.equal(net.y[nm], single), nm


def test_pass_full_layer_llama3_8b_mix():
    """One decoder layer of the Q4_K_M-style mix at the Llama-3-8B shapes the
    benchmark pass runs (hidden 4096, ffn 14336, k/v 1024 rows; v and down
    Q6_K, the rest Q4_K), chained stage to stage through qmm_gemv_pass (so
    the stage launches have the benchmark's grids and slot splits), plus a
    ragged 2999-row Q6_K head; every output against the oracle."""
    types = (G.Q4_K, G.Q4_K, G.Q6_K, G.Q4_K, G.Q4_K, G.Q4_K, G.Q6_K, G.Q6_K)
    spec = decoder_spec(1, 4096, 14336, 1024, 2999, types)
    net = Net(spec, {"h": G.gen_x(4096, 1, seed=41)[0]}, seed=400)
    say("pass full layer", len(spec), "GEMVs")
    net.run()
    net.verify("full layer")
