#!/usr/bin/env python3
"""Benchmark of the quantized-weight matmul on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--secondary all|none|<name>[,<name>...]]

A step is one decode pass over the largest workload that fits one GPU: the
Llama-3-8B-shaped Q4_K_M-style mix at batch 1 -- 32 layers of (q, k, v, o,
gate, up, down) with v and down in Q6_K, plus the 128256 x 4096 Q6_K LM
head: 225 GEMVs, 4.88 GB of weights.  The pass runs through qmm_gemv_pass
in the decoder's stage order (q|k|v, o, gate|up, down per layer, then the
head; one launch per stage, every stage after the one before it), captured
as one HIP graph and replayed once per step.  Inputs are resident in HBM
before timing starts; 4.88 GB is far larger than the 256 MB last-level
cache, so every pass reads the weights from HBM.

Printed: one JSON line with the whole-pass throughput (GB/s of algorithmic
bytes), its fraction of the 8 TB/s HBM peak, decode-equivalent tokens/s, the
roofline of the dominant kernel (the mixed-type stage GEMV that runs q|k|v
and gate|up) from HIP-event timings of its launches, the CPU oracle on the
host (one thread and all cores, per workload), and secondary figures with
their own roofline blocks: the Q8_0 2048 x 2048 GEMV, the TinyLlama Q4_0 and
Llama-3-8B Q4_K passes, the 512-token prefill GEMMs (TFLOP/s against the
fp16 dense peak), the same mix at batch 4 and 8 with the skinny GEMM beside
it, the 5-bit types, the embedding gather, the KV-cache codec and the
dequant-only kernel.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import qmm_inputs as G  # noqa: E402

METRIC = "quantized GEMV HBM GB/s (% of peak) + decode tok/s equiv; prefill GEMM TFLOP/s"
HBM_PEAK_GBS = 8000.0
FP16_PEAK_TFLOPS = 2500.0

# HBM bytes per launch of the dominant kernel from two rocprofv3 --pmc runs
# (FETCH_SIZE, then WRITE_SIZE, summed over the launches of the headline
# command and divided by them), each scaled by what the same counter reads
# for a plain 256 MiB device copy (reads x2.0, writes x1.0).  They describe
# the kernel sources they were taken on (SHA-256 prefix of the files in
# TRAFFIC_SOURCES): when the sources change, the line reports null until the
# counters are taken again.
# Taken with gemv3s_kernel<64, 8> over the 64 launches of one pass (256
# dispatches): FETCH_SIZE 20001.9 KiB x 2.0 + WRITE_SIZE 114.7 KiB x 1.0 per
# launch (profiles/gemv3s_stage_decode_pass_q4_k_m_mix.md).
TRAFFIC = {"sources_sha16": "b2ddcd09ae50d430", "bytes_per_launch": 41128074}
TRAFFIC_SOURCES = ("dequant_matmul_amd/csrc/qmm_gemv.hip", "dequant_matmul_amd/csrc/qmm_gemv_unit.h",
                   "dequant_matmul_amd/csrc/qmm_device.h")
SECONDARIES = ("q8_0", "tinyllama", "q4_k", "prefill", "mix_batch", "q5", "embed", "kv", "dequant")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sources_sha16():
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--secondary", default="all",
                   help="comma list of secondary workloads to run after the primary line's (all, none, or any of "
                        + ", ".join(SECONDARIES) + ")")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=2.0,
                   help="target CPU time of each oracle sample (per workload and thread count)")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB 10 times (reference for HBM byte counters)")
    p.add_argument("--reference-bw", action="store_true",
                   help="only time plain device fills, reads and copies (torch kernels) of 16 MB and 235 MB")
    p.add_argument("--dominant-only", action="store_true",
                   help="only replay the dominant kernel's launches of the headline pass (for counter runs)")
    a = p.parse_args()
    a.secondary = [s for s in a.secondary.split(",") if s] if a.secondary not in ("all", "none") else (
        list(SECONDARIES) if a.secondary == "all" else [])
    for s in a.secondary:
        if s not in SECONDARIES:
            p.error("unknown secondary %r" % s)
    return a


# ----------------------------------------------------------------- helpers --

class Problem:
    """One GEMV (or GEMM) with its device buffers and byte/flop counts."""

    def __init__(self, torch, name, t, n, k, w_dev, x_dev, y_dev, kind="gemv"):
        self.name, self.t, self.n, self.k, self.kind = name, t, n, k, kind
        self.w, self.x, self.y = w_dev, x_dev, y_dev
        self.batch = x_dev.shape[0]
        wbytes = n * G.row_bytes(t, k)
        if kind == "gemv":
            # algorithmic bytes: weights + x + y (x re-reads from cache not counted)
            self.bytes = wbytes + 4 * self.batch * k + 4 * self.batch * n
        else:
            self.bytes = wbytes + 2 * self.batch * k + 4 * self.batch * n
        self.flops = 2 * self.batch * n * k
        self.wbytes = wbytes

    def launch(self, q, stream):
        if self.kind == "gemv":
            st = q.lib.qmm_gemv(self.t, self.w.data_ptr(), self.n, self.k, self.x.data_ptr(), self.batch,
                                self.y.data_ptr(), stream)
        else:
            st = q.lib.qmm_gemm_prefill(self.t, self.w.data_ptr(), self.n, self.k, self.x.data_ptr(),
                                        self.batch, self.y.data_ptr(), stream)
        if st != 0:
            raise RuntimeError("%s %s: %s" % (self.kind, self.name, q.status_str(st)))


class BatchPass:
    """A decode pass at batch B > 1 in the decoder's stage order, the
    problems of a stage reading one x [B, k] (q / k / v, gate / up), as in
    Pass: each stage's problems of one block type go to one qmm_gemv_multi
    call (at batch 3..8 of the K-quants one matrix-core launch over all
    their tiles), a lone problem to qmm_gemv."""

    def __init__(self, torch, q, cfg, weights, batch, dev):
        import ctypes
        self.units, self.probs = [], []
        xs, groups = {}, {}
        for i, (name, t, n, k, w) in enumerate(weights):
            st = G.decode_stage(name)
            if st not in xs:
                xs[st] = torch.from_numpy(G.gen_x(k, batch, G.x_seed(cfg, i))).to(dev)
            y = torch.empty((batch, n), dtype=torch.float32, device=dev)
            p = Problem(torch, name, t, n, k, w, xs[st], y)
            self.probs.append(p)
            groups.setdefault((st, t), []).append(p)
        for (st, t), ps in sorted(groups.items(), key=lambda e: e[0][0]):
            if len(ps) == 1:
                self.units.append(ps[0])
                continue
            m = len(ps)
            self.units.append(("multi", t, m, ps[0].k, batch,
                               (ctypes.c_void_p * m)(*[p.w.data_ptr() for p in ps]),
                               (ctypes.c_int64 * m)(*[p.n for p in ps]),
                               (ctypes.c_void_p * m)(*[p.x.data_ptr() for p in ps]),
                               (ctypes.c_void_p * m)(*[p.y.data_ptr() for p in ps])))
        self.wbytes = sum(p.wbytes for p in self.probs)
        self.bytes = self.wbytes + sum(4 * x.numel() for x in xs.values()) + sum(4 * batch * p.n for p in self.probs)
        self.launches = len(self.units)

    def launch(self, q, stream):
        for u in self.units:
            if isinstance(u, Problem):
                u.launch(q, stream)
                continue
            _, t, m, k, batch, wp, nn, xp, yp = u
            st = q.lib.qmm_gemv_multi(t, m, wp, nn, k, xp, batch, yp, stream)
            if st != 0:
                raise RuntimeError("qmm_gemv_multi: %s" % q.status_str(st))


class Embed:
    """One embedding gather (qmm_embed / qmm_embed_f16) with its buffers."""

    def __init__(self, torch, name, t, vocab, k, table, ids, out):
        self.name, self.t, self.vocab, self.k = name, t, vocab, k
        self.table, self.ids, self.out = table, ids, out
        self.seq = ids.shape[0]
        self.f16 = out.dtype == torch.float16
        # algorithmic bytes: ids + the rows read + the output written
        self.bytes = 4 * self.seq + self.seq * G.row_bytes(t, k) + self.seq * k * (2 if self.f16 else 4)

    def launch(self, q, stream):
        f = q.lib.qmm_embed_f16 if self.f16 else q.lib.qmm_embed
        st = f(self.t, self.table.data_ptr(), self.vocab, self.k, self.ids.data_ptr(), self.seq,
               self.out.data_ptr(), stream)
        if st != 0:
            raise RuntimeError("embed %s: %s" % (self.name, q.status_str(st)))


class Codec:
    """One KV-cache codec call: encode (qmm_quantize_f16, fp16 -> blocks) or
    decode (qmm_dequant_f16, blocks -> fp16)."""

    def __init__(self, name, t, n, k, x, blocks, back, encode):
        self.name, self.t, self.n, self.k = name, t, n, k
        self.x, self.blocks, self.back, self.encode = x, blocks, back, encode
        # algorithmic bytes: fp16 values on one side, the blocks on the other
        self.bytes = 2 * n * k + n * G.row_bytes(t, k)

    def launch(self, q, stream):
        if self.encode:
            st = q.lib.qmm_quantize_f16(self.t, self.x.data_ptr(), self.n, self.k, self.blocks.data_ptr(), stream)
        else:
            st = q.lib.qmm_dequant_f16(self.t, self.blocks.data_ptr(), self.n, self.k, self.back.data_ptr(), stream)
        if st != 0:
            raise RuntimeError("codec %s: %s" % (self.name, q.status_str(st)))


class Dequant:
    """One dequant-only call (qmm_dequant or qmm_dequant_f16)."""

    def __init__(self, name, t, n, k, w, out, f16):
        self.name, self.t, self.n, self.k, self.w, self.out, self.f16 = name, t, n, k, w, out, f16
        # algorithmic bytes: the blocks read + the dense output written
        self.bytes = n * G.row_bytes(t, k) + n * k * (2 if f16 else 4)

    def launch(self, q, stream):
        f = q.lib.qmm_dequant_f16 if self.f16 else q.lib.qmm_dequant
        st = f(self.t, self.w.data_ptr(), self.n, self.k, self.out.data_ptr(), stream)
        if st != 0:
            raise RuntimeError("dequant %s: %s" % (self.name, q.status_str(st)))


class Pass:
    """A decode pass (qmm_gemv_pass) over a workload's matrices at batch 1, in
    the decoder's stage order.  share_x: the problems of a stage read one x
    (q / k / v the normalized hidden state, gate / up the normalized state
    after attention), as in a decoder; else each GEMV has its own x."""

    def __init__(self, torch, q, cfg, weights, dev, share_x=True, only=None):
        self.q = q
        self.probs, self.plist = [], []
        xs = {}
        for i, (name, t, n, k, w) in enumerate(weights):
            st = G.decode_stage(name)
            if only is not None and not only(name):
                continue
            key = st if share_x else i
            if key not in xs:
                xs[key] = torch.from_numpy(G.gen_x(k, 1, G.x_seed(cfg, i))).to(dev)
            x = xs[key]
            y = torch.empty((1, n), dtype=torch.float32, device=dev)
            self.probs.append(Problem(torch, name, t, n, k, w, x, y))
            self.plist.append((w, t, n, k, x.view(-1), y.view(-1), st))
        self.table = q.pass_table(self.plist)
        # algorithmic bytes: weights, each distinct x once, every y
        self.wbytes = sum(p.wbytes for p in self.probs)
        self.bytes = self.wbytes + sum(4 * x.numel() for x in xs.values()) + sum(4 * p.n for p in self.probs)
        self.stages = len({e[6] for e in self.plist})

    def launch(self, q, stream):
        q.gemv_pass(self.plist, table=self.table, stream=stream)


def capture(torch, q, work):
    """One HIP graph of `work` (a list of objects with .launch(q, stream), or
    one such object)."""
    work = work if isinstance(work, list) else [work]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for p in work:                                   # warm (outside capture)
            p.launch(q, torch.cuda.current_stream().cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for p in work:
            p.launch(q, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, steps, warmup, min_warm_s=0.03):
    """Event time per replay: the requested warm-up replays, continued until
    at least min_warm_s of replays have run (sustained load takes tens of
    milliseconds to reach steady clocks), then `steps` timed ones between
    two events on the stream the graph runs on."""
    t0 = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t0 < min_warm_s:
        g.replay()
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / steps


def roofline(achieved, peak, unit, bound, **extra):
    d = {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4)}
    d.update(extra)
    return d


def build_weights(torch, cfg, dev="cuda:0", keep_host=False):
    out, host = [], []
    for (name, t, n, k, seed) in G.workload(cfg):
        w = G.gen_weights(t, n, k, seed)
        out.append((name, t, n, k, torch.from_numpy(w).to(dev)))
        if keep_host:
            host.append(w)
    return (out, host) if keep_host else out


def make_gemvs(torch, cfg, weights, batch, dev="cuda:0"):
    probs = []
    for i, (name, t, n, k, w) in enumerate(weights):
        x = torch.from_numpy(G.gen_x(k, batch, G.x_seed(cfg, i))).to(dev)
        y = torch.empty((batch, n), dtype=torch.float32, device=dev)
        probs.append(Problem(torch, name, t, n, k, w, x, y))
    return probs


# ------------------------------------------------------------ CPU baseline --

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def _cpu_rate(items, target_s):
    """Run items [(fn, work)] in turn until target_s of time is spent (at
    least one); returns (work per second, items run, seconds)."""
    done, used, ran = 0.0, 0.0, 0
    i = 0
    while used < target_s or ran == 0:
        fn, work = items[i % len(items)]
        t0 = time.perf_counter()
        fn()
        used += time.perf_counter() - t0
        done += work
        ran += 1
        i += 1
    return done / used, ran, used


def cpu_baselines(target_s, mix_host=None, head_s=10.0):
    """The oracle (plain C, exact fp32 dequant then fp64 dot products, OpenMP
    over rows) on the host, on 1 thread and on every core, over bounded
    samples of each workload: the same matrices (same seeds) as the GPU runs,
    taken in chunks of rows (every matrix of a layer in turn, then the next
    chunk) until about target_s seconds are spent (head_s for the headline
    workload, the mix at batch 1); for the prefill GEMM, rows of one
    512-token chunk, one at a time."""
    import oracle
    allc = oracle.max_threads()

    def gemv_items(mats, chunk=256):
        """[(fn, bytes)]: row chunks of each matrix, interleaved."""
        per = []
        for (t, n, k, w, x) in mats:
            rb = G.row_bytes(t, k)
            w2 = w.reshape(n, rb)
            per.append([((lambda t=t, k=k, x=x, ww=np.ascontiguousarray(w2[r:r + chunk]), nr=min(chunk, n - r):
                          oracle.gemv(t, ww, nr, k, x)), min(chunk, n - r) * rb + 4 * k + 4 * min(chunk, n - r))
                        for r in range(0, n, chunk)])
        items = []
        for i in range(max(len(p) for p in per)):
            items += [p[i] for p in per if i < len(p)]
        return items

    def layer0(cfg):
        mats = []
        for i, (name, t, n, k, seed) in enumerate(G.workload(cfg)):
            if "." in name and not name.startswith("l0."):
                continue
            mats.append((t, n, k, G.gen_weights(t, n, k, seed), G.gen_x(k, 1, G.x_seed(cfg, i))))
        return mats

    work = {
        "q8_0_2048": ("the 2048 x 2048 Q8_0 GEMV", layer0(1)),
        "tinyllama_q4_0": ("the Q4_0 stream's first layer (7 GEMVs)", layer0(2)),
        "llama3_8b_q4_k": ("the Q4_K set's first layer (7 GEMVs)", layer0(3)),
    }
    if mix_host is not None:
        work["q4_k_m_mix_b1"] = ("the mix's first layer (7 GEMVs) and the LM head", mix_host)
    rates = {}
    for name, (what, mats) in work.items():
        items = gemv_items(mats)
        for nt in (1, allc):
            oracle.set_threads(nt)
            rate, ran, used = _cpu_rate(items if nt > 1 else items[:max(1, len(items) // 4)],
                                        head_s if name == "q4_k_m_mix_b1" else target_s)
            rates.setdefault(name, {})["1_thread" if nt == 1 else "all_cores"] = {
                "value": round(rate / 1e9, 4), "unit": "GB/s", "threads": nt,
                "sample": "row chunks of 256 of %s, in turn: %d chunks, %.1f s" % (what, ran, used)}
    m = G.PREFILL_M
    for name, t, n, k, seed in G.workload(4):
        w = G.gen_weights(t, n, k, seed)
        X = G.gen_x_f16(m, k, G.x_seed(4, 0))
        items = [((lambda r=r: oracle.gemm(t, w, n, k, X, rows=[r])), 2.0 * n * k) for r in range(0, m, 37)]
        for nt in (1, allc):
            oracle.set_threads(nt)
            rate, ran, used = _cpu_rate(items, target_s)
            rates.setdefault("prefill_" + name, {})["1_thread" if nt == 1 else "all_cores"] = {
                "value": round(rate / 1e9, 3), "unit": "GFLOP/s", "threads": nt,
                "sample": "%d rows of one 512 x %d x %d chunk, one at a time, %.1f s" % (ran, n, k, used)}
    oracle.set_threads(allc)
    return {"cpu_model": cpu_model(), "cores": allc, "configs": rates}


# -------------------------------------------------------------- secondaries --

def sec_q8_0(torch, q, steps, warmup, dev):
    """Q8_0 2048x2048: rotate over 256 copies (1.14 GB) so caches cannot serve
    it; also the cache-resident single-call time."""
    n = k = 2048
    w0 = torch.from_numpy(G.gen_weights(G.Q8_0, n, k, 1000)).to(dev)
    x = torch.from_numpy(G.gen_x(k, 1, G.x_seed(1, 0))).to(dev)
    copies = [w0.clone() for _ in range(256)]
    y = torch.empty((1, n), dtype=torch.float32, device=dev)
    probs = [Problem(torch, "w%d" % i, G.Q8_0, n, k, c, x, y) for i, c in enumerate(copies)]
    t = time_graph(torch, capture(torch, q, probs), max(2, steps // 4), 2) / len(probs)
    hot = [Problem(torch, "hot", G.Q8_0, n, k, w0, x, y)] * 256
    th = time_graph(torch, capture(torch, q, hot), max(2, steps // 4), 2) / 256
    b = probs[0].bytes
    del copies, probs
    return {"workload": "Q8_0 2048x2048 GEMV, batch 1, over 256 rotating copies (1.14 GB)",
            "us_per_gemv": round(t * 1e6, 3), "GB_s": round(b / t / 1e9, 1),
            "hot_us_per_gemv_cache_resident": round(th * 1e6, 3),
            "roofline": roofline(b / t / 1e9, HBM_PEAK_GBS, "GB/s", "hbm", kernel="gemv3_kernel<Q8_0>",
                                 bytes_per_launch=b, avg_launch_us=round(t * 1e6, 3))}


def sec_pass(torch, q, cfg, steps, warmup, dev, label, weights=None, single_launch_graph=False):
    wts = weights if weights is not None else build_weights(torch, cfg, dev)
    P = Pass(torch, q, cfg, wts, dev)
    tp = time_graph(torch, capture(torch, q, P), steps, warmup)
    out = {"workload": label, "gemvs": len(P.probs), "stages": P.stages, "batch": 1,
           "weight_bytes": P.wbytes, "algorithmic_bytes": P.bytes, "ms_per_pass": round(tp * 1e3, 4),
           "GB_s": round(P.bytes / tp / 1e9, 1), "decode_tok_s": round(1.0 / tp, 1),
           "roofline": roofline(P.bytes / tp / 1e9, HBM_PEAK_GBS, "GB/s", "hbm",
                                kernel="whole pass (qmm_gemv_pass, one launch per stage and x)")}
    if single_launch_graph:
        # the same GEMVs as one qmm_gemv launch each (one graph), for comparison
        ts = time_graph(torch, capture(torch, q, P.probs), steps, warmup)
        out["single_launches_ms_per_pass"] = round(ts * 1e3, 4)
        out["single_launches_GB_s"] = round(P.bytes / ts / 1e9, 1)
    del P
    if weights is None:
        del wts
    torch.cuda.empty_cache()
    return out


def sec_prefill(torch, q, steps, warmup, dev, cfg=4):
    res = {}
    m = G.PREFILL_M
    for name, t, n, k, seed in G.workload(cfg):
        w = torch.from_numpy(G.gen_weights(t, n, k, seed)).to(dev)
        probs = []
        for c in range(G.PREFILL_CHUNKS):
            X = torch.from_numpy(G.gen_x_f16(m, k, G.x_seed(cfg, 10 * c + len(res)))).to(dev)
            Y = torch.empty((m, n), dtype=torch.float32, device=dev)
            probs.append(Problem(torch, "%s.c%d" % (name, c), t, n, k, w, X, Y, kind="gemm"))
        tg = time_graph(torch, capture(torch, q, probs), steps, warmup)
        flops = sum(p.flops for p in probs)
        tf = flops / tg / 1e12
        res[name] = {"shape": "4 x (%d x %d x %d)" % (m, n, k), "ms_4_chunks": round(tg * 1e3, 4),
                     "us_per_chunk": round(tg * 1e6 / len(probs), 2), "TFLOP_s": round(tf, 1),
                     "roofline": roofline(tf, FP16_PEAK_TFLOPS, "TFLOP/s", "mfma", kernel="gemm_kernel",
                                          flops_per_launch=flops // len(probs),
                                          avg_launch_us=round(tg * 1e6 / len(probs), 2))}
        del probs, w
    torch.cuda.empty_cache()
    return res


def sec_mix_batch(torch, q, steps, warmup, dev, weights):
    """The Q4_K_M-style mix at batch 4 and 8 (x fp32 [B, k], one x per stage
    as in the batch-1 pass: qmm_gemv_multi per stage and block type), and the
    same pass as a skinny GEMM (fp16 X, M = B, one call per matrix)."""
    res = {}
    for batch in (4, 8):
        bp = BatchPass(torch, q, 5, weights, batch, dev)
        probs = bp.probs
        tot = bp.bytes
        tg = time_graph(torch, capture(torch, q, bp), max(3, steps // 2), 2)
        gp = [Problem(torch, p.name, p.t, p.n, p.k, p.w, torch.from_numpy(G.gen_x_f16(batch, p.k, 77)).to(dev),
                      p.y, kind="gemm") for p in probs]
        tgg = time_graph(torch, capture(torch, q, gp), max(3, steps // 2), 2)
        res["b%d" % batch] = {
            "workload": "Q4_K_M-style mix, 225 GEMVs, batch %d" % batch, "ms_per_pass": round(tg * 1e3, 4),
            "GB_s": round(tot / tg / 1e9, 1), "decode_tok_s": round(batch / tg, 1),
            "skinny_gemm_ms_per_pass": round(tgg * 1e3, 4), "skinny_gemm_tok_s": round(batch / tgg, 1),
            "launches_per_pass": bp.launches,
            "roofline": roofline(tot / tg / 1e9, HBM_PEAK_GBS, "GB/s", "hbm",
                                 kernel="whole pass (batch GEMV, qmm_gemv_multi per stage and type)")}
        del probs, gp, bp
        torch.cuda.empty_cache()
    return res


def sec_q5(torch, q, steps, warmup, dev):
    res = {"llama3_8b_q5_k": sec_pass(torch, q, 6, steps, warmup, dev,
                                      "Llama-3-8B-shaped Q5_K decode pass, 224 GEMVs, batch 1"),
           "tinyllama_q5_0": sec_pass(torch, q, 7, steps, warmup, dev,
                                      "TinyLlama-shaped Q5_0 decode pass, 154 GEMVs, batch 1"),
           "prefill_512_q5": sec_prefill(torch, q, steps, warmup, dev, cfg=8)}
    return res


def sec_embed(torch, q, steps, warmup, dev, rotate=32):
    """Embedding gathers from the Llama 3.2 1B Q8_0 and Llama-3-8B Q4_K token
    tables: one decode token and one 512-token chunk, fp32 and fp16 outputs;
    each graph issues `rotate` gathers with distinct ids and outputs."""
    res = {}
    for name, t, vocab, k, seed in G.workload(9):
        table = torch.from_numpy(G.gen_weights(t, vocab, k, seed)).to(dev)
        for seq in (1, 512):
            for dt, dn in ((torch.float32, "f32"), (torch.float16, "f16")):
                probs = []
                for r in range(rotate):
                    ids = torch.from_numpy(G.gen_ids(vocab, seq, G.x_seed(9, 1000 * r + seq))).to(dev)
                    probs.append(Embed(torch, name, t, vocab, k, table, ids,
                                       torch.empty((seq, k), dtype=dt, device=dev)))
                g = capture(torch, q, probs)
                tg = time_graph(torch, g, steps, warmup) / rotate
                b = probs[0].bytes
                res["%s_seq%d_%s" % (name, seq, dn)] = {
                    "table": "%d x %d %s" % (vocab, k, G.NAMES[t]), "tokens": seq, "out": dn,
                    "us_per_call": round(tg * 1e6, 3), "GB_s": round(b / tg / 1e9, 1),
                    "pct_hbm_peak": round(100 * b / tg / 1e9 / HBM_PEAK_GBS, 2)}
                del g, probs
        del table
        torch.cuda.empty_cache()
    return res


def sec_kv(torch, q, steps, warmup, dev):
    """KV-cache codec on the K rows of one Llama-3-8B layer (1024 fp16 values
    per token): encode / decode one new token, a 512-token chunk and an
    8192-token context; the large cases rotate over enough buffers
    (> 256 MB) that the last-level cache cannot hold them."""
    res = {}
    for name, t, n_ctx, k, seed in G.workload(10):
        for n in (1, 512, n_ctx):
            rotate = 16 if n == n_ctx else 32
            probs_e, probs_d = [], []
            for r in range(rotate):
                x = torch.from_numpy(G.gen_x_f16(n, k, seed + 17 * r)).to(dev)
                blocks = torch.empty((n, G.row_bytes(t, k)), dtype=torch.uint8, device=dev)
                back = torch.empty((n, k), dtype=torch.float16, device=dev)
                probs_e.append(Codec(name, t, n, k, x, blocks, back, True))
                probs_d.append(Codec(name, t, n, k, x, blocks, back, False))
            for kind, probs in (("encode", probs_e), ("decode", probs_d)):
                g = capture(torch, q, probs)
                tg = time_graph(torch, g, steps, warmup) / rotate
                b = probs[0].bytes
                res["%s_%s_%d" % (name, kind, n)] = {
                    "rows": "%d x %d" % (n, k), "us_per_call": round(tg * 1e6, 3), "GB_s": round(b / tg / 1e9, 1),
                    "pct_hbm_peak": round(100 * b / tg / 1e9 / HBM_PEAK_GBS, 2)}
                del g
            del probs_e, probs_d
            torch.cuda.empty_cache()
    return res


def sec_dequant(torch, q, steps, warmup, dev):
    """Dequant-only: the Q8_0 2048 x 2048 matrix and a Q4_K 14336 x 4096
    gate projection to fp32 and fp16, rotating over enough weight copies and
    outputs (> 256 MB per graph) that the last-level cache cannot hold them."""
    res = {}
    for name, t, n, k, seed in (("q8_0_2048", G.Q8_0, 2048, 2048, 1000), ("q4_k_gate", G.Q4_K, 14336, 4096, 3004)):
        w0 = torch.from_numpy(G.gen_weights(t, n, k, seed)).to(dev)
        for f16, dn in ((False, "f32"), (True, "f16")):
            per = n * G.row_bytes(t, k) + n * k * (2 if f16 else 4)
            copies = max(2, int(400e6 // per) + 1)
            ws = [w0.clone() for _ in range(copies)]
            probs = [Dequant(name, t, n, k, ws[i], torch.empty((n, k), dtype=torch.float16 if f16 else torch.float32,
                                                                device=dev), f16) for i in range(copies)]
            g = capture(torch, q, probs)
            tg = time_graph(torch, g, max(2, steps // 2), warmup) / copies
            b = probs[0].bytes
            res["%s_%s" % (name, dn)] = {"shape": "%d x %d %s" % (n, k, G.NAMES[t]), "out": dn, "copies": copies,
                                         "us_per_call": round(tg * 1e6, 3), "GB_s": round(b / tg / 1e9, 1),
                                         "pct_hbm_peak": round(100 * b / tg / 1e9 / HBM_PEAK_GBS, 2)}
            del g, probs, ws
            torch.cuda.empty_cache()
        del w0
    return res


def reference_bw(torch, dev):
    """Plain fill (write only), read (a sum over the buffer: reads it once
    and writes one number) and copy (read + write) of fp32 buffers, each
    rotating over more than 400 MB, timed with events after a warm-up."""
    res = {}
    for label, nbytes in (("235MB", 14336 * 4096 * 4), ("16MB", 2048 * 2048 * 4)):
        n = nbytes // 4
        cnt = max(2, int(400e6 // nbytes) + 1)
        dst = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(cnt)]
        src = [torch.ones(n, dtype=torch.float32, device=dev) for _ in range(cnt)]
        sums = torch.empty(cnt, dtype=torch.float32, device=dev)
        for name, moved in (("fill", nbytes), ("read", nbytes), ("copy", 2 * nbytes)):
            def once():
                for i in range(cnt):
                    if name == "fill":
                        dst[i].fill_(1.0)
                    elif name == "read":
                        torch.sum(src[i], dim=0, out=sums[i])
                    else:
                        dst[i].copy_(src[i])
            for _ in range(3):
                once()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(5):
                once()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / 1e3 / (5 * cnt)
            res["%s_%s" % (name, label)] = {"us": round(t * 1e6, 2), "GB_s": round(moved / t / 1e9, 1)}
        del dst, src, sums
        torch.cuda.empty_cache()
    return res




# -------------------------------------------------------------------- main --

def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(GEMV rows / GEMM columns would shard across GPUs, one shard per GPU)", file=sys.stderr)
        sys.exit(2)
    import torch
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        nb = args.calibrate_copy << 20
        a = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty(nb, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        for _ in range(10):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": nb, "bytes_written": nb, "launches": 10}))
        return
    if args.reference_bw:
        print(json.dumps(reference_bw(torch, dev)))
        return
    import dequant_matmul_amd as q
    log("device:", torch.cuda.get_device_name(0), "| lib:", q.version())

    # primary: the Q4_K_M-style mix decode pass, batch 1
    log("generating the Q4_K_M-style mix (225 GEMVs, 4.88 GB)")
    weights, host = build_weights(torch, 5, dev, keep_host=True)
    mix_host = [(t, n, k, host[i], G.gen_x(k, 1, G.x_seed(5, i)))
                for i, (name, t, n, k, _) in enumerate(weights) if name.startswith("l0.") or name == "lm_head"]
    del host
    P = Pass(torch, q, 5, weights, dev)
    # the dominant kernel: the mixed-type stage GEMV of the q|k|v and gate|up
    # stages (64 launches per pass), timed alone as a graph of its launches
    D = Pass(torch, q, 5, weights, dev, only=lambda nm: nm.split(".")[-1] in ("q", "k", "v", "gate", "up"))
    if args.dominant_only:
        g = capture(torch, q, D)
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        print(json.dumps({"dominant_only": True, "launches_per_replay": D.stages, "replays": args.steps}))
        return
    g = capture(torch, q, P)
    log("timing %d graph replays after %d warmup" % (args.steps, args.warmup))
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / args.steps
    ev_step_s = ev0.elapsed_time(ev1) * 1e-3 / args.steps
    singles = []
    for _ in range(20):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        singles.append(a.elapsed_time(b))
    singles.sort()
    del g
    gd = capture(torch, q, D)
    td = time_graph(torch, gd, args.steps, args.warmup)
    del gd
    avg_launch = td / D.stages
    achieved = (D.bytes / D.stages) / avg_launch / 1e9
    sha = sources_sha16()
    traffic = TRAFFIC["bytes_per_launch"] if TRAFFIC["sources_sha16"] == sha else None
    value = P.bytes / step_s / 1e9
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "Q4_K_M-style mix decode pass, Llama-3-8B shapes: 32 layers x (q 4096x4096, "
                               "k/v 1024x4096, o 4096x4096, gate/up 14336x4096, down 4096x14336; v and down "
                               "Q6_K, the rest Q4_K) + LM head 128256x4096 Q6_K = 225 GEMVs at batch 1, "
                               "stage by stage (q|k|v, o, gate|up, down; then the head), one HIP graph per pass",
                   "gemvs": len(P.probs), "stages": P.stages, "batch": 1, "weight_bytes": P.wbytes,
                   "algorithmic_bytes": P.bytes},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "decode_tok_s": round(1.0 / step_s, 1),
        "event_ms_per_step": round(ev_step_s * 1e3, 4),
        "single_pass_ms": {"median": round(0.5 * (singles[9] + singles[10]), 4), "min": round(singles[0], 4),
                           "max": round(singles[-1], 4), "passes": len(singles)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "gemv3s_kernel<64, 8>: the mixed-type stage GEMV of the q|k|v and gate|up stages "
                               "(64 launches per pass)",
                     "avg_launch_us": round(avg_launch * 1e6, 3),
                     "bytes_per_launch": round(D.bytes / D.stages), "kernel_sources_sha16": sha},
    }
    del D

    if not args.no_cpu_baseline:
        log("CPU oracle baselines (~%.0f s per sample)" % args.cpu_seconds)
        cb = cpu_baselines(args.cpu_seconds, mix_host)
        head = cb["configs"]["q4_k_m_mix_b1"]["all_cores"]
        line["cpu_baseline"] = {"value": head["value"], "unit": "GB/s", "cores": head["threads"], "kind": "oracle",
                                "sample": head["sample"], "cpu_model": cb["cpu_model"],
                                "one_thread": cb["configs"]["q4_k_m_mix_b1"]["1_thread"],
                                "per_workload": cb["configs"]}
    del mix_host

    sec = {}
    want = set(args.secondary)
    if "mix_batch" in want:
        log("secondary: the mix at batch 4 and 8")
        sec["q4_k_m_mix"] = sec_mix_batch(torch, q, args.steps, args.warmup, dev, weights)
    del P, weights
    torch.cuda.empty_cache()
    if "q8_0" in want:
        log("secondary: Q8_0 single matrix")
        sec["q8_0_2048"] = sec_q8_0(torch, q, args.steps, args.warmup, dev)
    if "tinyllama" in want:
        log("secondary: TinyLlama Q4_0 pass")
        sec["tinyllama_q4_0"] = sec_pass(torch, q, 2, args.steps, args.warmup, dev,
                                         "TinyLlama-shaped Q4_0 decode pass, 154 GEMVs, batch 1",
                                         single_launch_graph=True)
    if "q4_k" in want:
        log("secondary: Llama-3-8B Q4_K pass")
        sec["llama3_8b_q4_k"] = sec_pass(torch, q, 3, args.steps, args.warmup, dev,
                                         "Llama-3-8B-shaped Q4_K decode pass, 224 GEMVs, batch 1",
                                         single_launch_graph=True)
    if "prefill" in want:
        log("secondary: prefill GEMMs")
        sec["prefill_512"] = sec_prefill(torch, q, args.steps, args.warmup, dev)
    if "q5" in want:
        log("secondary: 5-bit types")
        sec["q5"] = sec_q5(torch, q, args.steps, args.warmup, dev)
    if "embed" in want:
        log("secondary: embedding gathers")
        sec["embed"] = sec_embed(torch, q, args.steps, args.warmup, dev)
    if "dequant" in want:
        log("secondary: dequant-only")
        sec["dequant"] = sec_dequant(torch, q, args.steps, args.warmup, dev)
    if "kv" in want:
        log("secondary: KV-cache codec")
        sec["kv_codec"] = sec_kv(torch, q, args.steps, args.warmup, dev)
    if sec:
        line["secondary"] = sec
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
