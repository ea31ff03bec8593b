#!/usr/bin/env python3
"""Benchmark of the quantized-weight matmul on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--secondary all|none|q8_0|q4_k|prefill|mix|q5|embed|kv|dequant]

A step is one decode pass over the TinyLlama-shaped Q4_0 weight stream:
22 layers x (q, k, v, o, gate, up, down) = 154 GEMVs at batch 1 on one
stream, each with a fresh fp32 activation, as one captured HIP graph (one
submission per token, no host synchronization inside the pass).  Inputs are
resident in HBM before timing starts.  The 545 MB stream is larger than the
256 MB last-level cache, so every pass reads the weights from HBM.

Printed: one JSON line with the whole-pass HBM throughput (GB/s), its fraction
of the 8 TB/s peak, the decode-equivalent tokens/s, the roofline of the
dominant kernel (the Q4_0 GEMV) from per-launch HIP-event timings, the CPU
oracle timed on a bounded sample of the same workload, and secondary figures
for the other workloads (Q8_0 single matrix, Llama-3-8B Q4_K set, 512-token
prefill GEMMs, Q4_K_M-style mix with a Q6_K LM head at batch 1/4/8, the
same shapes in the 5-bit types Q5_K / Q5_0, the quantized embedding
gather for one decode token and a 512-token chunk, and the Q8_0 / Q4_0
KV-cache codec: encoding and decoding K rows of one Llama-3-8B layer, and
the dequant-only kernel to fp32 / fp16).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import qmm_inputs as G  # noqa: E402

METRIC = "quantized GEMV HBM GB/s (% of peak) + decode tok/s equiv; prefill GEMM TFLOP/s"
HBM_PEAK_GBS = 8000.0
FP16_PEAK_TFLOPS = 2500.0
# HBM bytes per launch of the dominant kernel (the batch-1 Q4_0 GEMV over the
# decode stream) from rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by what the
# same counters read for a plain 256 MiB device copy (reads x2.0, writes
# x1.0).  It describes the kernels it was measured on: set it to None when
# they change, until the counters are taken again.
TRAFFIC = 3759748   # bytes per launch, averaged over one pass (gemv3_kernel<0,1,8/16>, gemv1_kernel<0,1,...>)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--secondary", choices=["all", "none", "q8_0", "q4_k", "prefill", "mix", "q5", "embed", "kv", "dequant"], default="all",
                   help="which secondary workloads to run after the primary line's (all by default)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="target length of the CPU oracle sample")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB 10 times (reference for HBM byte counters)")
    p.add_argument("--reference-bw", action="store_true",
                   help="only time plain device fills and copies (torch kernels) of 16 MB and 235 MB, rotating over "
                        "more than 400 MB: reference bandwidths for the streaming kernels")
    return p.parse_args()


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
            self.flops = 2 * self.batch * n * k
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


class Group:
    """Several same-type, same-k batch-1 GEMVs issued as one qmm_gemv_multi
    call; share_x: all of them read the first one's activation (as q / k / v
    and gate / up read one normalized hidden state in a decoder layer)."""

    def __init__(self, probs, share_x=False):
        import ctypes
        self.probs = probs
        npb = len(probs)
        self.t, self.k, self.batch = probs[0].t, probs[0].k, probs[0].batch
        self.np = npb
        self.w = (ctypes.c_void_p * npb)(*[p.w.data_ptr() for p in probs])
        self.x = (ctypes.c_void_p * npb)(*[(probs[0] if share_x else p).x.data_ptr() for p in probs])
        self.y = (ctypes.c_void_p * npb)(*[p.y.data_ptr() for p in probs])
        self.n = (ctypes.c_int64 * npb)(*[p.n for p in probs])
        self.name = "+".join(p.name for p in probs)

    def launch(self, q, stream):
        st = q.lib.qmm_gemv_multi(self.t, self.np, self.w, self.n, self.k, self.x, self.batch, self.y, stream)
        if st != 0:
            raise RuntimeError("gemv_multi %s: %s" % (self.name, q.status_str(st)))


def group_layers(probs, fuse, share_x=False):
    """Split a 7-projections-per-layer list into launch groups: fuse = set of
    projection-name tuples issued together (e.g. ("gate", "up"))."""
    out = []
    for L in range(0, len(probs), 7):
        layer = {p.name.split(".")[-1]: p for p in probs[L:L + 7]}
        done = set()
        for nm in ("q", "k", "v", "o", "gate", "up", "down"):
            if nm in done:
                continue
            grp = next((g for g in fuse if nm in g), (nm,))
            out.append(Group([layer[g] for g in grp], share_x) if len(grp) > 1 else layer[nm])
            done.update(grp)
    return out


def build_weights(torch, cfg, dev="cuda:0"):
    return [(name, t, n, k, torch.from_numpy(G.gen_weights(t, n, k, seed)).to(dev))
            for (name, t, n, k, seed) in G.workload(cfg)]


def make_gemvs(torch, cfg, weights, batch, dev="cuda:0"):
    probs = []
    for i, (name, t, n, k, w) in enumerate(weights):
        x = torch.from_numpy(G.gen_x(k, batch, G.x_seed(cfg, i))).to(dev)
        y = torch.empty((batch, n), dtype=torch.float32, device=dev)
        probs.append(Problem(torch, name, t, n, k, w, x, y))
    return probs


def run_pass(q, probs, stream):
    for p in probs:
        p.launch(q, stream)


def capture(torch, q, probs):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run_pass(q, probs, torch.cuda.current_stream().cuda_stream)   # warm (outside capture)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run_pass(q, probs, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, steps, warmup, min_warm_s=0.03):
    """Secondary timings: the requested warm-up replays, continued until at
    least min_warm_s of replays have run (sustained matrix-core load takes
    tens of milliseconds to reach steady clocks), then `steps` timed ones."""
    t0 = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t0 < min_warm_s:
        g.replay()
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def time_eager(torch, q, probs, steps, warmup):
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(warmup):
        run_pass(q, probs, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run_pass(q, probs, stream)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def cpu_baseline(cfg_probs_host, target_s):
    """The oracle (plain C, fp64, OpenMP over rows) on a bounded sample of the
    same workload: whole layers of the decode stream, taken in order (and
    again from the first layer once all are done) until about target_s
    seconds of CPU time are spent."""
    import oracle
    nthreads = oracle.max_threads()
    done_bytes, t_used, layers = 0, 0.0, 0
    per_layer = 7
    nl = len(cfg_probs_host) // per_layer
    while t_used < target_s or layers == 0:
        i = (layers % nl) * per_layer
        chunk = cfg_probs_host[i:i + per_layer]
        t0 = time.perf_counter()
        for (t, n, k, w, x) in chunk:
            oracle.gemv(t, w, n, k, x)
        t_used += time.perf_counter() - t0
        done_bytes += sum(n * G.row_bytes(t, k) + 4 * k + 4 * n for (t, n, k, w, x) in chunk)
        layers += 1
    return {"value": done_bytes / t_used / 1e9, "unit": "GB/s", "cores": nthreads, "kind": "oracle",
            "sample": "%d layers (%d GEMVs, %.1f MB of weights; the 22-layer Q4_0 stream repeated %.1f times), %.1f s"
                      % (layers, layers * per_layer, done_bytes / 1e6, layers / nl, t_used)}


# ------------------------------------------------------------- secondaries --

def sec_cfg1(torch, q, steps, warmup, dev):
    """Q8_0 2048x2048: rotate over 256 copies (1.14 GB) so caches cannot serve
    it; also the cache-resident single-call time."""
    n = k = 2048
    w0 = torch.from_numpy(G.gen_weights(G.Q8_0, n, k, 1000)).to(dev)
    x = torch.from_numpy(G.gen_x(k, 1, G.x_seed(1, 0))).to(dev)
    copies = [w0.clone() for _ in range(256)]
    y = torch.empty((1, n), dtype=torch.float32, device=dev)
    probs = [Problem(torch, "w%d" % i, G.Q8_0, n, k, c, x, y) for i, c in enumerate(copies)]
    g = capture(torch, q, probs)
    t = time_graph(torch, g, max(2, steps // 4), 2) / len(probs)
    hot = [Problem(torch, "hot", G.Q8_0, n, k, w0, x, y)] * 256
    gh = capture(torch, q, hot)
    th = time_graph(torch, gh, max(2, steps // 4), 2) / 256
    b = probs[0].bytes
    del copies, probs, g, gh
    return {"workload": "Q8_0 2048x2048 GEMV, batch 1, over 256 rotating copies",
            "us_per_gemv": t * 1e6, "GB_s": b / t / 1e9, "pct_hbm_peak": 100 * b / t / 1e9 / HBM_PEAK_GBS,
            "hot_us_per_gemv_cache_resident": th * 1e6}


def sec_stream(torch, q, cfg, weights, batch, steps, warmup, dev, label, with_gemm=False):
    probs = make_gemvs(torch, cfg, weights, batch, dev)
    wbytes = sum(p.wbytes for p in probs)
    tbytes = sum(p.bytes for p in probs)
    g = capture(torch, q, probs)
    tg = time_graph(torch, g, steps, warmup)
    out = {"workload": label, "gemvs": len(probs), "batch": batch, "weight_bytes": wbytes,
           "ms_per_pass": tg * 1e3, "GB_s": tbytes / tg / 1e9, "pct_hbm_peak": 100 * tbytes / tg / 1e9 / HBM_PEAK_GBS,
           "decode_tok_s": batch / tg}
    del g
    if with_gemm:
        # the same pass as a skinny GEMM (fp16 activations, M = batch)
        gp = []
        for p in probs:
            X = torch.from_numpy(G.gen_x_f16(batch, p.k, 77)).to(dev)
            gp.append(Problem(torch, p.name, p.t, p.n, p.k, p.w, X, p.y, kind="gemm"))
        gg = capture(torch, q, gp)
        tgg = time_graph(torch, gg, steps, warmup)
        out["skinny_gemm_ms_per_pass"] = tgg * 1e3
        out["skinny_gemm_tok_s"] = batch / tgg
        del gg, gp
    del probs
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
        g = capture(torch, q, probs)
        tg = time_graph(torch, g, steps, warmup)
        flops = sum(p.flops for p in probs)
        res[name] = {"shape": "4 x (%d x %d x %d)" % (m, n, k), "ms_4_chunks": tg * 1e3,
                     "TFLOP_s": flops / tg / 1e12, "pct_fp16_peak": 100 * flops / tg / 1e12 / FP16_PEAK_TFLOPS}
        del g, probs, w
    torch.cuda.empty_cache()
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

    # primary: TinyLlama-shaped Q4_0 decode stream, batch 1
    log("generating the Q4_0 decode stream (154 GEMVs)")
    host = []
    probs = []
    for i, (name, t, n, k, seed) in enumerate(G.workload(2)):
        w = G.gen_weights(t, n, k, seed)
        x = G.gen_x(k, 1, G.x_seed(2, i))
        host.append((t, n, k, w, x))
        probs.append(Problem(torch, name, t, n, k, torch.from_numpy(w).to(dev), torch.from_numpy(x).to(dev),
                             torch.empty((1, n), dtype=torch.float32, device=dev)))
    torch.cuda.synchronize()
    tot_bytes = sum(p.bytes for p in probs)
    w_bytes = sum(p.wbytes for p in probs)
    g = capture(torch, q, probs)
    log("timing %d graph replays after %d warmup" % (args.steps, args.warmup))
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    # HIP events on the stream the graph (and so every GEMV kernel) runs on
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / args.steps
    ev_step_s = ev0.elapsed_time(ev1) * 1e-3 / args.steps
    # spread of single passes: 20 replays, each between its own pair of events
    singles = []
    for _ in range(20):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        singles.append(a.elapsed_time(b))
    singles.sort()
    value = tot_bytes / step_s / 1e9
    # dominant kernel: every launch of the pass is the Q4_0 GEMV; its average
    # launch duration is the event time of the pass divided by the launches
    avg_launch_s = ev_step_s / len(probs)
    achieved = (tot_bytes / len(probs)) / avg_launch_s / 1e9
    eager_s = time_eager(torch, q, probs, max(3, args.steps // 2), 2)
    # the same 154 GEMVs with fewer launches per token: gate|up as one launch
    # (the dispatch count shimmy's pipeline page gives: 6 per layer) and
    # q|k|v + gate|up (4 per layer)
    grouped = {}
    # (and the 4-launch grouping once more with one activation per group, as
    # in a decoder layer: q / k / v read one x, gate / up another)
    for label, fuse, share in (("6_launches_per_layer", (("gate", "up"),), False),
                               ("4_launches_per_layer", (("q", "k", "v"), ("gate", "up")), False),
                               ("4_launches_per_layer_shared_x", (("q", "k", "v"), ("gate", "up")), True)):
        gp = group_layers(probs, fuse, share)
        gg = capture(torch, q, gp)
        tg = time_graph(torch, gg, args.steps, args.warmup)
        grouped[label] = {"launches": len(gp), "ms_per_pass": round(tg * 1e3, 4),
                          "GB_s": round(tot_bytes / tg / 1e9, 1), "decode_tok_s": round(1.0 / tg, 1)}
        del gg

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "TinyLlama-shaped Q4_0 decode weight stream: 22 layers x "
                               "(q 2048x2048, k/v 256x2048, o 2048x2048, gate/up 5632x2048, down 2048x5632) "
                               "= 154 GEMVs, batch 1, one HIP graph per pass",
                   "gemvs": len(probs), "batch": 1, "weight_bytes": w_bytes, "algorithmic_bytes": tot_bytes},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "decode_tok_s": round(1.0 / step_s, 1),
        "eager_ms_per_step": round(eager_s * 1e3, 4),
        "event_ms_per_step": round(ev_step_s * 1e3, 4),
        "single_pass_ms": {"median": round(0.5 * (singles[9] + singles[10]), 4), "min": round(singles[0], 4),
                           "max": round(singles[-1], 4), "passes": len(singles)},
        "grouped_launches": grouped,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": TRAFFIC,
                     "kernel": "Q4_0 batch-1 GEMV (gemv3_kernel for q/k/v/o and gate/up, gemv1_kernel for down, "
                               "k=5632)",
                     "avg_launch_us": round(avg_launch_s * 1e6, 3),
                     "bytes_per_launch": tot_bytes / len(probs)},
    }
    del g

    if not args.no_cpu_baseline:
        log("CPU oracle baseline (~%.0f s)" % args.cpu_seconds)
        line["cpu_baseline"] = cpu_baseline(host, args.cpu_seconds)
    del host

    if args.secondary != "none":
        want = (lambda s: args.secondary in ("all", s))
        sec = {}
        del probs
        torch.cuda.empty_cache()
        if want("q8_0"):
            log("secondary: Q8_0 single matrix")
            sec["q8_0_2048"] = sec_cfg1(torch, q, args.steps, args.warmup, dev)
        if want("q4_k"):
            log("secondary: Llama-3-8B Q4_K set")
            wts = build_weights(torch, 3, dev)
            sec["llama3_8b_q4_k"] = sec_stream(torch, q, 3, wts, 1, args.steps, args.warmup, dev,
                                               "Llama-3-8B-shaped Q4_K, 224 GEMVs, batch 1")
            del wts
            torch.cuda.empty_cache()
        if want("prefill"):
            log("secondary: prefill GEMMs")
            sec["prefill_512"] = sec_prefill(torch, q, args.steps, args.warmup, dev)
        if want("mix"):
            log("secondary: Q4_K_M-style mix weights")
            wts = build_weights(torch, 5, dev)
            for b in (1, 4, 8):
                log("secondary: Q4_K_M-style mix, batch", b)
                sec["q4_k_m_mix_b%d" % b] = sec_stream(
                    torch, q, 5, wts, b, max(3, args.steps // 2), 2, dev,
                    "Q4_K_M-style mix (v, down, LM head 128256x4096 in Q6_K), 225 GEMVs, batch %d" % b,
                    with_gemm=True)
            del wts
        if want("q5"):
            log("secondary: 5-bit types")
            wts = build_weights(torch, 6, dev)
            sec["llama3_8b_q5_k"] = sec_stream(torch, q, 6, wts, 1, args.steps, args.warmup, dev,
                                               "Llama-3-8B-shaped Q5_K, 224 GEMVs, batch 1")
            del wts
            torch.cuda.empty_cache()
            wts = build_weights(torch, 7, dev)
            sec["tinyllama_q5_0"] = sec_stream(torch, q, 7, wts, 1, args.steps, args.warmup, dev,
                                               "TinyLlama-shaped Q5_0 stream, 154 GEMVs, batch 1")
            del wts
            torch.cuda.empty_cache()
            sec["prefill_512_q5"] = sec_prefill(torch, q, args.steps, args.warmup, dev, cfg=8)
        if want("embed"):
            log("secondary: embedding gathers")
            sec["embed"] = sec_embed(torch, q, args.steps, args.warmup, dev)
        if want("dequant"):
            log("secondary: dequant-only")
            sec["dequant"] = sec_dequant(torch, q, args.steps, args.warmup, dev)
        if want("kv"):
            log("secondary: KV-cache codec")
            sec["kv_codec"] = sec_kv(torch, q, args.steps, args.warmup, dev)
        line["secondary"] = sec
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
