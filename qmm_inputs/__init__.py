"""Seeded synthetic inputs for the quantized-weight matmul.

This module only *draws* random field values and writes them into the byte
layout of each GGUF block type; it contains none of the method's arithmetic
(no decoding, no products).  Both the oracle-side tests and the GPU-side
tests/benchmark draw their inputs from here, so that the two paths see the
same bytes.

Block layouts written here (byte offsets inside one block, little-endian fp16):
  Q8_0  (32 elements, 34 B):  [0:2] d, [2:34] 32 x int8 codes
  Q4_0  (32 elements, 18 B):  [0:2] d, [2:18] 16 bytes of 4-bit codes
  Q4_K  (256 elements, 144 B): [0:2] d, [2:4] dmin, [4:16] 12 packed bytes of
                               6-bit scale/min fields, [16:144] 4-bit codes
  Q6_K  (256 elements, 210 B): [0:128] ql, [128:192] qh, [192:208] 16 x int8
                               scales, [208:210] d
  Q5_0  (32 elements, 22 B):  [0:2] d, [2:6] 32 high bits, [6:22] 4-bit codes
  Q5_K  (256 elements, 176 B): [0:2] d, [2:4] dmin, [4:16] scale/min bytes,
                               [16:48] high bits, [48:176] 4-bit codes

Distributions (the workload definitions that go with the pages):
  Q8_0: d ~ U[1e-3, 1e-2] rounded to fp16 (RNE), q ~ U{-127..127}
  Q4_0: d ~ U[1e-3, 1e-2], code bytes uniform (each nibble ~ U{0..15})
  Q4_K: d, dmin ~ U[1e-4, 1e-3]; the 12 scale bytes uniform (the packing is a
        bijection between 96 bits and 16 six-bit fields, so every field is
        ~ U{0..63}); code bytes uniform
  Q6_K: ql, qh uniform (so q ~ U{0..63}); scales ~ U{-64..63}; d ~ U[1e-4,1e-3]
  Q5_0 / Q5_K (no workload names them; the Q4_0 / Q4_K recipes): d (and
        dmin) as for Q4_0 / Q4_K, every other byte uniform (q ~ U{0..31})
  activations: fp32 (decode) or fp16 (prefill) ~ N(0, 1)
  token ids: int32 ~ U{0..vocab-1}
  KV-cache values to encode: fp16 ~ N(0, 1) (the pages give no distribution)

Seeds: matrix i of workload c uses seed 1000*c + i; its activation uses
1000*c + 500 + i.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

Q4_0, Q8_0, Q4_K, Q6_K, Q5_0, Q5_K = 0, 1, 2, 3, 4, 5
NAMES = {Q4_0: "Q4_0", Q8_0: "Q8_0", Q4_K: "Q4_K", Q6_K: "Q6_K", Q5_0: "Q5_0", Q5_K: "Q5_K"}
BLOCK_ELEMS = {Q4_0: 32, Q8_0: 32, Q4_K: 256, Q6_K: 256, Q5_0: 32, Q5_K: 256}
BLOCK_BYTES = {Q4_0: 18, Q8_0: 34, Q4_K: 144, Q6_K: 210, Q5_0: 22, Q5_K: 176}

DEFAULT_D_RANGE = {Q8_0: (1e-3, 1e-2), Q4_0: (1e-3, 1e-2), Q4_K: (1e-4, 1e-3), Q6_K: (1e-4, 1e-3),
                   Q5_0: (1e-3, 1e-2), Q5_K: (1e-4, 1e-3)}


def row_bytes(qtype: int, k: int) -> int:
    be = BLOCK_ELEMS[qtype]
    if k % be:
        raise ValueError("k=%d is not a multiple of the %s block size %d" % (k, NAMES[qtype], be))
    return (k // be) * BLOCK_BYTES[qtype]


def _f16_bytes(v: np.ndarray) -> np.ndarray:
    """fp64 draws -> fp16 (round to nearest even) -> little-endian bytes [..., 2]."""
    return v.astype("<f2").view(np.uint8).reshape(v.shape + (2,))


_CHUNK = 1 << 24   # bytes per independent uniform stream


def uniform_bytes(seed: int, nbytes: int) -> np.ndarray:
    """nbytes uniform random bytes.  Chunk c of 16 MiB comes from its own
    PCG64 stream seeded with (seed, c), so the result does not depend on how
    many threads draw it."""
    nch = (nbytes + _CHUNK - 1) // _CHUNK
    out = np.empty(nch * (_CHUNK // 8), dtype=np.uint64)

    def work(c):
        g = np.random.Generator(np.random.PCG64([seed, c]))
        out[c * (_CHUNK // 8):(c + 1) * (_CHUNK // 8)] = g.integers(
            0, 2 ** 64 - 1, size=_CHUNK // 8, dtype=np.uint64, endpoint=True)

    if nch == 1:
        work(0)
    else:
        with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1, nch))) as ex:
            list(ex.map(work, range(nch)))
    return out.view(np.uint8)[:nbytes]


def gen_weights(qtype: int, n: int, k: int, seed: int, d_range=None) -> np.ndarray:
    """Random quantized weight matrix as raw bytes, shape [n, row_bytes].

    Draw order (fixed, so a seed always gives the same bytes): one uniform
    byte string covering every block (``uniform_bytes``), then, from
    default_rng(seed), the fp16 scale fields (overwritten in place) and --
    for Q8_0 only -- the int8 codes."""
    rng = np.random.default_rng(seed)
    nb = k // BLOCK_ELEMS[qtype]
    rb = row_bytes(qtype, k)
    lo, hi = d_range if d_range is not None else DEFAULT_D_RANGE[qtype]
    blk = uniform_bytes(seed, n * rb).reshape(n, nb, BLOCK_BYTES[qtype])
    if qtype == Q8_0:
        blk[:, :, 0:2] = _f16_bytes(rng.uniform(lo, hi, size=(n, nb)))
        blk[:, :, 2:34] = rng.integers(-127, 128, size=(n, nb, 32), dtype=np.int8).view(np.uint8)
    elif qtype == Q4_0:
        # code bytes stay uniform: each nibble ~ U{0..15}
        blk[:, :, 0:2] = _f16_bytes(rng.uniform(lo, hi, size=(n, nb)))
    elif qtype == Q4_K:
        # scale bytes and code bytes stay uniform
        blk[:, :, 0:2] = _f16_bytes(rng.uniform(lo, hi, size=(n, nb)))
        blk[:, :, 2:4] = _f16_bytes(rng.uniform(lo, hi, size=(n, nb)))
    elif qtype == Q5_0:
        blk[:, :, 0:2] = _f16_bytes(rng.uniform(lo, hi, size=(n, nb)))
    elif qtype == Q5_K:
        blk[:, :, 0:2] = _f16_bytes(rng.uniform(lo, hi, size=(n, nb)))
        blk[:, :, 2:4] = _f16_bytes(rng.uniform(lo, hi, size=(n, nb)))
    elif qtype == Q6_K:
        # ql, qh uniform (q ~ U{0..63}); scale = (uniform byte & 127) - 64 ~ U{-64..63}
        sc = (blk[:, :, 192:208] & 0x7F).astype(np.int16) - 64
        blk[:, :, 192:208] = sc.astype(np.int8).view(np.uint8)
        blk[:, :, 208:210] = _f16_bytes(rng.uniform(lo, hi, size=(n, nb)))
    else:
        raise ValueError("unknown type %r" % (qtype,))
    return blk.reshape(n, rb)


def gen_x(k: int, batch: int, seed: int) -> np.ndarray:
    """fp32 activations [batch, k] ~ N(0, 1)."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((batch, k), dtype=np.float32)


def gen_ids(vocab: int, seq: int, seed: int) -> np.ndarray:
    """int32 token ids [seq] ~ U{0..vocab-1}."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, vocab, size=seq, dtype=np.int64).astype(np.int32)


def gen_x_f16(m: int, k: int, seed: int) -> np.ndarray:
    """fp16 activations [m, k] ~ N(0, 1) (drawn in fp32, rounded RNE)."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((m, k), dtype=np.float32).astype(np.float16)


# --------------------------------------------------------------------------
# Workloads (shapes, block types and seeds).  Each entry: (name, qtype, n, k).
# --------------------------------------------------------------------------

def _llama_layer(hidden, ffn, kv, t_default, t_v=None, t_down=None):
    t_v = t_default if t_v is None else t_v
    t_down = t_default if t_down is None else t_down
    return [("q", t_default, hidden, hidden), ("k", t_default, kv, hidden),
            ("v", t_v, kv, hidden), ("o", t_default, hidden, hidden),
            ("gate", t_default, ffn, hidden), ("up", t_default, ffn, hidden),
            ("down", t_down, hidden, ffn)]


def workload(cfg: int):
    """Matrix list of one workload: [(name, qtype, n, k, seed)], plus extras."""
    mats = []
    if cfg == 1:
        # single Q8_0 2048 x 2048 GEMV
        mats = [("w", Q8_0, 2048, 2048)]
    elif cfg == 2:
        # TinyLlama-shaped Q4_0 decode stream: 22 layers x 7 projections
        for layer in range(22):
            mats += [("l%d.%s" % (layer, nm), t, n, k)
                     for nm, t, n, k in _llama_layer(2048, 5632, 256, Q4_0)]
    elif cfg == 3:
        # Llama-3-8B-shaped Q4_K decode set: 32 layers x 7 projections
        for layer in range(32):
            mats += [("l%d.%s" % (layer, nm), t, n, k)
                     for nm, t, n, k in _llama_layer(4096, 14336, 1024, Q4_K)]
    elif cfg == 4:
        # prefill chunk GEMMs: N in {14336, 4096}, K = 4096, Q8_0 and Q4_K
        mats = [("gate_q8_0", Q8_0, 14336, 4096), ("q_q8_0", Q8_0, 4096, 4096),
                ("gate_q4_k", Q4_K, 14336, 4096), ("q_q4_k", Q4_K, 4096, 4096)]
    elif cfg == 5:
        # Q4_K_M-style mix: v and down in Q6_K, plus a Q6_K LM head
        for layer in range(32):
            mats += [("l%d.%s" % (layer, nm), t, n, k)
                     for nm, t, n, k in _llama_layer(4096, 14336, 1024, Q4_K, t_v=Q6_K, t_down=Q6_K)]
        mats.append(("lm_head", Q6_K, 128256, 4096))
    elif cfg == 6:
        # the 5-bit types (named by the pages, not by a workload): the
        # Llama-3-8B shapes of workload 3 in Q5_K
        for layer in range(32):
            mats += [("l%d.%s" % (layer, nm), t, n, k)
                     for nm, t, n, k in _llama_layer(4096, 14336, 1024, Q5_K)]
    elif cfg == 7:
        # the TinyLlama stream of workload 2 in Q5_0
        for layer in range(22):
            mats += [("l%d.%s" % (layer, nm), t, n, k)
                     for nm, t, n, k in _llama_layer(2048, 5632, 256, Q5_0)]
    elif cfg == 8:
        # the prefill chunk GEMMs of workload 4 in Q5_0 and Q5_K
        mats = [("gate_q5_0", Q5_0, 14336, 4096), ("q_q5_0", Q5_0, 4096, 4096),
                ("gate_q5_k", Q5_K, 14336, 4096), ("q_q5_k", Q5_K, 4096, 4096)]
    elif cfg == 9:
        # quantized token-embedding tables for the row gather: the Llama 3.2
        # 1B table in Q8_0 (the type the pages' embedding kernel reads) and
        # the Llama-3-8B table in Q4_K; ids ~ U{0..vocab-1}, 1 or 512 tokens
        mats = [("embd_q8_0", Q8_0, 128256, 2048), ("embd_q4_k", Q4_K, 128256, 4096)]
    elif cfg == 10:
        # KV-cache codec: one layer's K (or V) rows of Llama-3-8B (8 KV heads
        # x 128 = 1024 values per token) over an 8192-token context, encoded
        # to Q8_0 or Q4_0; the values are fp16 ~ N(0, 1) (gen_x_f16)
        mats = [("kv_q8_0", Q8_0, 8192, 1024), ("kv_q4_0", Q4_0, 8192, 1024)]
    else:
        raise ValueError("unknown workload %r" % (cfg,))
    return [(nm, t, n, k, 1000 * cfg + i) for i, (nm, t, n, k) in enumerate(mats)]


def decode_stage(name: str) -> int:
    """Stage of a decode-stream matrix in a decoder's dataflow: per layer L,
    q / k / v read the normalized hidden state (stage 4L), o reads the
    attention output (4L + 1), gate / up the normalized hidden state after
    attention (4L + 2), down the gated FFN activation (4L + 3); the LM head
    comes after the last layer."""
    if name == "lm_head":
        return 1 << 20
    layer, proj = name.split(".")
    L = int(layer[1:])
    return 4 * L + {"q": 0, "k": 0, "v": 0, "o": 1, "gate": 2, "up": 2, "down": 3}[proj]


def x_seed(cfg: int, i: int) -> int:
    return 1000 * cfg + 500 + i


PREFILL_M = 512
PREFILL_CHUNKS = 4
