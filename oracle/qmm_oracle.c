/*
 * qmm_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU reference for the quantized-weight
 * matmul with inline block dequantization.  Only the tests, the smoke check
 * and the benchmark's CPU-baseline leg may load this library; the product
 * path (the HIP library) never links, loads or calls it, and it shares no
 * code, header or table with that path.
 *
 * What it computes (plain definitions, no blocking, fusion or reordering):
 *   - dequant:  every weight w = f(block fields), computed exactly in fp64 and
 *               rounded once to fp32 (the exact value is always representable
 *               or, for Q4_K with extreme scales, rounded to nearest-even);
 *   - gemv:     y[b][n] = sum_k w[n][k] * x[b][k], fp64, k in ascending order,
 *               plus a[b][n] = sum_k |w[n][k] * x[b][k]| for the tolerance;
 *   - gemm:     Y[m][n] = sum_k X[m][k] * w[n][k] with X given as IEEE fp16
 *               bits, w the exact fp32 dequant (not rounded to fp16), fp64
 *               accumulation in ascending k, plus the same |.| sum.
 *   - embed:    out[i] = dequant of table row ids[i] (zeros for an id out of
 *               range);
 *   - fp16:     any fp32 result rounded to binary16, nearest-even (the FP16
 *               outputs of the dequant and the embedding gather).
 *   - quantize: fp32 (or fp16) values -> Q8_0 / Q4_0 blocks by the GGUF
 *               rule, in fp32 (the KV-cache encoder).
 *
 * Sources (page / section):
 *   - shimmy "Airframe GPU pipeline", per-layer ops: dequantization happens
 *     inline inside each matmul (the operation being checked).
 *   - shimmy "Architecture", Quantization table: the GGUF block types the GPU
 *     shaders decode (Q4_0 32-element 4-bit, Q8_0 32-element 8-bit, K-quant
 *     super-blocks, Q6_K 6-bit) and "fp16 unpack" for the scales.
 *   - dotLLM "GPU Inference", Quantization on GPU table and Weight Strategy:
 *     weights stay in their original quantized bytes; Q4_K is about
 *     4.5 bits per parameter.
 *   - Field layouts the pages do not print are taken from the workload
 *     definitions that accompany them (Q8_0: fp16 d then 32 int8; Q4_0: fp16 d
 *     then 16 bytes of nibbles, low nibbles = elements 0-15; Q4_K: fp16 d,
 *     fp16 dmin, 12 bytes of 6-bit scale/min pairs, 128 bytes of nibbles;
 *     Q6_K: 128 bytes ql, 64 bytes qh, 16 int8 scales, fp16 d).
 *   - Where neither says how codes map to elements (the Q4_K nibble order and
 *     the Q6_K ql/qh bit planes) this follows the public GGUF convention; that
 *     mapping is "parity unpinned" against real files (none are available) and
 *     is pinned only by encoder/decoder self-consistency tests.
 *   - Q5_0 and Q5_K: shimmy "Architecture", Quantization table names a
 *     5-bit super-block with a high-bit plane, and dotLLM "GPU Inference",
 *     Quantization on GPU table lists Q5_0 and Q5_K (dequant-only there);
 *     neither prints a layout.  Theirs here (GGUF convention, parity
 *     unpinned) is the 4-bit layout of Q4_0 / Q4_K plus one high bit per
 *     element in a separate bit plane.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC.
 * Parallelism is an OpenMP loop over independent output rows only; it does not
 * change any result.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Type ids, mirrored by value (not by header) from the public ABI. */
enum { OR_Q4_0 = 0, OR_Q8_0 = 1, OR_Q4_K = 2, OR_Q6_K = 3, OR_Q5_0 = 4, OR_Q5_K = 5 };

/* Return codes: 0 = ok, -1 = bad type, -2 = bad shape, -3 = out of memory. */

int oracle_block_elems(int t)
{
    switch (t) {
    case OR_Q4_0: return 32;
    case OR_Q8_0: return 32;
    case OR_Q4_K: return 256;
    case OR_Q6_K: return 256;
    case OR_Q5_0: return 32;
    case OR_Q5_K: return 256;
    default: return 0;
    }
}

int oracle_block_bytes(int t)
{
    switch (t) {
    case OR_Q4_0: return 2 + 16;            /* d, 16 bytes of nibbles        */
    case OR_Q8_0: return 2 + 32;            /* d, 32 int8 codes              */
    case OR_Q4_K: return 2 + 2 + 12 + 128;  /* d, dmin, scales, nibbles      */
    case OR_Q6_K: return 128 + 64 + 16 + 2; /* ql, qh, int8 scales, d        */
    case OR_Q5_0: return 2 + 4 + 16;        /* d, 32 high bits, nibbles      */
    case OR_Q5_K: return 2 + 2 + 12 + 32 + 128; /* d, dmin, scales, qh, nibbles */
    default: return 0;
    }
}

/*
 * IEEE 754 binary16 -> value, written from the format definition
 * (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits):
 *   e == 0       : (-1)^s * f * 2^-24          (zero / subnormal)
 *   e == 31      : +-Inf if f == 0, else NaN
 *   otherwise    : (-1)^s * (1024 + f) * 2^(e - 25)
 * Every binary16 value is exactly representable in fp32 and fp64.
 * (shimmy "Architecture", Quantization table: "fp16 unpack".)
 */
double oracle_half_to_double(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return s ? -v : v;
}

float oracle_half_to_float(uint16_t h)
{
    return (float)oracle_half_to_double(h);
}

void oracle_half_to_float_array(const uint16_t *h, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_half_to_float(h[i]);
}

/*
 * value -> IEEE 754 binary16 bits, round to nearest with ties to even,
 * written from the format definition.  A finite nonzero |v| is rounded to a
 * multiple of the quantum 2^(E - 10) of its binade, E = floor(log2 |v|),
 * with E raised to -14 below the normal range (the subnormal quantum
 * 2^-24):  m = rint(|v| / 2^(E - 10)) (ties to even in the default rounding
 * mode), bits = ((E + 15) << 10) + m - 1024.  The formula also covers the
 * subnormals (E = -14, m < 1024 gives bits = m) and the carry into the next
 * binade (m = 2048); a result at or above the Inf pattern 0x7c00 is Inf.
 * NaN -> quiet NaN 0x7e00 with the sign kept.
 * (dotLLM "GPU Inference", Forward Pass: the hidden state is FP16; Custom
 * Kernels table: dequant_* kernels write FP16.)
 */
uint16_t oracle_double_to_half(double v)
{
    uint16_t s = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return (uint16_t)(s | 0x7e00);
    if (isinf(a))
        return (uint16_t)(s | 0x7c00);
    if (a == 0.0)
        return s;
    int E;
    frexp(a, &E); /* a = f 2^E with 0.5 <= f < 1 */
    E -= 1;       /* now 1 <= a / 2^E < 2 */
    if (E < -14)
        E = -14;
    double m = rint(ldexp(a, 10 - E)); /* scaling by a power of two is exact */
    long bits = ((long)(E + 15) << 10) + (long)m - 1024;
    if (bits >= 0x7c00)
        return (uint16_t)(s | 0x7c00);
    return (uint16_t)(s | bits);
}

void oracle_float_to_half_array(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_double_to_half((double)x[i]);
}

static uint16_t rd16(const uint8_t *p)
{
    return (uint16_t)(p[0] | (p[1] << 8)); /* little-endian */
}

/*
 * Q4_K 6-bit scale / min of sub-block j (0..7) from the 12 packed bytes s[].
 * Rule, as given with the Llama-3-8B Q4_K workload:
 *   sub-blocks 0-3: scale = low 6 bits of byte j, min = low 6 bits of byte j+4;
 *   sub-blocks 4-7: scale = low nibble of byte j+4 with the top 2 bits of
 *                   byte j-4 as bits 4-5; min = high nibble of byte j+4 with
 *                   the top 2 bits of byte j as bits 4-5.
 */
void oracle_q4k_scale_min(const uint8_t *s, int j, int *sc, int *m)
{
    if (j < 4) {
        *sc = s[j] & 63;
        *m = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/* Exact value of element e (0 <= e < block_elems) of one block, in fp64. */
static double elem_value(int t, const uint8_t *blk, int e)
{
    switch (t) {
    case OR_Q8_0: {
        /* w = d * q, q the int8 at byte 2+e. */
        double d = oracle_half_to_double(rd16(blk));
        int q = (int)(int8_t)blk[2 + e];
        return d * (double)q;
    }
    case OR_Q4_0: {
        /* 16 bytes of nibbles: low nibbles are elements 0-15, high nibbles
         * elements 16-31; w = d * (q - 8). */
        double d = oracle_half_to_double(rd16(blk));
        const uint8_t *qs = blk + 2;
        int q = (e < 16) ? (qs[e] & 15) : (qs[e - 16] >> 4);
        return d * (double)(q - 8);
    }
    case OR_Q4_K: {
        /* w = d * sc_j * q - dmin * m_j, sub-block j = e / 32.
         * Code placement (GGUF convention, parity unpinned): the 128 code
         * bytes form 4 groups of 32; group p holds sub-block 2p in its low
         * nibbles and sub-block 2p+1 in its high nibbles, element l of the
         * sub-block sitting in byte l of the group. */
        double d = oracle_half_to_double(rd16(blk));
        double dmin = oracle_half_to_double(rd16(blk + 2));
        const uint8_t *s = blk + 4;
        const uint8_t *qs = blk + 16;
        int j = e / 32, l = e % 32, sc, m;
        oracle_q4k_scale_min(s, j, &sc, &m);
        uint8_t byte = qs[32 * (j / 2) + l];
        int q = (j % 2 == 0) ? (byte & 15) : (byte >> 4);
        return d * (double)sc * (double)q - dmin * (double)m;
    }
    case OR_Q6_K: {
        /* w = d * scale[e/16] * (q - 32), q a 6-bit code split into a low
         * nibble (ql) and 2 high bits (qh).  Bit placement (GGUF convention,
         * parity unpinned): the block is two halves h of 128 elements; within
         * a half, r = e % 128, g = r / 32, l = r % 32; the low nibble is in
         * ql[64h + 32(g%2) + l] (low nibble for g < 2, high nibble for
         * g >= 2) and the high bits are bits 2g..2g+1 of qh[32h + l]. */
        const uint8_t *ql = blk;
        const uint8_t *qh = blk + 128;
        const int8_t *sc = (const int8_t *)(blk + 192);
        double d = oracle_half_to_double(rd16(blk + 208));
        int h = e / 128, r = e % 128, g = r / 32, l = r % 32;
        uint8_t lb = ql[64 * h + 32 * (g % 2) + l];
        int lo = (g < 2) ? (lb & 15) : (lb >> 4);
        int hi = (qh[32 * h + l] >> (2 * g)) & 3;
        int q = lo | (hi << 4);
        return d * (double)sc[e / 16] * (double)(q - 32);
    }
    case OR_Q5_0: {
        /* 5-bit codes: the low 4 bits as in Q4_0 (16 bytes of nibbles at
         * byte 6, low nibbles elements 0-15, high nibbles 16-31), bit 4 of
         * element e is bit e of the little-endian 32-bit word at byte 2;
         * w = d * (q - 16).  (Layout: GGUF convention, parity unpinned.) */
        double d = oracle_half_to_double(rd16(blk));
        uint32_t qh = (uint32_t)blk[2] | ((uint32_t)blk[3] << 8) | ((uint32_t)blk[4] << 16) |
                      ((uint32_t)blk[5] << 24);
        const uint8_t *qs = blk + 6;
        int lo = (e < 16) ? (qs[e] & 15) : (qs[e - 16] >> 4);
        int q = lo | (int)(((qh >> e) & 1u) << 4);
        return d * (double)(q - 16);
    }
    case OR_Q5_K: {
        /* w = d * sc_j * q - dmin * m_j as Q4_K (same scale/min packing),
         * q a 5-bit code: the low 4 bits placed as in Q4_K (code bytes at
         * byte 48), bit 4 is bit j of qh[l], the 32 bytes at byte 16, for
         * element l of sub-block j.  (Layout: GGUF convention, parity
         * unpinned.) */
        double d = oracle_half_to_double(rd16(blk));
        double dmin = oracle_half_to_double(rd16(blk + 2));
        const uint8_t *s = blk + 4;
        const uint8_t *qh = blk + 16;
        const uint8_t *qs = blk + 48;
        int j = e / 32, l = e % 32, sc, m;
        oracle_q4k_scale_min(s, j, &sc, &m);
        uint8_t byte = qs[32 * (j / 2) + l];
        int lo = (j % 2 == 0) ? (byte & 15) : (byte >> 4);
        int q = lo | (((qh[l] >> j) & 1) << 4);
        return d * (double)sc * (double)q - dmin * (double)m;
    }
    default:
        return NAN;
    }
}

static int check(int t, int64_t n, int64_t k)
{
    int be = oracle_block_elems(t);
    if (be == 0)
        return -1;
    if (n < 0 || k < 0 || k % be != 0)
        return -2;
    return 0;
}

size_t oracle_row_bytes(int t, int64_t k)
{
    int be = oracle_block_elems(t);
    if (be == 0 || k < 0 || k % be != 0)
        return 0;
    return (size_t)(k / be) * (size_t)oracle_block_bytes(t);
}

/* One row of k weights -> fp32 (exact value rounded once). */
static void dequant_row(int t, const uint8_t *row, int64_t k, float *out)
{
    int be = oracle_block_elems(t), bb = oracle_block_bytes(t);
    for (int64_t i = 0; i < k; i++)
        out[i] = (float)elem_value(t, row + (i / be) * bb, (int)(i % be));
}

/* out[n][k] = dequantized weights, row-major fp32. */
int oracle_dequant(int t, const uint8_t *w, int64_t n, int64_t k, float *out)
{
    int rc = check(t, n, k);
    if (rc)
        return rc;
    size_t rb = oracle_row_bytes(t, k);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; r++)
        dequant_row(t, w + (size_t)r * rb, k, out + (size_t)r * k);
    return 0;
}

/* fp64 value of each weight (no fp32 rounding), for exact-arithmetic pins. */
int oracle_dequant_f64(int t, const uint8_t *w, int64_t n, int64_t k, double *out)
{
    int rc = check(t, n, k);
    if (rc)
        return rc;
    size_t rb = oracle_row_bytes(t, k);
    int be = oracle_block_elems(t), bb = oracle_block_bytes(t);
    for (int64_t r = 0; r < n; r++)
        for (int64_t i = 0; i < k; i++)
            out[r * k + i] = elem_value(t, w + r * rb + (i / be) * bb, (int)(i % be));
    return 0;
}

/*
 * Embedding row gather: out[i][:] = the fp32 dequant of row ids[i] of the
 * table [vocab][k]; an id outside [0, vocab) gives a row of zeros (a choice
 * of this library: the pages do not say what an invalid id does).
 * (dotLLM "GPU Inference", Forward Pass step 2 and Weight Loading Pipeline:
 * the token embeddings stay quantized on the GPU and the lookup kernel
 * dequantizes the rows of the given token ids into the hidden state.)
 */
int oracle_embed(int t, const uint8_t *table, int64_t vocab, int64_t k,
                 const int32_t *ids, int64_t seq, float *out)
{
    int rc = check(t, vocab, k);
    if (rc)
        return rc;
    if (seq < 0)
        return -2;
    size_t rb = oracle_row_bytes(t, k);
    for (int64_t i = 0; i < seq; i++) {
        int64_t id = ids[i];
        float *dst = out + (size_t)i * k;
        if (id >= 0 && id < vocab)
            dequant_row(t, table + (size_t)id * rb, k, dst);
        else
            memset(dst, 0, (size_t)k * sizeof(float));
    }
    return 0;
}

/*
 * Quantize (the KV-cache encoder): each block of 32 fp32 values -> one Q8_0 or
 * Q4_0 block, by the GGUF rule for these types, every step in fp32 (the
 * precision in which the codes are decided):
 *   Q8_0: amax = max |x_i|; d = amax / 127; id = 1 / d (0 when d == 0);
 *         q_i = x_i * id rounded half away from zero; stored d = fp16(d).
 *   Q4_0: v = the x_i of largest magnitude (the first one on a tie);
 *         d = v / -8; id = 1 / d (0 when d == 0);
 *         q_i = min(15, trunc(x_i * id + 8.5)); stored d = fp16(d).
 * Codes are computed with the fp32 d, before d is rounded to fp16.
 * (dotLLM "GPU Inference", Implementation: a GPU KV-cache quantized to Q8_0
 * or Q4_0 with an FP16 window; the pages do not state the rounding rule.)
 * x: fp32 [n][k], k a multiple of 32; out: n rows of row-bytes.
 */
static void quantize_block(int t, const float *x, uint8_t *blk)
{
    if (t == OR_Q8_0) {
        float amax = 0.0f;
        for (int i = 0; i < 32; i++)
            if (fabsf(x[i]) > amax)
                amax = fabsf(x[i]);
        float d = amax / 127.0f;
        float id = (d != 0.0f) ? 1.0f / d : 0.0f;
        uint16_t h = oracle_double_to_half((double)d);
        blk[0] = (uint8_t)(h & 0xff);
        blk[1] = (uint8_t)(h >> 8);
        for (int i = 0; i < 32; i++) {
            float v = x[i] * id;
            blk[2 + i] = (uint8_t)(int8_t)(int)roundf(v);
        }
    } else { /* Q4_0 */
        float amax = 0.0f, vmax = 0.0f;
        for (int i = 0; i < 32; i++)
            if (fabsf(x[i]) > amax) {
                amax = fabsf(x[i]);
                vmax = x[i];
            }
        float d = vmax / -8.0f;
        float id = (d != 0.0f) ? 1.0f / d : 0.0f;
        uint16_t h = oracle_double_to_half((double)d);
        blk[0] = (uint8_t)(h & 0xff);
        blk[1] = (uint8_t)(h >> 8);
        int q[32];
        for (int i = 0; i < 32; i++) {
            float v = x[i] * id;
            float u = v + 8.5f;
            int c = (int)truncf(u);
            q[i] = c < 15 ? c : 15;
        }
        for (int i = 0; i < 16; i++)
            blk[2 + i] = (uint8_t)(q[i] | (q[i + 16] << 4));
    }
}

int oracle_quantize(int t, const float *x, int64_t n, int64_t k, uint8_t *out)
{
    if (t != OR_Q8_0 && t != OR_Q4_0)
        return -1;
    int rc = check(t, n, k);
    if (rc)
        return rc;
    int bb = oracle_block_bytes(t);
    int64_t nblk = n * (k / 32);
    for (int64_t b = 0; b < nblk; b++)
        quantize_block(t, x + b * 32, out + b * bb);
    return 0;
}

/* The same with fp16 input (IEEE bits), converted exactly to fp32 first. */
int oracle_quantize_f16(int t, const uint16_t *x, int64_t n, int64_t k, uint8_t *out)
{
    if (t != OR_Q8_0 && t != OR_Q4_0)
        return -1;
    int rc = check(t, n, k);
    if (rc)
        return rc;
    int bb = oracle_block_bytes(t);
    int64_t nblk = n * (k / 32);
    for (int64_t b = 0; b < nblk; b++) {
        float xf[32];
        for (int i = 0; i < 32; i++)
            xf[i] = oracle_half_to_float(x[b * 32 + i]);
        quantize_block(t, xf, out + b * bb);
    }
    return 0;
}

/*
 * y[b][n] = sum_k w[n][k] * x[b][k];  a[b][n] = sum_k |w[n][k] * x[b][k]|.
 * x is fp32 [batch][k].  Products of two fp32 values are exact in fp64, so
 * only the ascending-k summation rounds (relative error <= k * 2^-53).
 */
int oracle_gemv(int t, const uint8_t *w, int64_t n, int64_t k,
                const float *x, int64_t batch, double *y, double *a)
{
    int rc = check(t, n, k);
    if (rc)
        return rc;
    if (batch < 0)
        return -2;
    size_t rb = oracle_row_bytes(t, k);
    int fail = 0;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; r++) {
        /* one fp32 dequant pass over the row, then fp64 dot products */
        float *wrow = (float *)malloc((size_t)(k > 0 ? k : 1) * sizeof(float));
        if (!wrow) {
#pragma omp atomic write
            fail = 1;
            continue;
        }
        dequant_row(t, w + (size_t)r * rb, k, wrow);
        for (int64_t b = 0; b < batch; b++) {
            double acc = 0.0, aac = 0.0;
            for (int64_t i = 0; i < k; i++) {
                double p = (double)wrow[i] * (double)x[b * k + i];
                acc += p;
                aac += fabs(p);
            }
            y[b * n + r] = acc;
            a[b * n + r] = aac;
        }
        free(wrow);
    }
    if (fail)
        return -3;
    return 0;
}

/*
 * Y[m][n] = sum_k X[m][k] * w[n][k];  A[m][n] = sum_k |X[m][k] * w[n][k]|.
 * X is IEEE fp16 bits [m][k], converted exactly; w is the exact fp32 dequant.
 * rows (optional, may be NULL): compute only output rows rows[0..nrows) of
 * Y/A, stored compactly as [nrows][n]; with rows == NULL, nrows must equal m.
 */
int oracle_gemm(int t, const uint8_t *w, int64_t n, int64_t k,
                const uint16_t *x, int64_t m, const int64_t *rows, int64_t nrows,
                double *y, double *a)
{
    int rc = check(t, n, k);
    if (rc)
        return rc;
    if (m < 0 || nrows < 0 || (rows == NULL && nrows != m))
        return -2;
    for (int64_t i = 0; rows && i < nrows; i++)
        if (rows[i] < 0 || rows[i] >= m)
            return -2;
    size_t rb = oracle_row_bytes(t, k);
    int fail = 0;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; r++) {
        float *wrow = (float *)malloc((size_t)(k > 0 ? k : 1) * sizeof(float));
        if (!wrow) {
#pragma omp atomic write
            fail = 1;
            continue;
        }
        dequant_row(t, w + (size_t)r * rb, k, wrow);
        for (int64_t ii = 0; ii < nrows; ii++) {
            int64_t mm = rows ? rows[ii] : ii;
            double acc = 0.0, aac = 0.0;
            for (int64_t i = 0; i < k; i++) {
                double p = oracle_half_to_double(x[mm * k + i]) * (double)wrow[i];
                acc += p;
                aac += fabs(p);
            }
            y[ii * n + r] = acc;
            a[ii * n + r] = aac;
        }
        free(wrow);
    }
    if (fail)
        return -3;
    return 0;
}

void oracle_set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
