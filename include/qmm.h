/*
 * qmm.h -- C ABI of libqmm.so: matrix products whose weights are stored as
 * GGUF quantized blocks and decoded on the fly on an AMD Instinct MI355X
 * (gfx950).
 *
 * The operation (shimmy "Airframe GPU pipeline", per-layer ops): every matmul
 * decodes the quantized weight blocks inline and multiplies them by the
 * activations; there is no separate dequantize-then-multiply pass.  dotLLM
 * "GPU Inference" (Forward Pass, step 4a) splits the same projections by
 * sequence length: one token (decode) uses a quantized GEMV straight from the
 * blocks, many tokens (prefill) a dense FP16 GEMM; its kernel table lists
 * dequant-to-FP16 kernels and quantized GEMV kernels with one block per
 * output row.  Weights stay resident in their original quantized bytes
 * (dotLLM "GPU Inference", Weight Loading Pipeline).
 *
 * Block types (shimmy "Architecture", Quantization table; dotLLM "GPU
 * Inference", Quantization on GPU table).  Byte layout of one block,
 * little-endian fp16 fields:
 *   QMM_Q4_0  32 elements, 18 B:  d | 16 B codes        w = d (q - 8)
 *             element i < 16: low nibble of code byte i; i >= 16: high
 *             nibble of code byte i - 16
 *   QMM_Q8_0  32 elements, 34 B:  d | 32 int8 codes     w = d q
 *   QMM_Q4_K  256 elements, 144 B: d | dmin | 12 B scales | 128 B codes
 *             w = d sc_j q - dmin m_j, j = e / 32 (6-bit sc_j, m_j packed in
 *             the 12 bytes: j < 4 low 6 bits of bytes j and j+4; j >= 4 the
 *             nibbles of byte j+4 plus the top 2 bits of bytes j-4 and j);
 *             element (j, l) is nibble (j % 2) of code byte 32 (j / 2) + l
 *   QMM_Q6_K  256 elements, 210 B: 128 B ql | 64 B qh | 16 int8 scales | d
 *             w = d scale[e / 16] (q - 32); element e = 128 h + 32 g + l has
 *             its low 4 bits in nibble (g / 2) of ql[64 h + 32 (g % 2) + l]
 *             and its high 2 bits at bit 2 g of qh[32 h + l]
 *   QMM_Q5_0  32 elements, 22 B:  d | 4 B high bits | 16 B codes
 *             w = d (q - 16); low 4 bits of element i as in Q4_0, bit 4 is
 *             bit i of the little-endian 32-bit word
 *   QMM_Q5_K  256 elements, 176 B: d | dmin | 12 B scales | 32 B qh |
 *             128 B codes; w = d sc_j q - dmin m_j as in Q4_K (same scale
 *             packing and low-4-bit placement); bit 4 of element (j, l) is
 *             bit j of qh[l]
 *   (shimmy "Architecture", Quantization table names the 5-bit super-block
 *   with a high-bit plane and dotLLM "GPU Inference", Quantization on GPU
 *   table lists Q5_0 / Q5_K; neither prints their layout, which here is the
 *   public GGUF one.)
 *
 * Common conventions
 *   - Weight matrix w: n rows (output features) of qmm_row_bytes(t, k)
 *     bytes each, packed back to back; a row holds the k inputs in block
 *     order.  Row-major outputs (dotLLM "GPU Inference", cuBLAS GEMM/GEMV:
 *     row-major C = A x B).
 *   - All pointers are device pointers (HIP device memory, or memory the
 *     device can access) and must be 16-byte aligned.  The caller owns every
 *     buffer; the library allocates nothing and keeps no state between calls
 *     besides device properties it reads once per device (CU count, resident
 *     workgroups per kernel, cached with atomics), and is safe to call from
 *     several host threads.
 *   - stream: a hipStream_t passed as void* (NULL = the default stream).
 *     Every call only enqueues work on that stream and never synchronizes
 *     (dotLLM "GPU Inference", Synchronization Model: one stream, all
 *     launches asynchronous).  Outputs are overwritten, never accumulated.
 *   - Argument errors are detected on the host before anything is enqueued;
 *     the call then returns the error and touches no memory.  A launch error
 *     reported by the HIP runtime returns QMM_ERR_HIP.  Errors of earlier,
 *     unrelated work on the stream are not reported here.
 *   - Empty problems (n == 0, or batch / m == 0) return QMM_OK and enqueue
 *     nothing; k == 0 with n > 0 writes zeros to the output (empty sums).
 *     This is deliberate, not an argument error: an empty matrix product is
 *     well defined, and callers whose row or token counts vary need no
 *     special case.  Negative sizes are errors.
 *   - Block types are passed as int (the qmm_type values) and streams as
 *     void *, so that this header needs no HIP header.
 */
#ifndef QMM_H
#define QMM_H

#include <stddef.h>
#include <stdint.h>

#ifndef QMM_API
#define QMM_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qmm_type {
    QMM_Q4_0 = 0,
    QMM_Q8_0 = 1,
    QMM_Q4_K = 2,
    QMM_Q6_K = 3,
    QMM_Q5_0 = 4,
    QMM_Q5_K = 5
} qmm_type;

typedef enum qmm_status {
    QMM_OK = 0,
    QMM_ERR_NULL = 1,  /* a required pointer is NULL                     */
    QMM_ERR_TYPE = 2,  /* unknown block type                             */
    QMM_ERR_SHAPE = 3, /* negative size, k not a block multiple, batch>8 */
    QMM_ERR_ALIGN = 4, /* a pointer is not 16-byte aligned               */
    QMM_ERR_HIP = 5    /* the HIP runtime rejected a launch              */
} qmm_status;

/* Elements per block (32 or 256); 0 for an unknown type. */
QMM_API int qmm_block_elems(int type);

/* Bytes per block (18, 34, 144, 210, 22, 176); 0 for an unknown type. */
QMM_API int qmm_block_bytes(int type);

/* Bytes of one row of k weights; 0 if the type is unknown, k < 0 or k is not
 * a multiple of the block size. */
QMM_API size_t qmm_row_bytes(int type, int64_t k);

/*
 * Dequantize: out[n][k] (fp32, row-major) = the weights of w.
 * Each value is the exact weight rounded once to fp32; no division,
 * reciprocal or fp16 intermediate is used, so the result is bit-identical to
 * any exact decoder.  (dotLLM "GPU Inference", Custom Kernels table: the
 * dequant_* kernels; here the output is fp32 so it can be exact.)
 */
QMM_API int qmm_dequant(int type, const void *w, int64_t n, int64_t k, float *out, void *stream);

/*
 * Dequantize to FP16: out[n][k] holds IEEE fp16 bit patterns, each the fp32
 * value of qmm_dequant rounded to nearest-even (magnitudes of 65520 and
 * above become +-Inf).  (dotLLM "GPU Inference", Custom Kernels table: the
 * dequant_*_f16 kernels write the FP16 scratch of the prefill GEMM.)
 */
QMM_API int qmm_dequant_f16(int type, const void *w, int64_t n, int64_t k, uint16_t *out, void *stream);

/*
 * Embedding gather: out[r][:] = the weights of row ids[r] of the quantized
 * table [vocab][k], for r < seq, each value as in qmm_dequant (fp32, exact).
 * An id outside [0, vocab) gives a row of +0 (the pages do not say what an
 * invalid id does; this library neither reads out of the table nor fails,
 * since the ids are device data).  table: vocab rows of qmm_row_bytes(type,
 * k) bytes; ids: int32 [seq], device memory, 4-byte aligned (the one pointer
 * exempt from 16-byte alignment); out: fp32 [seq][k].  vocab == 0 is allowed
 * (every row is zero, table may be NULL); seq == 0 or k == 0 is a no-op.
 * (dotLLM "GPU Inference", Forward Pass step 2 and Weight Loading Pipeline:
 * the token embeddings stay in their quantized format on the GPU and the
 * lookup kernel dequantizes the rows of the token ids into the hidden state;
 * Custom Kernels table: embedding_lookup_* with one workgroup row per token.)
 */
QMM_API int qmm_embed(int type, const void *table, int64_t vocab, int64_t k, const int32_t *ids, int64_t seq,
                      float *out, void *stream);

/* As qmm_embed with an FP16 output (fp16 bit patterns [seq][k], each the
 * fp32 value rounded to nearest-even): dotLLM's hidden state is FP16. */
QMM_API int qmm_embed_f16(int type, const void *table, int64_t vocab, int64_t k, const int32_t *ids,
                          int64_t seq, uint16_t *out, void *stream);

/*
 * Quantize (the encoder of a quantized KV cache): x [n][k] (fp32, k a
 * multiple of 32) -> out, n rows of qmm_row_bytes(type, k) bytes of Q8_0 or
 * Q4_0 blocks (other types: QMM_ERR_TYPE).  Each block of 32 values follows
 * the GGUF rule, every step in fp32:
 *   Q8_0  d = amax / 127, codes = x / d rounded half away from zero
 *         (computed as x * (1 / d)); 0 codes and d = 0 for a zero block;
 *   Q4_0  v = the value of largest magnitude (the first on a tie),
 *         d = v / -8, codes = min(15, trunc(x * (1 / d) + 8.5)); a zero
 *         block gets d = -0 and codes 8;
 * the codes use the fp32 d, which is stored rounded to fp16 (nearest-even).
 * The divisions are correctly rounded and nothing is fused, so the bytes
 * are those of any exact fp32 evaluation.  x must be finite (otherwise the
 * block's bytes are unspecified).  Decoding back: qmm_dequant_f16 /
 * qmm_dequant.  (dotLLM "GPU Inference", Implementation: a GPU KV-cache
 * quantized to Q8_0 / Q4_0 with an FP16 window of recent tokens; the pages
 * state no rounding rule.)
 */
QMM_API int qmm_quantize(int type, const float *x, int64_t n, int64_t k, void *out, void *stream);

/* As qmm_quantize with fp16 input (IEEE bit patterns [n][k], converted
 * exactly): the KV cache holds FP16 keys and values. */
QMM_API int qmm_quantize_f16(int type, const uint16_t *x, int64_t n, int64_t k, void *out, void *stream);

/*
 * Decode GEMV: y[b][j] = sum_i w[j][i] * x[b][i] for b < batch, j < n.
 * x: fp32 [batch][k], y: fp32 [batch][n], 1 <= batch <= 8 (batch 0 = empty).
 * Weights are read once from the quantized bytes and decoded in registers.
 * Every product uses the element's own weight (integer code offsets are
 * applied to the code before the multiply, K-quant weights d sc q - dmin m
 * are formed per element), so there is no cancellation after a rounding:
 * |y - exact| <= 2e-5 * sum_i |w[j][i] x[b][i]| for every output, and a row
 * of zero weights gives exactly 0.
 * Batch 1 (all types), batch 2..8 of Q8_0 / Q4_0 / Q5_0 / Q5_K and batch 2
 * of Q4_K / Q6_K with n < 65536: fp32 products and sums.  The other batches
 * 2..8 of Q4_K / Q6_K run on the fp16 matrix cores: per 256-element block and activation row, x is scaled by a power
 * of two and split into two fp16 parts (about 22 significant bits); Q6_K
 * weights enter as two exact fp16 integers ((q - 32) times the even part of
 * the int8 scale, and times its low bit), Q4_K weights as two fp16 parts of
 * the fp32 weight; sums are fp32.  On that
 * path an element of x smaller than about 2^-34 of the largest |x| of its
 * 256-element block keeps an absolute error of about 2^-50 of that largest
 * value (not a relative one): the bound above can fail only for rows whose
 * sum is carried by such elements.  x must be finite.  All paths are
 * deterministic.  (dotLLM "GPU Inference", Custom Kernels table:
 * quantized_gemv_* operating directly on quantized weights; the decode path
 * is memory-bandwidth bound.)
 */
QMM_API int qmm_gemv(int type, const void *w, int64_t n, int64_t k,
             const float *x, int64_t batch, float *y, void *stream);

/*
 * Grouped decode GEMV: for each problem i < nprob, y[i][b][j] =
 * sum_l w[i][j][l] * x[i][b][l], all problems sharing the block type, k and
 * batch -- e.g. the q, k, v projections or the gate and up projections of a
 * layer.  Small batch-1 problems then share one launch (up to 8 per launch)
 * instead of one launch each; shimmy "Airframe GPU pipeline" (dispatch
 * counts) already issues the FFN gate and up projections as one dispatch.
 * w, n, x, y are host arrays of nprob entries (device pointers / row counts),
 * read during the call only.  Per problem the same conventions and errors as
 * qmm_gemv apply; n[i] == 0 problems are skipped; nprob == 0 is a no-op.
 * Results are identical to nprob separate qmm_gemv calls.  When every x[i]
 * of a batch-1 call is the same pointer (q, k, v or gate, up reading one
 * activation), that x is staged once per workgroup, which is faster than
 * distinct x pointers holding equal values.
 */
QMM_API int qmm_gemv_multi(int type, int nprob, const void *const *w, const int64_t *n, int64_t k,
                           const float *const *x, int64_t batch, float *const *y, void *stream);

/*
 * Prefill GEMM: y[r][j] = sum_i x[r][i] * w[j][i] for r < m, j < n.
 * x: IEEE fp16 bit patterns [m][k], y: fp32 [m][n].  Weight tiles are decoded
 * to fp16 (round to nearest even) in on-chip memory and fed to fp16 matrix
 * cores with fp32 accumulation.  (dotLLM "GPU Inference", Future Work: a
 * fused quantized GEMM replacing dequant-to-scratch + FP16 GEMM for
 * prefill; shimmy "Airframe GPU pipeline": prompts are prefilled in
 * 512-token chunks.)
 * When m and n give too few output tiles to fill the GPU even with the
 * smaller tiles (e.g. m <= 128 with n = 4096, or m = 512 with n <= 2048 on
 * 256 compute units), K is split into up to 4
 * chunks whose partial sums are added into y with fp32 atomics after y is
 * zeroed on the same stream (two launches); the order of those additions
 * varies, so such results may differ between calls in the last bits
 * (always within the fp32 rounding of the sum).  512-token chunks with
 * n >= 4096 are not split and are deterministic.
 */
QMM_API int qmm_gemm_prefill(int type, const void *w, int64_t n, int64_t k,
                     const uint16_t *x, int64_t m, float *y, void *stream);

/*
 * Decode pass: the batch-1 GEMVs of one token, stage by stage.  (shimmy
 * "Airframe GPU pipeline", dispatch counts: a token's dispatches are encoded
 * in one command buffer, the FFN gate and up projections as one dispatch;
 * dotLLM "GPU Inference", Synchronization Model: one stream, no host sync
 * inside the forward pass; both pages: decode is bound by reading the
 * weights.)
 *
 * Problem i computes probs[i].y = W_i x_i as qmm_gemv at batch 1 (same
 * decode, same 2e-5 bound).  probs[i].stage must not decrease along the
 * array; problems with equal stage values form one stage, and every problem
 * of a stage is complete before any problem of a later stage reads its x,
 * so a later stage may read an earlier stage's y (o reading attention
 * output, down reading the gated FFN activation, ...).  Problems of one
 * stage must not write what another problem of the same stage reads.
 *
 * Launches: one per stage and x -- the problems of a stage that read the
 * same x (q / k / v, or gate / up) run as one launch even when their block
 * types differ (up to three types of up to eight problems each, of the same
 * lane-unit size: the 256-element K-quants, or the 32-element types), with
 * x staged once per workgroup; a problem whose k spans several lane-unit
 * segments (k > 4096 for the K-quants, > 2048 for the others) or whose rows
 * are not 16-byte multiples gets a launch of its own.  Each launch is
 * stream-ordered after the ones before it.
 *
 * Per problem the conventions and errors of qmm_gemv apply (w, x, y may be
 * NULL when n == 0; k == 0 writes zeros).  Any argument error returns before
 * anything is enqueued.
 */
typedef struct qmm_pass_gemv {
    const void *w;  /* device: n rows of qmm_row_bytes(type, k) bytes */
    const float *x; /* device: fp32 [k] */
    float *y;       /* device: fp32 [n] */
    int64_t n;
    int64_t k;
    int32_t type;   /* qmm_type */
    int32_t stage;  /* nondecreasing along the array */
} qmm_pass_gemv;

QMM_API int qmm_gemv_pass(int nprob, const qmm_pass_gemv *probs, void *stream);

/* Static text for a status code (never NULL). */
QMM_API const char *qmm_status_str(int status);

/* Library version string, e.g. "qmm 0.1.0 gfx950". */
QMM_API const char *qmm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H */
