// qmm_api.cpp -- the C ABI of libqmm.so (declared in include/qmm.h): argument
// validation on the host, then kernel launches on the caller's stream.
// Nothing here allocates, synchronizes or keeps state.
#include <hip/hip_runtime.h>

#include "../../include/qmm.h"
#include "qmm_launch.h"

#include <vector>

namespace {

int block_elems(int t)
{
    switch (t) {
    case QMM_Q4_0: case QMM_Q8_0: case QMM_Q5_0: return 32;
    case QMM_Q4_K: case QMM_Q6_K: case QMM_Q5_K: return 256;
    default: return 0;
    }
}

int block_bytes(int t)
{
    switch (t) {
    case QMM_Q4_0: return 18;
    case QMM_Q8_0: return 34;
    case QMM_Q4_K: return 144;
    case QMM_Q6_K: return 210;
    case QMM_Q5_0: return 22;
    case QMM_Q5_K: return 176;
    default: return 0;
    }
}

// Elements per lane-unit of the GEMV decode: 64 for the 256-element
// super-blocks, 32 for the 32-element blocks.
int unit_elems(int t) { return block_elems(t) == 256 ? 64 : 32; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Shared checks; on success *rb holds the row size in bytes.
int check_common(int type, const void *w, int64_t n, int64_t k, size_t *rb)
{
    const int be = block_elems(type);
    if (be == 0)
        return QMM_ERR_TYPE;
    if (n < 0 || k < 0 || k % be != 0)
        return QMM_ERR_SHAPE;
    // keep every index the kernels form inside int32 element counts per row
    if (n > 0x7fffffff || k > 0x7fffffff)
        return QMM_ERR_SHAPE;
    *rb = (size_t)(k / be) * (size_t)block_bytes(type);
    if (n > 0 && k > 0) {
        if (w == nullptr)
            return QMM_ERR_NULL;
        if (!aligned16(w))
            return QMM_ERR_ALIGN;
    }
    return QMM_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? QMM_OK : QMM_ERR_HIP; }

}  // namespace

extern "C" {

int qmm_block_elems(int type) { return block_elems(type); }

int qmm_block_bytes(int type) { return block_bytes(type); }

size_t qmm_row_bytes(int type, int64_t k)
{
    const int be = block_elems(type);
    if (be == 0 || k < 0 || k % be != 0)
        return 0;
    return (size_t)(k / be) * (size_t)block_bytes(type);
}

int qmm_dequant(int type, const void *w, int64_t n, int64_t k, float *out, void *stream)
{
    size_t rb = 0;
    int st = check_common(type, w, n, k, &rb);
    if (st != QMM_OK)
        return st;
    if (n == 0 || k == 0)
        return QMM_OK;
    if (out == nullptr)
        return QMM_ERR_NULL;
    if (!aligned16(out))
        return QMM_ERR_ALIGN;
    return hip_status(qmm::launch_dequant(type, w, n, k, rb, out, (hipStream_t)stream));
}

int qmm_dequant_f16(int type, const void *w, int64_t n, int64_t k, uint16_t *out, void *stream)
{
    size_t rb = 0;
    int st = check_common(type, w, n, k, &rb);
    if (st != QMM_OK)
        return st;
    if (n == 0 || k == 0)
        return QMM_OK;
    if (out == nullptr)
        return QMM_ERR_NULL;
    if (!aligned16(out))
        return QMM_ERR_ALIGN;
    return hip_status(qmm::launch_dequant_f16(type, w, n, k, rb, out, (hipStream_t)stream));
}

// Shared checks of the two embedding gathers (the table is checked like a
// weight matrix of vocab rows).
static int check_embed(int type, const void *table, int64_t vocab, int64_t k, const int32_t *ids, int64_t seq,
                const void *out, size_t *rb)
{
    int st = check_common(type, table, vocab, k, rb);
    if (st != QMM_OK)
        return st;
    if (seq < 0 || seq > 0x7fffffff)
        return QMM_ERR_SHAPE;
    if (seq == 0 || k == 0)
        return QMM_OK;
    if (ids == nullptr || out == nullptr)
        return QMM_ERR_NULL;
    if (((uintptr_t)ids & 3u) != 0 || !aligned16(out))
        return QMM_ERR_ALIGN;
    return QMM_OK;
}

int qmm_embed(int type, const void *table, int64_t vocab, int64_t k, const int32_t *ids, int64_t seq, float *out,
              void *stream)
{
    size_t rb = 0;
    int st = check_embed(type, table, vocab, k, ids, seq, out, &rb);
    if (st != QMM_OK || seq == 0 || k == 0)
        return st;
    return hip_status(qmm::launch_embed(type, table, vocab, k, rb, ids, seq, out, (hipStream_t)stream));
}

int qmm_embed_f16(int type, const void *table, int64_t vocab, int64_t k, const int32_t *ids, int64_t seq,
                  uint16_t *out, void *stream)
{
    size_t rb = 0;
    int st = check_embed(type, table, vocab, k, ids, seq, out, &rb);
    if (st != QMM_OK || seq == 0 || k == 0)
        return st;
    return hip_status(qmm::launch_embed_f16(type, table, vocab, k, rb, ids, seq, out, (hipStream_t)stream));
}

// Shared checks of the two encoders (the output is checked like a weight
// matrix of n rows).
static int check_quantize(int type, const void *x, int64_t n, int64_t k, void *out, size_t *rb)
{
    if (type != QMM_Q8_0 && type != QMM_Q4_0)
        return QMM_ERR_TYPE;
    int st = check_common(type, out, n, k, rb);
    if (st != QMM_OK)
        return st;
    if (n == 0 || k == 0)
        return QMM_OK;
    if (x == nullptr)
        return QMM_ERR_NULL;
    if (!aligned16(x))
        return QMM_ERR_ALIGN;
    return QMM_OK;
}

int qmm_quantize(int type, const float *x, int64_t n, int64_t k, void *out, void *stream)
{
    size_t rb = 0;
    int st = check_quantize(type, x, n, k, out, &rb);
    if (st != QMM_OK || n == 0 || k == 0)
        return st;
    return hip_status(qmm::launch_quantize(type, x, n, k, out, (hipStream_t)stream));
}

int qmm_quantize_f16(int type, const uint16_t *x, int64_t n, int64_t k, void *out, void *stream)
{
    size_t rb = 0;
    int st = check_quantize(type, x, n, k, out, &rb);
    if (st != QMM_OK || n == 0 || k == 0)
        return st;
    return hip_status(qmm::launch_quantize_f16(type, x, n, k, out, (hipStream_t)stream));
}

int qmm_gemv(int type, const void *w, int64_t n, int64_t k, const float *x, int64_t batch, float *y,
             void *stream)
{
    size_t rb = 0;
    int st = check_common(type, w, n, k, &rb);
    if (st != QMM_OK)
        return st;
    if (batch < 0 || batch > 8)
        return QMM_ERR_SHAPE;
    if (n == 0 || batch == 0)
        return QMM_OK;
    if (y == nullptr || (k > 0 && x == nullptr))
        return QMM_ERR_NULL;
    if (!aligned16(y) || (k > 0 && !aligned16(x)))
        return QMM_ERR_ALIGN;
    if (k == 0)
        return hip_status(qmm::launch_fill_zero(y, batch * n, (hipStream_t)stream));
    return hip_status(qmm::launch_gemv(type, w, n, k, rb, x, (int)batch, y, (hipStream_t)stream));
}

int qmm_gemv_multi(int type, int nprob, const void *const *w, const int64_t *n, int64_t k,
                   const float *const *x, int64_t batch, float *const *y, void *stream)
{
    if (nprob < 0)
        return QMM_ERR_SHAPE;
    if (nprob == 0)
        return QMM_OK;
    if (w == nullptr || n == nullptr || x == nullptr || y == nullptr)
        return QMM_ERR_NULL;
    if (block_elems(type) == 0)
        return QMM_ERR_TYPE;
    if (batch < 0 || batch > 8)
        return QMM_ERR_SHAPE;
    size_t rb = 0;
    int64_t rows = 0;
    for (int i = 0; i < nprob; ++i) {
        int st = check_common(type, w[i], n[i], k, &rb);
        if (st != QMM_OK)
            return st;
        rows += n[i];
        if (n[i] == 0 || batch == 0)
            continue;
        if (y[i] == nullptr || (k > 0 && x[i] == nullptr))
            return QMM_ERR_NULL;
        if (!aligned16(y[i]) || (k > 0 && !aligned16(x[i])))
            return QMM_ERR_ALIGN;
    }
    if (batch == 0 || rows == 0)
        return QMM_OK;
    if (k == 0) {
        for (int i = 0; i < nprob; ++i) {
            if (n[i] == 0)
                continue;
            const int st = hip_status(qmm::launch_fill_zero(y[i], batch * n[i], (hipStream_t)stream));
            if (st != QMM_OK)
                return st;
        }
        return QMM_OK;
    }
    return hip_status(qmm::launch_gemv_multi(type, nprob, w, n, k, rb, x, (int)batch, y, (hipStream_t)stream));
}

int qmm_gemm_prefill(int type, const void *w, int64_t n, int64_t k, const uint16_t *x, int64_t m, float *y,
                     void *stream)
{
    size_t rb = 0;
    int st = check_common(type, w, n, k, &rb);
    if (st != QMM_OK)
        return st;
    if (m < 0 || m > 0x7fffffff)
        return QMM_ERR_SHAPE;
    if (n == 0 || m == 0)
        return QMM_OK;
    if (y == nullptr || (k > 0 && x == nullptr))
        return QMM_ERR_NULL;
    if (!aligned16(y) || (k > 0 && !aligned16(x)))
        return QMM_ERR_ALIGN;
    if (k == 0)
        return hip_status(qmm::launch_fill_zero(y, m * n, (hipStream_t)stream));
    return hip_status(qmm::launch_gemm(type, w, n, k, rb, x, m, y, (hipStream_t)stream));
}

int qmm_gemv_pass(int nprob, const qmm_pass_gemv *probs, void *stream)
{
    if (nprob < 0)
        return QMM_ERR_SHAPE;
    if (nprob == 0)
        return QMM_OK;
    if (probs == nullptr)
        return QMM_ERR_NULL;
    for (int i = 0; i < nprob; ++i) {
        const qmm_pass_gemv &P = probs[i];
        size_t rb = 0;
        const int st = check_common(P.type, P.w, P.n, P.k, &rb);
        if (st != QMM_OK)
            return st;
        if (P.stage < 0 || (i > 0 && P.stage < probs[i - 1].stage))
            return QMM_ERR_SHAPE;
        if (P.n == 0 || P.k == 0)
            continue;
        if (P.x == nullptr || P.y == nullptr)
            return QMM_ERR_NULL;
        if (!aligned16(P.x) || !aligned16(P.y))
            return QMM_ERR_ALIGN;
    }
    hipStream_t s = (hipStream_t)stream;
    std::vector<bool> done(nprob, false);
    for (int a = 0; a < nprob;) {
        int b = a;
        while (b < nprob && probs[b].stage == probs[a].stage)
            ++b;
        // stage [a, b): problems with rows, grouped by the x they read
        for (int i = a; i < b; ++i) {
            const qmm_pass_gemv &Pi = probs[i];
            if (done[i])
                continue;
            if (Pi.n == 0) {
                done[i] = true;
                continue;
            }
            if (Pi.k == 0) {
                done[i] = true;
                const int st = hip_status(qmm::launch_fill_zero(Pi.y, Pi.n, s));
                if (st != QMM_OK)
                    return st;
                continue;
            }
            // the problems of this stage reading the same x, with single-segment
            // 16-byte rows of the same lane-unit size: one launch (up to three
            // block types of up to eight problems each); any other problem:
            // its own launch
            const int ue = unit_elems(Pi.type);
            const size_t rbi = qmm_row_bytes(Pi.type, Pi.k);
            const bool one_seg = Pi.k <= 64 * ue && rbi % 16 == 0;
            if (!one_seg) {
                done[i] = true;
                const int st = hip_status(qmm::launch_gemv(Pi.type, Pi.w, Pi.n, Pi.k, rbi, Pi.x, 1, Pi.y, s));
                if (st != QMM_OK)
                    return st;
                continue;
            }
            int types[qmm::STAGE_GROUPS], np[qmm::STAGE_GROUPS], ng = 0;
            const void *w[qmm::STAGE_GROUPS * qmm::STAGE_PROBS];
            int64_t n[qmm::STAGE_GROUPS * qmm::STAGE_PROBS];
            float *y[qmm::STAGE_GROUPS * qmm::STAGE_PROBS];
            int members[qmm::STAGE_GROUPS][qmm::STAGE_PROBS];
            for (int j = i; j < b; ++j) {
                const qmm_pass_gemv &Pj = probs[j];
                if (done[j] || Pj.n == 0 || Pj.x != Pi.x || Pj.k != Pi.k || unit_elems(Pj.type) != ue ||
                    qmm_row_bytes(Pj.type, Pj.k) % 16 != 0)
                    continue;
                int g = 0;
                while (g < ng && types[g] != Pj.type)
                    ++g;
                if (g == ng) {
                    if (ng == qmm::STAGE_GROUPS)
                        continue;   // a later launch takes it
                    types[ng] = Pj.type;
                    np[ng++] = 0;
                }
                if (np[g] == qmm::STAGE_PROBS)
                    continue;
                members[g][np[g]++] = j;
                done[j] = true;
            }
            int total = 0;
            for (int g = 0; g < ng; ++g)
                total += np[g];
            if (total == 1) {
                const int j = members[0][0];
                const int st = hip_status(qmm::launch_gemv(probs[j].type, probs[j].w, probs[j].n, probs[j].k,
                                                           qmm_row_bytes(probs[j].type, probs[j].k), probs[j].x,
                                                           1, probs[j].y, s));
                if (st != QMM_OK)
                    return st;
                continue;
            }
            int c = 0;
            for (int g = 0; g < ng; ++g)
                for (int m = 0; m < np[g]; ++m, ++c) {
                    const qmm_pass_gemv &Pj = probs[members[g][m]];
                    w[c] = Pj.w;
                    n[c] = Pj.n;
                    y[c] = Pj.y;
                }
            const int st = hip_status(qmm::launch_gemv_stage(ng, types, np, w, n, Pi.k, Pi.x, y, s));
            if (st != QMM_OK)
                return st;
        }
        a = b;
    }
    return QMM_OK;
}

const char *qmm_status_str(int status)
{
    switch (status) {
    case QMM_OK: return "ok";
    case QMM_ERR_NULL: return "null pointer";
    case QMM_ERR_TYPE: return "unknown block type";
    case QMM_ERR_SHAPE: return "invalid shape";
    case QMM_ERR_ALIGN: return "pointer not 16-byte aligned";
    case QMM_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
    }
}

const char *qmm_version(void) { return "qmm 0.1.0 gfx950"; }

}  // extern "C"
