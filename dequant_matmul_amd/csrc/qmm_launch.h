// qmm_launch.h -- internal launchers of libqmm (host side).  Arguments are
// already validated by the C-ABI layer (qmm_api.cpp): known type, k a
// multiple of the block size, n, k, m/batch/seq > 0, pointers non-null and
// 16-byte aligned (token ids: 4-byte aligned).  Each launcher only enqueues on stream s and returns the
// HIP status of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace qmm {

// A positive per-device value (a CU count, resident workgroups of a kernel)
// computed on first use for the current device and cached in slot[device].
// Relaxed atomics: concurrent first calls compute the same value, so a race
// only repeats the query.  Returns 0 if compute() fails (not cached).
template <class F>
inline int per_device_cached(std::atomic<int> (&slot)[64], F compute)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return compute();
    int v = slot[dev].load(std::memory_order_relaxed);
    if (v <= 0) {
        v = compute();
        if (v > 0)
            slot[dev].store(v, std::memory_order_relaxed);
    }
    return v > 0 ? v : 0;
}

// Compute units of the current device (0 if the runtime cannot tell).
inline int device_cu_count()
{
    static std::atomic<int> slot[64];
    return per_device_cached(slot, [] {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        return v;
    });
}

hipError_t launch_dequant(int type, const void *w, int64_t n, int64_t k, size_t rb, float *out,
                          hipStream_t s);

hipError_t launch_dequant_f16(int type, const void *w, int64_t n, int64_t k, size_t rb, uint16_t *out,
                              hipStream_t s);

// Embedding gather: out row r = dequant of table row ids[r] (zeros for an id
// outside [0, vocab)), r < seq.
hipError_t launch_embed(int type, const void *table, int64_t vocab, int64_t k, size_t rb, const int32_t *ids,
                        int64_t seq, float *out, hipStream_t s);
hipError_t launch_embed_f16(int type, const void *table, int64_t vocab, int64_t k, size_t rb,
                            const int32_t *ids, int64_t seq, uint16_t *out, hipStream_t s);

// Encoder (Q8_0 / Q4_0 only): x [n][k] -> n rows of row-bytes.
hipError_t launch_quantize(int type, const float *x, int64_t n, int64_t k, void *out, hipStream_t s);
hipError_t launch_quantize_f16(int type, const uint16_t *x, int64_t n, int64_t k, void *out, hipStream_t s);

hipError_t launch_gemv(int type, const void *w, int64_t n, int64_t k, size_t rb, const float *x,
                       int batch, float *y, hipStream_t s);

hipError_t launch_gemv_multi(int type, int np, const void *const *w, const int64_t *n, int64_t k, size_t rb,
                             const float *const *x, int batch, float *const *y, hipStream_t s);

// Batch 2..8 GEMV on the matrix cores (Q4_K, Q6_K); launch_gemv uses it for
// the batches and types that gemv_mfma_supported accepts.
bool gemv_mfma_supported(int type, int batch);
// np problems of one type and k sharing x [batch, k] on the matrix cores, one
// launch for up to eight of them (k <= 4096; gemv_mfma_multi_supported).
bool gemv_mfma_multi_supported(int type, int batch, int64_t k);
hipError_t launch_gemv_mfma_multi(int type, int np, const void *const *w, const int64_t *n, int64_t k, size_t rb,
                                  const float *x, int batch, float *const *y, hipStream_t s);
hipError_t launch_gemv_mfma(int type, const void *w, int64_t n, int64_t k, size_t rb, const float *x, int batch,
                            float *y, hipStream_t s);

hipError_t launch_gemm(int type, const void *w, int64_t n, int64_t k, size_t rb, const uint16_t *x,
                       int64_t m, float *y, hipStream_t s);

hipError_t launch_fill_zero(float *p, int64_t count, hipStream_t s);

// One stage of a decode pass in one launch (batch 1): ng <= 3 groups of
// problems, group g of block type type[g] with np[g] <= 8 problems (w, n, y
// listed group after group), every problem reading x (k elements, at most
// one lane-unit segment for its type); all types of a launch have the same
// lane-unit size (the 256-element types, or the 32-element ones).
constexpr int STAGE_GROUPS = 3;
constexpr int STAGE_PROBS = 8;
hipError_t launch_gemv_stage(int ng, const int *type, const int *np, const void *const *w, const int64_t *n,
                             int64_t k, const float *x, float *const *y, hipStream_t s);

}  // namespace qmm
