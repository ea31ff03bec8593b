// qmm_dequant.hip -- quantized blocks -> fp32, row-major [n][k], on gfx950.
//
// dotLLM "GPU Inference", Custom Kernels table: dequant_* kernels turn
// quantized weights into a dense array (there FP16 for a cuBLAS GEMM).  Here
// the output is fp32 and every value is the exact weight rounded once:
//   Q8_0  d q                 (11-bit x 8-bit product, exact in fp32)
//   Q4_0  d (q - 8)           (exact)
//   Q4_K  fma(q, d sc, -dmin m): d sc and dmin m are exact products, so the
//         single rounding of the fma is the rounding of the exact weight
//   Q6_K  (d sc) (q - 32)     (at most 23 significant bits, exact)
//   Q5_0  d (q - 16)          (exact)
//   Q5_K  fma(q, d sc, -dmin m) as Q4_K
// No division, reciprocal or fp16 intermediate is involved.
//
// The FP16 outputs (qmm_dequant_f16, qmm_embed_f16) round that fp32 value to
// nearest-even (v_cvt_pk_f16_f32), as the pages' dequant-to-FP16 kernels and
// FP16 hidden state do.
//
// The embedding gather (dotLLM "GPU Inference", Forward Pass step 2: the
// lookup kernel dequantizes the rows of the given token ids) is the same
// kernel with the source row taken from the id list; an id outside the table
// produces a row of +0.
//
// Work split: one thread per 8 consecutive outputs of a row, so a wavefront
// stores 2 KB of contiguous fp32 (1 KB of fp16); the kernel is bound by these
// writes (the fp32 output is 3.8x-7.1x the input bytes).  Inputs are read
// with naturally aligned 2- or 4-byte loads (blocks of 34, 18, 22 and 210
// bytes are only 2-byte aligned); the reads hit in cache because
// neighbouring threads share blocks.  The grid is capped and strides over the
// outputs, so any size stays within the 32-bit dispatch limits.
#include "qmm_device.h"
#include "qmm_launch.h"

namespace qmm {

__device__ __forceinline__ uint32_t ld16(const uint8_t *p)
{
    return *(const uint16_t *)p;
}

// Four 2-byte aligned loads -> 8 consecutive bytes as two dwords.
__device__ __forceinline__ void ld8_u16(const uint8_t *p, uint32_t &lo, uint32_t &hi)
{
    const uint16_t *q = (const uint16_t *)p;
    lo = (uint32_t)q[0] | ((uint32_t)q[1] << 16);
    hi = (uint32_t)q[2] | ((uint32_t)q[3] << 16);
}

// The 8 weights of block blk starting at element eb (a multiple of 8).
template <int T>
__device__ __forceinline__ void decode8(const uint8_t *blk, int eb, float v[8])
{
    if constexpr (T == T_Q8_0) {
        const float d = h2f(ld16(blk));
        uint32_t c0, c1;
        ld8_u16(blk + 2 + eb, c0, c1);
        v[0] = d * sb0(c0); v[1] = d * sb1(c0); v[2] = d * sb2(c0); v[3] = d * sb3(c0);
        v[4] = d * sb0(c1); v[5] = d * sb1(c1); v[6] = d * sb2(c1); v[7] = d * sb3(c1);
    } else if constexpr (T == T_Q4_0) {
        const float d = h2f(ld16(blk));
        uint32_t c0, c1;
        ld8_u16(blk + 2 + (eb & 15), c0, c1);
        if (eb >= 16) {   // high nibbles hold elements 16..31
            c0 >>= 4;
            c1 >>= 4;
        }
        c0 &= 0x0f0f0f0fu;
        c1 &= 0x0f0f0f0fu;
        v[0] = d * (ub0(c0) - 8.f); v[1] = d * (ub1(c0) - 8.f);
        v[2] = d * (ub2(c0) - 8.f); v[3] = d * (ub3(c0) - 8.f);
        v[4] = d * (ub0(c1) - 8.f); v[5] = d * (ub1(c1) - 8.f);
        v[6] = d * (ub2(c1) - 8.f); v[7] = d * (ub3(c1) - 8.f);
    } else if constexpr (T == T_Q4_K) {
        // 144-byte blocks keep 16-byte alignment: dword loads are natural.
        const uint32_t *hd = (const uint32_t *)blk;
        const uint32_t dd = hd[0], s0 = hd[1], s1 = hd[2], s2 = hd[3];
        const int j = eb >> 5, l0 = eb & 31;
        uint32_t sc, m;
        q4k_scale_min(s0, s1, s2, j, sc, m);
        const float dsc = h2f(dd & 0xffffu) * (float)sc;
        const float dm = h2f(dd >> 16) * (float)m;
        const uint32_t *cs = (const uint32_t *)(blk + 16 + 32 * (j >> 1) + l0);
        uint32_t c0 = cs[0], c1 = cs[1];
        if (j & 1) {
            c0 >>= 4;
            c1 >>= 4;
        }
        c0 &= 0x0f0f0f0fu;
        c1 &= 0x0f0f0f0fu;
        v[0] = __builtin_fmaf(ub0(c0), dsc, -dm); v[1] = __builtin_fmaf(ub1(c0), dsc, -dm);
        v[2] = __builtin_fmaf(ub2(c0), dsc, -dm); v[3] = __builtin_fmaf(ub3(c0), dsc, -dm);
        v[4] = __builtin_fmaf(ub0(c1), dsc, -dm); v[5] = __builtin_fmaf(ub1(c1), dsc, -dm);
        v[6] = __builtin_fmaf(ub2(c1), dsc, -dm); v[7] = __builtin_fmaf(ub3(c1), dsc, -dm);
    } else if constexpr (T == T_Q5_0) {
        // 22-byte blocks: 2-byte aligned loads only
        const float d = h2f(ld16(blk));
        const uint32_t hbits = ld16(blk + 2) | (ld16(blk + 4) << 16);
        uint32_t c0, c1;
        ld8_u16(blk + 6 + (eb & 15), c0, c1);
        if (eb >= 16) {
            c0 >>= 4;
            c1 >>= 4;
        }
        const uint32_t hb = hbits >> eb;   // bits of elements eb .. eb+7
        c0 = (c0 & 0x0f0f0f0fu) | bits_to_byte_bit4(hb);
        c1 = (c1 & 0x0f0f0f0fu) | bits_to_byte_bit4(hb >> 4);
        v[0] = d * (ub0(c0) - 16.f); v[1] = d * (ub1(c0) - 16.f);
        v[2] = d * (ub2(c0) - 16.f); v[3] = d * (ub3(c0) - 16.f);
        v[4] = d * (ub0(c1) - 16.f); v[5] = d * (ub1(c1) - 16.f);
        v[6] = d * (ub2(c1) - 16.f); v[7] = d * (ub3(c1) - 16.f);
    } else if constexpr (T == T_Q5_K) {
        // 176-byte blocks keep 16-byte alignment
        const uint32_t *hd = (const uint32_t *)blk;
        const uint32_t dd = hd[0], s0 = hd[1], s1 = hd[2], s2 = hd[3];
        const int j = eb >> 5, l0 = eb & 31;
        uint32_t sc, m;
        q4k_scale_min(s0, s1, s2, j, sc, m);
        const float dsc = h2f(dd & 0xffffu) * (float)sc;
        const float dm = h2f(dd >> 16) * (float)m;
        const uint32_t *qh = (const uint32_t *)(blk + 16 + l0);
        const uint32_t *cs = (const uint32_t *)(blk + 48 + 32 * (j >> 1) + l0);
        uint32_t c0 = cs[0], c1 = cs[1];
        if (j & 1) {
            c0 >>= 4;
            c1 >>= 4;
        }
        c0 = (c0 & 0x0f0f0f0fu) | (((qh[0] >> j) & 0x01010101u) << 4);
        c1 = (c1 & 0x0f0f0f0fu) | (((qh[1] >> j) & 0x01010101u) << 4);
        v[0] = __builtin_fmaf(ub0(c0), dsc, -dm); v[1] = __builtin_fmaf(ub1(c0), dsc, -dm);
        v[2] = __builtin_fmaf(ub2(c0), dsc, -dm); v[3] = __builtin_fmaf(ub3(c0), dsc, -dm);
        v[4] = __builtin_fmaf(ub0(c1), dsc, -dm); v[5] = __builtin_fmaf(ub1(c1), dsc, -dm);
        v[6] = __builtin_fmaf(ub2(c1), dsc, -dm); v[7] = __builtin_fmaf(ub3(c1), dsc, -dm);
    } else {  // Q6_K
        const int h = eb >> 7, r = eb & 127, gq = r >> 5, l0 = r & 31;
        uint32_t l_lo, l_hi, h_lo, h_hi;
        ld8_u16(blk + 64 * h + 32 * (gq & 1) + l0, l_lo, l_hi);
        ld8_u16(blk + 128 + 32 * h + l0, h_lo, h_hi);
        if (gq >= 2) {   // g = 2, 3 use the high nibbles of ql
            l_lo >>= 4;
            l_hi >>= 4;
        }
        const uint32_t sh = 2u * (uint32_t)gq;
        const uint32_t q0 = (l_lo & 0x0f0f0f0fu) | (((h_lo >> sh) & 0x03030303u) << 4);
        const uint32_t q1 = (l_hi & 0x0f0f0f0fu) | (((h_hi >> sh) & 0x03030303u) << 4);
        const int si = 192 + (eb >> 4);
        const uint32_t sw = ld16(blk + (si & ~1));
        const float sc = (float)(int8_t)(sw >> (8 * (si & 1)));
        const float dsc = h2f(ld16(blk + 208)) * sc;
        v[0] = dsc * (ub0(q0) - 32.f); v[1] = dsc * (ub1(q0) - 32.f);
        v[2] = dsc * (ub2(q0) - 32.f); v[3] = dsc * (ub3(q0) - 32.f);
        v[4] = dsc * (ub0(q1) - 32.f); v[5] = dsc * (ub1(q1) - 32.f);
        v[6] = dsc * (ub2(q1) - 32.f); v[7] = dsc * (ub3(q1) - 32.f);
    }
}

__device__ __forceinline__ void store8(float *o, const float v[8])
{
    float4 *p = (float4 *)o;
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
}

typedef float f2v __attribute__((ext_vector_type(2)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));

// fp16_RNE of two fp32 values, packed (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_h2(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){a, b}, h2v));
}

__device__ __forceinline__ void store8(uint16_t *o, const float v[8])
{
    *(uint4 *)o = make_uint4(pack_h2(v[0], v[1]), pack_h2(v[2], v[3]), pack_h2(v[4], v[5]), pack_h2(v[6], v[7]));
}

// Output row r (r < n) = source row r, or with GATHER source row ids[r]
// (a row of zeros when that id is outside [0, vocab)).
template <int T, typename O, bool GATHER>
__global__ void __launch_bounds__(256)
dequant_kernel(const uint8_t *__restrict__ w, int64_t n, int64_t k, int64_t rb, const int32_t *__restrict__ ids,
               int64_t vocab, O *__restrict__ out)
{
    using F = Fmt<T>;
    const int64_t per_row = k >> 3;
    const int64_t total = n * per_row;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < total; g += stride) {
        const int64_t row = g / per_row;
        const int e0 = (int)(g - row * per_row) * 8;  // first element (row-relative)
        float v[8];
        int64_t src = row;
        bool valid = true;
        if constexpr (GATHER) {
            src = ids[row];
            valid = src >= 0 && src < vocab;
        }
        if (valid) {
            const uint8_t *blk = w + src * rb + (int64_t)(e0 / F::BE) * F::BB;
            decode8<T>(blk, e0 % F::BE, v);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = 0.f;
        }
        store8(out + row * k + e0, v);
    }
}

namespace {

template <typename O, bool GATHER>
hipError_t launch_any(int type, const void *w, int64_t n, int64_t k, size_t rb, const int32_t *ids,
                      int64_t vocab, O *out, hipStream_t s)
{
    const int64_t threads = n * (k >> 3);
    const int64_t blocks = (threads + 255) / 256;
    // at most 2^20 workgroups (2^28 work-items); larger problems stride
    const dim3 grid((unsigned)(blocks < (1 << 20) ? blocks : (1 << 20))), block(256);
    const uint8_t *wb = (const uint8_t *)w;
    const int64_t r = (int64_t)rb;
    switch (type) {
    case T_Q4_0: hipLaunchKernelGGL((dequant_kernel<T_Q4_0, O, GATHER>), grid, block, 0, s, wb, n, k, r, ids, vocab, out); break;
    case T_Q8_0: hipLaunchKernelGGL((dequant_kernel<T_Q8_0, O, GATHER>), grid, block, 0, s, wb, n, k, r, ids, vocab, out); break;
    case T_Q4_K: hipLaunchKernelGGL((dequant_kernel<T_Q4_K, O, GATHER>), grid, block, 0, s, wb, n, k, r, ids, vocab, out); break;
    case T_Q6_K: hipLaunchKernelGGL((dequant_kernel<T_Q6_K, O, GATHER>), grid, block, 0, s, wb, n, k, r, ids, vocab, out); break;
    case T_Q5_0: hipLaunchKernelGGL((dequant_kernel<T_Q5_0, O, GATHER>), grid, block, 0, s, wb, n, k, r, ids, vocab, out); break;
    case T_Q5_K: hipLaunchKernelGGL((dequant_kernel<T_Q5_K, O, GATHER>), grid, block, 0, s, wb, n, k, r, ids, vocab, out); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant(int type, const void *w, int64_t n, int64_t k, size_t rb, float *out, hipStream_t s)
{
    return launch_any<float, false>(type, w, n, k, rb, nullptr, n, out, s);
}

hipError_t launch_dequant_f16(int type, const void *w, int64_t n, int64_t k, size_t rb, uint16_t *out,
                              hipStream_t s)
{
    return launch_any<uint16_t, false>(type, w, n, k, rb, nullptr, n, out, s);
}

hipError_t launch_embed(int type, const void *table, int64_t vocab, int64_t k, size_t rb, const int32_t *ids,
                        int64_t seq, float *out, hipStream_t s)
{
    return launch_any<float, true>(type, table, seq, k, rb, ids, vocab, out, s);
}

hipError_t launch_embed_f16(int type, const void *table, int64_t vocab, int64_t k, size_t rb,
                            const int32_t *ids, int64_t seq, uint16_t *out, hipStream_t s)
{
    return launch_any<uint16_t, true>(type, table, seq, k, rb, ids, vocab, out, s);
}

}  // namespace qmm
