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
// Work split: one thread per 8 consecutive outputs of a row, so a wavefront
// stores 2 KB of contiguous fp32 (the kernel is bound by these writes: the
// output is 3.8x-7.1x the input bytes).  Inputs are read with naturally
// aligned 2- or 4-byte loads (blocks of 34, 18, 22 and 210 bytes are only 2-byte
// aligned); the reads hit in cache because neighbouring threads share blocks.
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

template <int T>
__global__ void __launch_bounds__(256)
dequant_kernel(const uint8_t *__restrict__ w, int64_t n, int64_t k, int64_t rb, float *__restrict__ out)
{
    using F = Fmt<T>;
    const int64_t per_row = k >> 3;
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g >= n * per_row)
        return;
    const int64_t row = g / per_row;
    const int e0 = (int)(g - row * per_row) * 8;  // first element (row-relative)
    const int b = e0 / F::BE;
    const int eb = e0 % F::BE;                     // first element inside the block
    const uint8_t *blk = w + row * rb + (int64_t)b * F::BB;
    float v[8];

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
    float4 *o = (float4 *)(out + row * k + e0);
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
}

hipError_t launch_dequant(int type, const void *w, int64_t n, int64_t k, size_t rb, float *out,
                          hipStream_t s)
{
    const int64_t threads = n * (k >> 3);
    const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    const uint8_t *wb = (const uint8_t *)w;
    switch (type) {
    case T_Q4_0: hipLaunchKernelGGL(dequant_kernel<T_Q4_0>, grid, block, 0, s, wb, n, k, (int64_t)rb, out); break;
    case T_Q8_0: hipLaunchKernelGGL(dequant_kernel<T_Q8_0>, grid, block, 0, s, wb, n, k, (int64_t)rb, out); break;
    case T_Q4_K: hipLaunchKernelGGL(dequant_kernel<T_Q4_K>, grid, block, 0, s, wb, n, k, (int64_t)rb, out); break;
    case T_Q6_K: hipLaunchKernelGGL(dequant_kernel<T_Q6_K>, grid, block, 0, s, wb, n, k, (int64_t)rb, out); break;
    case T_Q5_0: hipLaunchKernelGGL(dequant_kernel<T_Q5_0>, grid, block, 0, s, wb, n, k, (int64_t)rb, out); break;
    case T_Q5_K: hipLaunchKernelGGL(dequant_kernel<T_Q5_K>, grid, block, 0, s, wb, n, k, (int64_t)rb, out); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace qmm
