// qmm_gemm.hip -- prefill GEMM Y[m][n] = sum_k X[m][k] W[n][k] with W in
// quantized blocks, X in fp16, Y in fp32, on gfx950 matrix cores.
//
// dotLLM "GPU Inference", Weight Strategy / Future Work: prefill needs a dense
// FP16 contraction; instead of dequantizing a whole projection to an FP16
// scratch buffer and calling a library HGEMM, a fused kernel decodes the
// weights as it goes.  shimmy "Airframe GPU pipeline" prefills prompts in
// 512-token chunks; dequantization happens inline inside each matmul.
//
// gfx950 design (first version)
//   - Workgroup tile 128 (m) x 128 (n), K step 128; 4 wavefronts in a 2 x 2
//     grid, each owning a 64 x 64 sub-tile = 4 x 4 blocks of
//     v_mfma_f32_16x16x32_f16 with fp32 accumulators.
//   - Each K step, the workgroup decodes the 128 x 128 weight tile straight
//     from the quantized bytes (one 32-element group per thread-item) to fp32,
//     rounds to fp16 with round-to-nearest-even, and stores it in LDS as
//     [n][k]; the X tile is copied to LDS as [m][k].  Rows are padded by
//     8 halves so the 128-bit fragment reads are bank-conflict free.
//   - The global loads of step t+1 are issued before the MFMAs of step t
//     (register double buffering); the decode of step t+1 follows them.
//   - Ragged M, N and K are handled by zero-filling LDS outside the matrix and
//     masking the stores.
#include "qmm_device.h"
#include "qmm_launch.h"

namespace qmm {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int GBM = 128, GBN = 128, GBK = 128;
constexpr int GLD = GBK + 8;        // LDS row stride in halves
constexpr int GITEMS = GBN * (GBK / 32) / 256;   // 32-element weight groups per thread per step = 2

// NDW dwords from an even byte address p, realigned in registers, reading
// only bytes in [p - 2, p + 4*NDW): the last two bytes come from a 2-byte
// load when p is not 4-byte aligned, so nothing past the range is touched.
template <int NDW>
__device__ __forceinline__ void gload_bytes(const uint8_t *p, uint32_t *out)
{
    const uintptr_t a = (uintptr_t)p & ~(uintptr_t)3;
    const uint32_t sh = (uint32_t)((uintptr_t)p & 3u);
    const uint32_t *q = (const uint32_t *)a;
    uint32_t d[NDW + 1];
#pragma unroll
    for (int i = 0; i < NDW; ++i)
        d[i] = q[i];
    d[NDW] = sh ? (uint32_t)(*(const uint16_t *)(q + NDW)) : 0u;
#pragma unroll
    for (int i = 0; i < NDW; ++i)
        out[i] = align_bytes(d[i + 1], d[i], sh);
}

// Raw bytes of one 32-element weight group, as loaded from global memory.
template <int T> struct GRaw;
template <> struct GRaw<T_Q8_0> { uint32_t d; uint32_t c[8]; };
template <> struct GRaw<T_Q4_0> { uint32_t d; uint32_t c[4]; };
template <> struct GRaw<T_Q4_K> { uint32_t hd[4]; uint32_t c[8]; };
template <> struct GRaw<T_Q6_K> { uint32_t dsc; uint32_t ql[8]; uint32_t qh[8]; };

// Load group g (32 elements starting at element 32 g) of a row.
template <int T>
__device__ __forceinline__ void gload_group(const uint8_t *row, int g, GRaw<T> &r)
{
    using F = Fmt<T>;
    if constexpr (T == T_Q8_0) {
        const uint8_t *blk = row + (int64_t)g * F::BB;
        r.d = *(const uint16_t *)blk;
        gload_bytes<8>(blk + 2, r.c);
    } else if constexpr (T == T_Q4_0) {
        const uint8_t *blk = row + (int64_t)g * F::BB;
        r.d = *(const uint16_t *)blk;
        gload_bytes<4>(blk + 2, r.c);
    } else if constexpr (T == T_Q4_K) {
        const uint8_t *blk = row + (int64_t)(g >> 3) * F::BB;   // 16-byte aligned
        const int j = g & 7;
        const u32x4 h = *(const u32x4 *)blk;
        const u32x4 c0 = *(const u32x4 *)(blk + 16 + 32 * (j >> 1));
        const u32x4 c1 = *(const u32x4 *)(blk + 32 + 32 * (j >> 1));
        r.hd[0] = h.x; r.hd[1] = h.y; r.hd[2] = h.z; r.hd[3] = h.w;
        r.c[0] = c0.x; r.c[1] = c0.y; r.c[2] = c0.z; r.c[3] = c0.w;
        r.c[4] = c1.x; r.c[5] = c1.y; r.c[6] = c1.z; r.c[7] = c1.w;
    } else {
        // 32 elements (h, gq): e = 128h + 32gq + l, l = 0..31
        const uint8_t *blk = row + (int64_t)(g >> 3) * F::BB;
        const int part = g & 7, h = part >> 2, gq = part & 3;
        gload_bytes<8>(blk + 64 * h + 32 * (gq & 1), r.ql);
        gload_bytes<8>(blk + 128 + 32 * h, r.qh);
        // the two scales of this group (bytes 192 + 8h + 2gq, +1) and d
        const uint32_t s2 = *(const uint16_t *)(blk + 192 + 8 * h + 2 * gq);
        const uint32_t dd = *(const uint16_t *)(blk + 208);
        r.dsc = s2 | (dd << 16);
    }
}

__device__ __forceinline__ uint32_t pack2h(float a, float b)
{
    // round to nearest even (v_cvt_f16_f32), then pack
    const _Float16 ha = (_Float16)a, hb = (_Float16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// Decode the group's 32 weights to fp16 (as 16 dwords of packed halves).
template <int T>
__device__ __forceinline__ void decode_group(const GRaw<T> &r, int g, uint32_t *o)
{
    float v[32];
    if constexpr (T == T_Q8_0) {
        const float d = h2f(r.d);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[4 * i + 0] = d * sb0(r.c[i]); v[4 * i + 1] = d * sb1(r.c[i]);
            v[4 * i + 2] = d * sb2(r.c[i]); v[4 * i + 3] = d * sb3(r.c[i]);
        }
    } else if constexpr (T == T_Q4_0) {
        const float d = h2f(r.d);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = r.c[i] & 0x0f0f0f0fu, hi = (r.c[i] >> 4) & 0x0f0f0f0fu;
            v[4 * i + 0] = d * (ub0(lo) - 8.f); v[4 * i + 1] = d * (ub1(lo) - 8.f);
            v[4 * i + 2] = d * (ub2(lo) - 8.f); v[4 * i + 3] = d * (ub3(lo) - 8.f);
            v[16 + 4 * i + 0] = d * (ub0(hi) - 8.f); v[16 + 4 * i + 1] = d * (ub1(hi) - 8.f);
            v[16 + 4 * i + 2] = d * (ub2(hi) - 8.f); v[16 + 4 * i + 3] = d * (ub3(hi) - 8.f);
        }
    } else if constexpr (T == T_Q4_K) {
        const int j = g & 7;
        uint32_t sc, m;
        q4k_scale_min(r.hd[1], r.hd[2], r.hd[3], j, sc, m);
        const float dsc = h2f(r.hd[0] & 0xffffu) * (float)sc;
        const float dm = h2f(r.hd[0] >> 16) * (float)m;
        const uint32_t sh = (j & 1) ? 4u : 0u;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t q = (r.c[i] >> sh) & 0x0f0f0f0fu;
            v[4 * i + 0] = __builtin_fmaf(ub0(q), dsc, -dm); v[4 * i + 1] = __builtin_fmaf(ub1(q), dsc, -dm);
            v[4 * i + 2] = __builtin_fmaf(ub2(q), dsc, -dm); v[4 * i + 3] = __builtin_fmaf(ub3(q), dsc, -dm);
        }
    } else {
        const int part = g & 7, gq = part & 3;
        const float d = h2f(r.dsc >> 16);
        const float dsc0 = d * (float)(int8_t)(r.dsc & 0xffu);        // elements l = 0..15
        const float dsc1 = d * (float)(int8_t)((r.dsc >> 8) & 0xffu); // elements l = 16..31
        const uint32_t nsh = (gq >= 2) ? 4u : 0u, hsh = 2u * (uint32_t)gq;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t q = ((r.ql[i] >> nsh) & 0x0f0f0f0fu) | (((r.qh[i] >> hsh) & 0x03030303u) << 4);
            const float ds = (i < 4) ? dsc0 : dsc1;
            v[4 * i + 0] = ds * (ub0(q) - 32.f); v[4 * i + 1] = ds * (ub1(q) - 32.f);
            v[4 * i + 2] = ds * (ub2(q) - 32.f); v[4 * i + 3] = ds * (ub3(q) - 32.f);
        }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
        o[i] = pack2h(v[2 * i], v[2 * i + 1]);
}

template <int T>
__global__ void __launch_bounds__(256)
gemm_kernel(const uint8_t *__restrict__ w, int n, int k, int64_t rb, const uint16_t *__restrict__ x, int m,
            float *__restrict__ y)
{
    __shared__ __attribute__((aligned(16))) _Float16 As[GBM * GLD];
    __shared__ __attribute__((aligned(16))) _Float16 Bs[GBN * GLD];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int n0 = blockIdx.x * GBN, m0 = blockIdx.y * GBM;
    const int nk = (k + GBK - 1) / GBK;
    const int ngroups = k >> 5;

    // per-thread load assignment
    // X tile: 128 rows x 16 chunks of 8 halves -> 8 chunks per thread
    // W tile: 128 rows x 4 groups -> 2 items per thread (row = tid/2 + 0/64... )
    u32x4 xa[8];
    GRaw<T> wr[GITEMS];

    auto load_step = [&](int kt) __attribute__((always_inline)) {
        const int kb = kt * GBK;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = tid + 256 * i;          // 0..2047
            const int r = c >> 4, ch = c & 15;
            const int gm = m0 + r, gk = kb + 8 * ch;
            if (gm < m && gk < k)
                xa[i] = *(const u32x4 *)(x + (int64_t)gm * k + gk);
            else
                xa[i] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int it = 0; it < GITEMS; ++it) {
            const int item = tid + 256 * it;      // 0..511
            const int r = item >> 2, gl = item & 3;
            const int gn = n0 + r, g = (kb >> 5) + gl;
            if (gn < n && g < ngroups)
                gload_group<T>(w + (int64_t)gn * rb, g, wr[it]);
        }
    };

    auto store_step = [&](int kt) __attribute__((always_inline)) {
        const int kb = kt * GBK;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = tid + 256 * i;
            const int r = c >> 4, ch = c & 15;
            *(u32x4 *)(As + r * GLD + 8 * ch) = xa[i];
        }
#pragma unroll
        for (int it = 0; it < GITEMS; ++it) {
            const int item = tid + 256 * it;
            const int r = item >> 2, gl = item & 3;
            const int gn = n0 + r, g = (kb >> 5) + gl;
            uint32_t o[16];
            if (gn < n && g < ngroups) {
                decode_group<T>(wr[it], g, o);
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) o[i] = 0u;
            }
            u32x4 *dst = (u32x4 *)(Bs + r * GLD + 32 * gl);
            dst[0] = u32x4{o[0], o[1], o[2], o[3]};
            dst[1] = u32x4{o[4], o[5], o[6], o[7]};
            dst[2] = u32x4{o[8], o[9], o[10], o[11]};
            dst[3] = u32x4{o[12], o[13], o[14], o[15]};
        }
    };

    float4v acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = float4v{0.f, 0.f, 0.f, 0.f};

    load_step(0);
    for (int kt = 0; kt < nk; ++kt) {
        __syncthreads();
        store_step(kt);
        __syncthreads();
        if (kt + 1 < nk)
            load_step(kt + 1);
        const int fr = lane & 15, fk = 8 * (lane >> 4);
#pragma unroll
        for (int kk = 0; kk < GBK / 32; ++kk) {
            half8 a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = *(const half8 *)(As + (wm * 64 + 16 * i + fr) * GLD + 32 * kk + fk);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b[j] = *(const half8 *)(Bs + (wn * 64 + 16 * j + fr) * GLD + 32 * kk + fk);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }

    // C fragment: lane holds rows 4*(lane/16) + 0..3, column lane%16
    const int cr = 4 * (lane >> 4), cc = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int gn = n0 + wn * 64 + 16 * j + cc;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int gm = m0 + wm * 64 + 16 * i + cr + r;
                if (gm < m && gn < n)
                    y[(int64_t)gm * n + gn] = acc[i][j][r];
            }
        }
}

hipError_t launch_gemm(int type, const void *w, int64_t n, int64_t k, size_t rb, const uint16_t *x, int64_t m,
                       float *y, hipStream_t s)
{
    const dim3 grid((unsigned)((n + GBN - 1) / GBN), (unsigned)((m + GBM - 1) / GBM)), block(256);
    const uint8_t *wb = (const uint8_t *)w;
    switch (type) {
    case T_Q4_0: hipLaunchKernelGGL(gemm_kernel<T_Q4_0>, grid, block, 0, s, wb, (int)n, (int)k, (int64_t)rb, x, (int)m, y); break;
    case T_Q8_0: hipLaunchKernelGGL(gemm_kernel<T_Q8_0>, grid, block, 0, s, wb, (int)n, (int)k, (int64_t)rb, x, (int)m, y); break;
    case T_Q4_K: hipLaunchKernelGGL(gemm_kernel<T_Q4_K>, grid, block, 0, s, wb, (int)n, (int)k, (int64_t)rb, x, (int)m, y); break;
    case T_Q6_K: hipLaunchKernelGGL(gemm_kernel<T_Q6_K>, grid, block, 0, s, wb, (int)n, (int)k, (int64_t)rb, x, (int)m, y); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

__global__ void fill_zero_kernel(float *p, int64_t count)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < count)
        p[i] = 0.f;
}

hipError_t launch_fill_zero(float *p, int64_t count, hipStream_t s)
{
    if (count <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, p, count);
    return hipGetLastError();
}

}  // namespace qmm
