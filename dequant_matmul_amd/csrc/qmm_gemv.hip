// qmm_gemv.hip -- decode GEMV y[b] = W x[b] straight from quantized blocks.
//
// dotLLM "GPU Inference", cuBLAS GEMM/GEMV and Custom Kernels table: at
// seqLen = 1 every projection is a quantized GEMV that operates directly on
// the quantized weights and is memory-bandwidth bound; shimmy "Airframe GPU
// pipeline" (decode) says the same: reading the weight tensors dominates.
//
// gfx950 design
//   - A workgroup is 4 wavefronts; each wavefront owns R consecutive rows
//     and walks the whole K range in segments of 64 lane-units.
//   - Weights: for each segment and row the wave copies the row's bytes with
//     fully coalesced 16-byte loads (64 lanes x 16 B contiguous) into a
//     wave-private LDS buffer; each lane then reads its own unit (one Q8_0 /
//     Q4_0 block, or a 64-element quarter of a Q4_K / Q6_K super-block) from
//     LDS.  Blocks of 34, 18 and 210 bytes are only 2-byte aligned, so lanes
//     read aligned dwords and realign them with v_alignbyte_b32.
//   - Activations: the segment of x (all batches) is staged once per
//     workgroup in LDS, padded by 4 floats per unit so that the 64 lanes'
//     128-bit reads do not collide on banks.  A lane reads each x value once
//     per segment and applies it to all R rows of its wavefront.
//   - Codes are converted with one mask per dword plus v_cvt_f32_ubyteN (or
//     the sign-extending SDWA convert for Q8_0) and accumulated in fp32 per
//     block / sub-block; the scale is applied once per (sub-)block.  Constant
//     code offsets (-8, -32, -dmin*m) are applied through the per-sub-block
//     sum of x, which every row of the wave shares.
//   - The per-lane partial sums are reduced across the wavefront with
//     cross-lane shuffles; lane 0 writes y.
#include "qmm_device.h"
#include "qmm_launch.h"

namespace qmm {

template <int T> struct GemvUnit;
// UE: elements per lane-unit; a segment is 64 units.
template <> struct GemvUnit<T_Q4_0> { static constexpr int UE = 32; };
template <> struct GemvUnit<T_Q8_0> { static constexpr int UE = 32; };
template <> struct GemvUnit<T_Q4_K> { static constexpr int UE = 64; };
template <> struct GemvUnit<T_Q6_K> { static constexpr int UE = 64; };

// Read NDW dwords starting at an arbitrary even byte offset of an LDS byte
// buffer (given as dwords), realigning in registers.
template <int NDW>
__device__ __forceinline__ void lds_read_bytes(const uint32_t *lds, uint32_t byte_off, uint32_t *out)
{
    const uint32_t base = byte_off >> 2, sh = byte_off & 3u;
    uint32_t d[NDW + 1];
#pragma unroll
    for (int i = 0; i <= NDW; ++i)
        d[i] = lds[base + i];
#pragma unroll
    for (int i = 0; i < NDW; ++i)
        out[i] = align_bytes(d[i + 1], d[i], sh);
}

__device__ __forceinline__ uint32_t lds_read_u16(const uint32_t *lds, uint32_t byte_off)
{
    return (lds[byte_off >> 2] >> (8u * (byte_off & 2u))) & 0xffffu;
}

// Padded LDS index of element e of the x segment (4 floats of padding per
// lane-unit of UE elements).
template <int UE>
__device__ __forceinline__ int xpad(int e)
{
    return e + (e / UE) * 4;
}

template <int B>
__device__ __forceinline__ void load_x4(const float *xs, int stride, int idx, float4 *v)
{
#pragma unroll
    for (int b = 0; b < B; ++b)
        v[b] = *(const float4 *)(xs + b * stride + idx);
}

__device__ __forceinline__ float dot4_u(uint32_t q, const float4 &x, float acc)
{
    acc = __builtin_fmaf(ub0(q), x.x, acc);
    acc = __builtin_fmaf(ub1(q), x.y, acc);
    acc = __builtin_fmaf(ub2(q), x.z, acc);
    acc = __builtin_fmaf(ub3(q), x.w, acc);
    return acc;
}

__device__ __forceinline__ float dot4_s(uint32_t q, const float4 &x, float acc)
{
    acc = __builtin_fmaf(sb0(q), x.x, acc);
    acc = __builtin_fmaf(sb1(q), x.y, acc);
    acc = __builtin_fmaf(sb2(q), x.z, acc);
    acc = __builtin_fmaf(sb3(q), x.w, acc);
    return acc;
}

__device__ __forceinline__ float sum4(const float4 &v) { return (v.x + v.y) + (v.z + v.w); }

// One lane-unit for R rows and B batches.  wst: this wave's staged row
// segments (R of them, each SEGB bytes).  xs: staged x segment.  Adds each
// (row, batch) contribution to acc.
template <int T, int B, int R, int SEGB, int XS>
__device__ __forceinline__ void gemv_unit(const uint32_t *wst, const float *xs, int lane, float (&acc)[R][B])
{
    constexpr int UE = GemvUnit<T>::UE;
    const int xb = xpad<UE>(lane * UE);   // padded start of this lane's elements
    if constexpr (T == T_Q8_0) {
        // unit = one block: fp16 d at byte 34*lane, 32 int8 codes after it
        float d[R];
        uint32_t c[R][8];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t off = 34u * lane;
            d[r] = h2f(lds_read_u16(wst + r * (SEGB / 4), off));
            lds_read_bytes<8>(wst + r * (SEGB / 4), off + 2, c[r]);
        }
        float s[R][B];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) s[r][b] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float4 xv[B];
            load_x4<B>(xs, XS, xb + 4 * i, xv);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int b = 0; b < B; ++b) s[r][b] = dot4_s(c[r][i], xv[b], s[r][b]);
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[r][b] = __builtin_fmaf(d[r], s[r][b], acc[r][b]);
    } else if constexpr (T == T_Q4_0) {
        // unit = one block: fp16 d at byte 18*lane, 16 code bytes after it;
        // low nibble of byte i = element i, high nibble = element 16+i
        float d[R];
        uint32_t c[R][4];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t off = 18u * lane;
            d[r] = h2f(lds_read_u16(wst + r * (SEGB / 4), off));
            lds_read_bytes<4>(wst + r * (SEGB / 4), off + 2, c[r]);
        }
        float slo[R][B], shi[R][B], xsum[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            xsum[b] = 0.f;
#pragma unroll
            for (int r = 0; r < R; ++r) slo[r][b] = shi[r][b] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float4 xl[B], xh[B];
            load_x4<B>(xs, XS, xb + 4 * i, xl);
            load_x4<B>(xs, XS, xb + 16 + 4 * i, xh);
#pragma unroll
            for (int b = 0; b < B; ++b) xsum[b] += sum4(xl[b]) + sum4(xh[b]);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t lo = opaque(c[r][i] & 0x0f0f0f0fu);
                const uint32_t hi = opaque(c[r][i] & 0xf0f0f0f0u);  // 16 * code
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    slo[r][b] = dot4_u(lo, xl[b], slo[r][b]);
                    shi[r][b] = dot4_u(hi, xh[b], shi[r][b]);
                }
            }
        }
        // d * sum (q - 8) x = d * (slo + shi/16 - 8 * sum x)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const float t = __builtin_fmaf(shi[r][b], 0.0625f, slo[r][b]);
                acc[r][b] = __builtin_fmaf(d[r], __builtin_fmaf(-8.f, xsum[b], t), acc[r][b]);
            }
    } else if constexpr (T == T_Q4_K) {
        // unit = (super-block sb = lane/4, code group p = lane%4): sub-blocks
        // 2p (low nibbles) and 2p+1 (high nibbles) of 32 elements each
        const int sb = lane >> 2, p = lane & 3;
        float dsc0[R], dsc1[R], dm0[R], dm1[R];
        uint32_t c[R][8];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t *blk = wst + r * (SEGB / 4) + sb * 36;   // 144 B = 36 dwords
            const uint4 hd = *(const uint4 *)blk;
            const uint4 c0 = *(const uint4 *)(blk + 4 + 8 * p);
            const uint4 c1 = *(const uint4 *)(blk + 8 + 8 * p);
            c[r][0] = c0.x; c[r][1] = c0.y; c[r][2] = c0.z; c[r][3] = c0.w;
            c[r][4] = c1.x; c[r][5] = c1.y; c[r][6] = c1.z; c[r][7] = c1.w;
            uint32_t sc0, m0, sc1, m1;
            q4k_scale_min(hd.y, hd.z, hd.w, 2 * p, sc0, m0);
            q4k_scale_min(hd.y, hd.z, hd.w, 2 * p + 1, sc1, m1);
            const float d = h2f(hd.x & 0xffffu), dmin = h2f(hd.x >> 16);
            dsc0[r] = d * (float)sc0;
            dsc1[r] = d * (float)sc1 * 0.0625f;  // high nibbles convert as 16 q
            dm0[r] = dmin * (float)m0;
            dm1[r] = dmin * (float)m1;
        }
        float s0[R][B], s1[R][B], x0[B], x1[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            x0[b] = x1[b] = 0.f;
#pragma unroll
            for (int r = 0; r < R; ++r) s0[r][b] = s1[r][b] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float4 xl[B], xh[B];
            load_x4<B>(xs, XS, xb + 4 * i, xl);
            load_x4<B>(xs, XS, xb + 32 + 4 * i, xh);
#pragma unroll
            for (int b = 0; b < B; ++b) {
                x0[b] += sum4(xl[b]);
                x1[b] += sum4(xh[b]);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t lo = opaque(c[r][i] & 0x0f0f0f0fu);
                const uint32_t hi = opaque(c[r][i] & 0xf0f0f0f0u);
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    s0[r][b] = dot4_u(lo, xl[b], s0[r][b]);
                    s1[r][b] = dot4_u(hi, xh[b], s1[r][b]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) {
                float t = dsc0[r] * s0[r][b];
                t = __builtin_fmaf(dsc1[r], s1[r][b], t);
                t = __builtin_fmaf(-dm0[r], x0[b], t);
                t = __builtin_fmaf(-dm1[r], x1[b], t);
                acc[r][b] += t;
            }
    } else {  // Q6_K
        // unit = (super-block sb = lane/4, half h, l-range l0..l0+15): for
        // g = 0..3 the 16 elements 128h + 32g + l0 + i, i.e. sub-block
        // 8h + 2g + (l0/16); their low nibbles sit in ql[64h + l0 + i]
        // (g = 0 low, g = 2 high) and ql[64h + 32 + l0 + i] (g = 1 low,
        // g = 3 high), their high bits at bit 2g of qh[32h + l0 + i].
        const int sb = lane >> 2, u = lane & 3, h = u >> 1, hf = u & 1, l0 = 16 * hf;
        float dsc[R][4];
        uint32_t qa[R][4], qb[R][4], qh[R][4];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint32_t *rw = wst + r * (SEGB / 4);
            const uint32_t off = 210u * sb;
            lds_read_bytes<4>(rw, off + 64 * h + l0, qa[r]);
            lds_read_bytes<4>(rw, off + 64 * h + 32 + l0, qb[r]);
            lds_read_bytes<4>(rw, off + 128 + 32 * h + l0, qh[r]);
            uint32_t sc[2];
            lds_read_bytes<2>(rw, off + 192 + 8 * h, sc);
            const float d = h2f(lds_read_u16(rw, off + 208));
            const uint32_t sh = 8u * hf;
            dsc[r][0] = d * (float)(int8_t)(sc[0] >> sh);          // scale 8h + hf
            dsc[r][1] = d * (float)(int8_t)(sc[0] >> (16 + sh));   // scale 8h + 2 + hf
            dsc[r][2] = d * (float)(int8_t)(sc[1] >> sh);          // scale 8h + 4 + hf
            dsc[r][3] = d * (float)(int8_t)(sc[1] >> (16 + sh));   // scale 8h + 6 + hf
        }
        // element offset of (g, i) inside this lane's unit in the padded x
        // layout: the unit's elements are the 4 runs 128h + 32g + l0 + i of
        // super-block sb, i.e. segment elements 256 sb + 128 h + 32 g + l0 + i
        const int ebase = 256 * sb + 128 * h + l0;
        float s[R][B][4], xg[B][4];
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                xg[b][g] = 0.f;
#pragma unroll
                for (int r = 0; r < R; ++r) s[r][b][g] = 0.f;
            }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float4 xv[B];
                load_x4<B>(xs, XS, xpad<64>(ebase + 32 * g + 4 * i), xv);
#pragma unroll
                for (int b = 0; b < B; ++b) xg[b][g] += sum4(xv[b]);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint32_t a = qa[r][i], bq = qb[r][i], hb = qh[r][i];
                    uint32_t q;
                    if (g == 0) q = (a & 0x0f0f0f0fu) | ((hb & 0x03030303u) << 4);
                    else if (g == 1) q = (bq & 0x0f0f0f0fu) | ((hb & 0x0c0c0c0cu) << 2);
                    else if (g == 2) q = ((a >> 4) & 0x0f0f0f0fu) | (hb & 0x30303030u);
                    else q = ((bq >> 4) & 0x0f0f0f0fu) | ((hb >> 2) & 0x30303030u);
                    q = opaque(q);
#pragma unroll
                    for (int b = 0; b < B; ++b) s[r][b][g] = dot4_u(q, xv[b], s[r][b][g]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) {
                float t = 0.f;
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    t = __builtin_fmaf(dsc[r][g], __builtin_fmaf(-32.f, xg[b][g], s[r][b][g]), t);
                acc[r][b] += t;
            }
    }
}

template <int T, int B, int R, bool A16>
__global__ void __launch_bounds__(256)
gemv_kernel(const uint8_t *__restrict__ w, int n, int k, int64_t rb, const float *__restrict__ x,
            float *__restrict__ y)
{
    using F = Fmt<T>;
    constexpr int UE = GemvUnit<T>::UE;
    constexpr int SEGE = 64 * UE;                 // elements per segment
    constexpr int SEGB = SEGE / F::BE * F::BB;    // bytes of one row's segment
    constexpr int XS = SEGE + (SEGE / UE) * 4;    // padded floats per batch
    __shared__ __attribute__((aligned(16))) float xs[B * XS];
    __shared__ __attribute__((aligned(16))) uint32_t ws[4][R][SEGB / 4 + 4];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row0 = (blockIdx.x * 4 + wave) * R;
    float acc[R][B];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[r][b] = 0.f;

    const int nseg = (k + SEGE - 1) / SEGE;
    for (int seg = 0; seg < nseg; ++seg) {
        const int e0 = seg * SEGE;
        const int segE = min(SEGE, k - e0);
        const int segBytes = segE / F::BE * F::BB;
        __syncthreads();   // all reads of the previous segment are done
        // stage x[b][e0 .. e0+segE) (segE is a multiple of 32)
        for (int i4 = threadIdx.x; i4 < B * (segE >> 2); i4 += 256) {
            const int b = i4 / (segE >> 2), e = 4 * (i4 - b * (segE >> 2));
            const float4 v = *(const float4 *)(x + (int64_t)b * k + e0 + e);
            *(float4 *)(xs + b * XS + xpad<UE>(e)) = v;
        }
        // stage this wave's row segments
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = row0 + r;
            if (row < n) {
                const uint8_t *src = w + (int64_t)row * rb + (int64_t)seg * SEGB;
                if constexpr (A16) {
                    for (int c = lane; c < (segBytes >> 4); c += 64)
                        *(uint4 *)(&ws[wave][r][4 * c]) = *(const uint4 *)(src + 16 * c);
                } else {
                    uint16_t *dst = (uint16_t *)&ws[wave][r][0];
                    for (int c = lane; c < (segBytes >> 1); c += 64)
                        dst[c] = ((const uint16_t *)src)[c];
                }
            }
        }
        __syncthreads();
        if (lane < segE / UE)
            gemv_unit<T, B, R, 4 * (SEGB / 4 + 4), XS>(&ws[wave][0][0], xs, lane, acc);
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const float v = wave_sum(acc[r][b]);
            const int row = row0 + r;
            if (lane == 0 && row < n)
                y[(int64_t)b * n + row] = v;
        }
}

template <int T, int B, int R>
static hipError_t launch_tbr(const void *w, int64_t n, int64_t k, size_t rb, const float *x, float *y,
                             hipStream_t s)
{
    const dim3 grid((unsigned)((n + 4 * R - 1) / (4 * R))), block(256);
    const uint8_t *wb = (const uint8_t *)w;
    if (rb % 16 == 0)
        hipLaunchKernelGGL((gemv_kernel<T, B, R, true>), grid, block, 0, s, wb, (int)n, (int)k, (int64_t)rb, x, y);
    else
        hipLaunchKernelGGL((gemv_kernel<T, B, R, false>), grid, block, 0, s, wb, (int)n, (int)k, (int64_t)rb, x, y);
    return hipGetLastError();
}

template <int T>
static hipError_t launch_t(const void *w, int64_t n, int64_t k, size_t rb, const float *x, int batch, float *y,
                           hipStream_t s)
{
    switch (batch) {
    case 1: return launch_tbr<T, 1, 2>(w, n, k, rb, x, y, s);
    case 2: return launch_tbr<T, 2, 2>(w, n, k, rb, x, y, s);
    case 3: return launch_tbr<T, 3, 1>(w, n, k, rb, x, y, s);
    case 4: return launch_tbr<T, 4, 1>(w, n, k, rb, x, y, s);
    case 5: return launch_tbr<T, 5, 1>(w, n, k, rb, x, y, s);
    case 6: return launch_tbr<T, 6, 1>(w, n, k, rb, x, y, s);
    case 7: return launch_tbr<T, 7, 1>(w, n, k, rb, x, y, s);
    case 8: return launch_tbr<T, 8, 1>(w, n, k, rb, x, y, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv(int type, const void *w, int64_t n, int64_t k, size_t rb, const float *x, int batch,
                       float *y, hipStream_t s)
{
    switch (type) {
    case T_Q4_0: return launch_t<T_Q4_0>(w, n, k, rb, x, batch, y, s);
    case T_Q8_0: return launch_t<T_Q8_0>(w, n, k, rb, x, batch, y, s);
    case T_Q4_K: return launch_t<T_Q4_K>(w, n, k, rb, x, batch, y, s);
    case T_Q6_K: return launch_t<T_Q6_K>(w, n, k, rb, x, batch, y, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
