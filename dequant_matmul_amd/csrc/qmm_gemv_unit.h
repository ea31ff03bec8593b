// qmm_gemv_unit.h -- the lane-unit decode of the batch-1..8 VALU GEMV
// kernels (qmm_gemv.hip) and the decode-pass kernel (qmm_pass.hip): unit
// layout of each block type, the raw bytes of one lane-unit (from LDS or
// global memory), the per-unit dot product with x, and the row-segment
// staging through LDS.
//
// A lane-unit is one Q8_0 / Q4_0 / Q5_0 block (32 elements) or a 64-element
// quarter of a Q4_K / Q5_K / Q6_K super-block; a segment is 64 consecutive
// units of a row, one per lane of a wavefront.  Block layouts: shimmy
// "Architecture", Quantization table; dotLLM "GPU Inference", Quantization on
// GPU table (byte layouts as read with the workload definitions).
#pragma once

#include "qmm_device.h"

namespace qmm {

// ------------------------------------------------------------ unit layout --

template <int T> struct GemvUnit;
// UE: elements per lane-unit; NRUN: runs of 4 consecutive elements per unit.
template <> struct GemvUnit<T_Q4_0> { static constexpr int UE = 32, NRUN = 8; };
template <> struct GemvUnit<T_Q8_0> { static constexpr int UE = 32, NRUN = 8; };
template <> struct GemvUnit<T_Q4_K> { static constexpr int UE = 64, NRUN = 16; };
template <> struct GemvUnit<T_Q6_K> { static constexpr int UE = 64, NRUN = 16; };
template <> struct GemvUnit<T_Q5_0> { static constexpr int UE = 32, NRUN = 8; };
template <> struct GemvUnit<T_Q5_K> { static constexpr int UE = 64, NRUN = 16; };

// Element (relative to the segment start) of the first element of run j of
// lane-unit u.  The run order is the order in which unit_dot consumes x.
template <int T>
__device__ __forceinline__ int run_elem(int u, int j)
{
    if constexpr (T == T_Q8_0) {
        return 32 * u + 4 * j;                                // codes 4j..4j+3
    } else if constexpr (T == T_Q4_0 || T == T_Q5_0) {
        return 32 * u + (j < 4 ? 4 * j : 16 + 4 * (j - 4));   // low nibbles, then high
    } else if constexpr (T == T_Q4_K || T == T_Q5_K) {
        return 64 * u + (j < 8 ? 4 * j : 32 + 4 * (j - 8));   // sub-block 2p, then 2p+1
    } else {
        // u = 4 sb + 2 h + hf: elements 128h + 32g + 16hf + i of super-block sb,
        // run j = 4g + i/4
        const int sb = u >> 2, h = (u >> 1) & 1, hf = u & 1;
        return 256 * sb + 128 * h + 16 * hf + 32 * (j >> 2) + 4 * (j & 3);
    }
}

// Padded LDS index of element e of an x segment: 4 floats of padding per
// lane-unit, so the 64 lanes' 128-bit reads do not collide on banks.
template <int UE>
__device__ __forceinline__ int xpad(int e)
{
    return e + (e / UE) * 4;
}

// Raw bytes of one lane-unit of one row.
template <int T> struct URaw;
template <> struct URaw<T_Q8_0> { uint32_t d; uint32_t c[8]; };
template <> struct URaw<T_Q4_0> { uint32_t d; uint32_t c[4]; };
template <> struct URaw<T_Q4_K> { u32x4 hd; uint32_t c[8]; };
template <> struct URaw<T_Q6_K> { uint32_t qa[4], qb[4], qh[4], sc[2], d; };
template <> struct URaw<T_Q5_0> { uint32_t d; uint32_t qh; uint32_t c[4]; };
template <> struct URaw<T_Q5_K> { u32x4 hd; uint32_t h[8]; uint32_t c[8]; };

// Read NDW dwords starting at an even byte offset of an LDS byte buffer
// (addressed as dwords), realigning in registers.
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

// Unit u of a row segment staged in LDS (raw bytes from offset 0).
template <int T>
__device__ __forceinline__ void raw_from_lds(const uint32_t *seg, int u, URaw<T> &r)
{
    if constexpr (T == T_Q8_0) {
        const uint32_t off = 34u * u;               // fp16 d, then 32 int8 codes
        r.d = lds_read_u16(seg, off);
        lds_read_bytes<8>(seg, off + 2, r.c);
    } else if constexpr (T == T_Q4_0) {
        const uint32_t off = 18u * u;               // fp16 d, then 16 code bytes
        r.d = lds_read_u16(seg, off);
        lds_read_bytes<4>(seg, off + 2, r.c);
    } else if constexpr (T == T_Q5_0) {
        const uint32_t off = 22u * u;               // fp16 d, 32 high bits, 16 code bytes
        uint32_t t[5];
        r.d = lds_read_u16(seg, off);
        lds_read_bytes<5>(seg, off + 2, t);
        r.qh = t[0];
        r.c[0] = t[1]; r.c[1] = t[2]; r.c[2] = t[3]; r.c[3] = t[4];
    } else if constexpr (T == T_Q5_K) {
        const int p = u & 3;
        const uint32_t *blk = seg + 44 * (u >> 2);  // 176 B = 44 dwords
        r.hd = *(const u32x4 *)blk;
        const u32x4 h0 = *(const u32x4 *)(blk + 4), h1 = *(const u32x4 *)(blk + 8);
        const u32x4 c0 = *(const u32x4 *)(blk + 12 + 8 * p), c1 = *(const u32x4 *)(blk + 16 + 8 * p);
        r.h[0] = h0.x; r.h[1] = h0.y; r.h[2] = h0.z; r.h[3] = h0.w;
        r.h[4] = h1.x; r.h[5] = h1.y; r.h[6] = h1.z; r.h[7] = h1.w;
        r.c[0] = c0.x; r.c[1] = c0.y; r.c[2] = c0.z; r.c[3] = c0.w;
        r.c[4] = c1.x; r.c[5] = c1.y; r.c[6] = c1.z; r.c[7] = c1.w;
    } else if constexpr (T == T_Q4_K) {
        const int p = u & 3;
        const uint32_t *blk = seg + 36 * (u >> 2);  // 144 B = 36 dwords
        r.hd = *(const u32x4 *)blk;
        const u32x4 c0 = *(const u32x4 *)(blk + 4 + 8 * p);
        const u32x4 c1 = *(const u32x4 *)(blk + 8 + 8 * p);
        r.c[0] = c0.x; r.c[1] = c0.y; r.c[2] = c0.z; r.c[3] = c0.w;
        r.c[4] = c1.x; r.c[5] = c1.y; r.c[6] = c1.z; r.c[7] = c1.w;
    } else {
        const int sb = u >> 2, h = (u >> 1) & 1, hf = u & 1, l0 = 16 * hf;
        const uint32_t off = 210u * sb;
        lds_read_bytes<4>(seg, off + 64 * h + l0, r.qa);        // ql, g = 0 (low) / 2 (high)
        lds_read_bytes<4>(seg, off + 64 * h + 32 + l0, r.qb);   // ql, g = 1 (low) / 3 (high)
        lds_read_bytes<4>(seg, off + 128 + 32 * h + l0, r.qh);  // qh, bits 2g
        lds_read_bytes<2>(seg, off + 192 + 8 * h, r.sc);        // scales 8h .. 8h+7
        r.d = lds_read_u16(seg, off + 208);
    }
}

// ------------------------------------------------------------- unit dot --

__device__ __forceinline__ float dot4_u(uint32_t q, const f32x4 &x, float acc)
{
    acc = __builtin_fmaf(ub0(q), x.x, acc);
    acc = __builtin_fmaf(ub1(q), x.y, acc);
    acc = __builtin_fmaf(ub2(q), x.z, acc);
    acc = __builtin_fmaf(ub3(q), x.w, acc);
    return acc;
}

__device__ __forceinline__ float dot4_s(uint32_t q, const f32x4 &x, float acc)
{
    acc = __builtin_fmaf(sb0(q), x.x, acc);
    acc = __builtin_fmaf(sb1(q), x.y, acc);
    acc = __builtin_fmaf(sb2(q), x.z, acc);
    acc = __builtin_fmaf(sb3(q), x.w, acc);
    return acc;
}

__device__ __forceinline__ float sum4(const f32x4 &v) { return (v.x + v.y) + (v.z + v.w); }

// Batch 1 keeps four partial sums per accumulator (one per byte position):
// four independent FMA chains instead of one long dependent chain, which at
// a few waves per SIMD is bound by the FMA latency.  Larger batches already
// have B independent chains.
__device__ __forceinline__ f32x4 dot4_u(uint32_t q, const f32x4 &x, f32x4 acc)
{
    acc.x = __builtin_fmaf(ub0(q), x.x, acc.x);
    acc.y = __builtin_fmaf(ub1(q), x.y, acc.y);
    acc.z = __builtin_fmaf(ub2(q), x.z, acc.z);
    acc.w = __builtin_fmaf(ub3(q), x.w, acc.w);
    return acc;
}

__device__ __forceinline__ f32x4 dot4_s(uint32_t q, const f32x4 &x, f32x4 acc)
{
    acc.x = __builtin_fmaf(sb0(q), x.x, acc.x);
    acc.y = __builtin_fmaf(sb1(q), x.y, acc.y);
    acc.z = __builtin_fmaf(sb2(q), x.z, acc.z);
    acc.w = __builtin_fmaf(sb3(q), x.w, acc.w);
    return acc;
}

template <int B> struct AccOf { typedef float type; };
template <> struct AccOf<1> { typedef f32x4 type; };
__device__ __forceinline__ float fin(float v) { return v; }
__device__ __forceinline__ float fin(const f32x4 &v) { return sum4(v); }
template <class A> __device__ __forceinline__ A zero_acc();
template <> __device__ __forceinline__ float zero_acc<float>() { return 0.f; }
template <> __device__ __forceinline__ f32x4 zero_acc<f32x4>() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// x of run j for batch b, from LDS (padded layout) ...
template <int T, int XS>
struct XFromLds {
    const float *xs;
    int u;
    __device__ __forceinline__ f32x4 operator()(int j, int b) const
    {
        return *(const f32x4 *)(xs + b * XS + xpad<GemvUnit<T>::UE>(run_elem<T>(u, j)));
    }
};

// ... or from registers (batch 1): the lane's unit is the same for every row.
template <int T>
struct XFromRegs {
    const f32x4 *xr;
    __device__ __forceinline__ f32x4 operator()(int j, int) const { return xr[j]; }
};

// Weights of four elements with unsigned codes q_c (bytes of q): each is
// d sc q - dmin m rounded once, exactly as the dequantizer forms it.
__device__ __forceinline__ f32x4 wts4(uint32_t q, float dsc, float ndm)
{
    return f32x4{__builtin_fmaf(ub0(q), dsc, ndm), __builtin_fmaf(ub1(q), dsc, ndm),
                 __builtin_fmaf(ub2(q), dsc, ndm), __builtin_fmaf(ub3(q), dsc, ndm)};
}

__device__ __forceinline__ float dot4_f(const f32x4 &w, const f32x4 &x, float acc)
{
    acc = __builtin_fmaf(w.x, x.x, acc);
    acc = __builtin_fmaf(w.y, x.y, acc);
    acc = __builtin_fmaf(w.z, x.z, acc);
    acc = __builtin_fmaf(w.w, x.w, acc);
    return acc;
}

__device__ __forceinline__ f32x4 dot4_f(const f32x4 &w, const f32x4 &x, f32x4 acc)
{
    acc.x = __builtin_fmaf(w.x, x.x, acc.x);
    acc.y = __builtin_fmaf(w.y, x.y, acc.y);
    acc.z = __builtin_fmaf(w.z, x.z, acc.z);
    acc.w = __builtin_fmaf(w.w, x.w, acc.w);
    return acc;
}

// Contribution of lane-unit u of R rows to acc[r][b].
//
// Every product is taken with the element's own weight, offset included, so
// that the rounding error of the sums is relative to sum |w x| for any input
// (a row of zero weights gives exactly 0):
//   - the constant code offsets become signed integer bytes before the
//     convert: a b-bit code q with offset 2^(b-1) is XOR-ed with 2^(b-1),
//     which is q - 2^(b-1) in b-bit two's complement, and shifted to the top
//     of its byte, so the sign-extending byte convert gives 2^(8-b) (q - off)
//     exactly (Q4_0 16 (q - 8), Q5_0 8 (q - 16), Q6_K 4 (q - 32)); the power
//     of two is folded into the block scale;
//   - Q4_K / Q5_K weights d sc q - dmin m are formed per element with one
//     fused multiply-add (d sc and dmin m are exact products).
template <int T, int B, int R, class XG>
__device__ __forceinline__ void unit_dot(const URaw<T> (&raw)[R], int u, const XG &xg, float (&acc)[R][B])
{
    typedef typename AccOf<B>::type AccT;
    if constexpr (T == T_Q8_0) {
        AccT s[R][B];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) s[r][b] = zero_acc<AccT>();
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            f32x4 xv[B];
#pragma unroll
            for (int b = 0; b < B; ++b) xv[b] = xg(j, b);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int b = 0; b < B; ++b) s[r][b] = dot4_s(raw[r].c[j], xv[b], s[r][b]);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float d = h2f(raw[r].d);
#pragma unroll
            for (int b = 0; b < B; ++b) acc[r][b] = __builtin_fmaf(d, fin(s[r][b]), acc[r][b]);
        }
    } else if constexpr (T == T_Q4_0 || T == T_Q5_0) {
        // Q4_0: bytes 16 (q - 8); Q5_0: bytes 8 (q - 16)
        AccT slo[R][B], shi[R][B];
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int r = 0; r < R; ++r) slo[r][b] = shi[r][b] = zero_acc<AccT>();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 xl[B], xh[B];
#pragma unroll
            for (int b = 0; b < B; ++b) {
                xl[b] = xg(i, b);
                xh[b] = xg(4 + i, b);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                uint32_t lo, hi;
                if constexpr (T == T_Q4_0) {
                    // 16 q with bit 7 flipped: 16 (q - 8) as int8
                    lo = opaque(((raw[r].c[i] << 4) & 0xf0f0f0f0u) ^ 0x80808080u);
                    hi = opaque((raw[r].c[i] & 0xf0f0f0f0u) ^ 0x80808080u);
                } else {
                    // 5-bit q = nibble | bit 4 from the block's word; flipping
                    // the word's bits gives q - 16 (5-bit), moved up by 3
                    const uint32_t c = raw[r].c[i], hn = ~raw[r].qh;
                    lo = opaque(((c & 0x0f0f0f0fu) | bits_to_byte_bit4(hn >> (4 * i))) << 3);
                    hi = opaque((((c >> 4) & 0x0f0f0f0fu) | bits_to_byte_bit4(hn >> (16 + 4 * i))) << 3);
                }
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    slo[r][b] = dot4_s(lo, xl[b], slo[r][b]);
                    shi[r][b] = dot4_s(hi, xh[b], shi[r][b]);
                }
            }
        }
        constexpr float INV = T == T_Q4_0 ? 0.0625f : 0.125f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float d = h2f(raw[r].d) * INV;
#pragma unroll
            for (int b = 0; b < B; ++b) acc[r][b] = __builtin_fmaf(d, fin(slo[r][b]) + fin(shi[r][b]), acc[r][b]);
        }
    } else if constexpr (T == T_Q4_K) {
        // unit = (super-block, code group p = u % 4): sub-block 2p in the low
        // nibbles, 2p+1 in the high nibbles.  A nibble q alone in bits 0..3
        // (or 4..7) of a 16-bit half is the fp16 subnormal q 2^-24 (q 2^-20),
        // exactly; the fma that forms the weight takes the half as it is
        // (v_fma_mix_f32) with the scale times 2^24 (2^20): one masking per
        // two weights and no separate convert.
        const int p = u & 3;
        float dsc0[R], dsc1[R], ndm0[R], ndm1[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            // bytes 2 (p % 2) and 2 (p % 2) + 1 of the three scale dwords
            const uint32_t sh = 16u * (uint32_t)(p & 1);
            const uint32_t a = raw[r].hd.y >> sh, b = raw[r].hd.z >> sh, c = raw[r].hd.w >> sh;
            // (sc_2p, sc_2p+1) and (m_2p, m_2p+1) in bytes 0 and 1: sub-blocks
            // 0..3 are the low 6 bits of bytes j and j + 4; 4..7 the nibbles of
            // byte j + 4 with the top 2 bits of bytes j - 4 and j
            const uint32_t scp = p < 2 ? (a & 0x3f3fu) : ((c & 0x0f0fu) | ((a >> 2) & 0x3030u));
            const uint32_t mp = p < 2 ? (b & 0x3f3fu) : (((c >> 4) & 0x0f0fu) | ((b >> 2) & 0x3030u));
            const float d = h2f(raw[r].hd.x & 0xffffu) * 16777216.f, dmin = h2f(raw[r].hd.x >> 16);
            dsc0[r] = d * ub0(scp);
            dsc1[r] = d * 0.0625f * ub1(scp);
            ndm0[r] = -(dmin * ub0(mp));
            ndm1[r] = -(dmin * ub1(mp));
        }
        // one chain per sub-block: the fma latency is covered by the other
        // chain and the weight forming between them
        float s0[R][B], s1[R][B];
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int r = 0; r < R; ++r) s0[r][b] = s1[r][b] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            f32x4 xl[B], xh[B];
#pragma unroll
            for (int b = 0; b < B; ++b) {
                xl[b] = xg(i, b);
                xh[b] = xg(8 + i, b);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                // bytes 0..3 of the code dword are elements 4i..4i+3 (low
                // nibbles) and 32+4i..32+4i+3 (high nibbles): halves of
                // (c & 0x000f000f) are elements 0 and 2, of (c & 0x00f000f0)
                // 32 and 34, and the same of c >> 8 elements 1, 3, 33, 35
                const uint32_t c = raw[r].c[i], c8 = c >> 8;
                const h16x2 e02 = __builtin_bit_cast(h16x2, opaque(c & 0x000f000fu));
                const h16x2 e13 = __builtin_bit_cast(h16x2, opaque(c8 & 0x000f000fu));
                const h16x2 f02 = __builtin_bit_cast(h16x2, opaque(c & 0x00f000f0u));
                const h16x2 f13 = __builtin_bit_cast(h16x2, opaque(c8 & 0x00f000f0u));
                const f32x4 wl{__builtin_fmaf((float)e02.x, dsc0[r], ndm0[r]), __builtin_fmaf((float)e13.x, dsc0[r], ndm0[r]),
                               __builtin_fmaf((float)e02.y, dsc0[r], ndm0[r]), __builtin_fmaf((float)e13.y, dsc0[r], ndm0[r])};
                const f32x4 wh{__builtin_fmaf((float)f02.x, dsc1[r], ndm1[r]), __builtin_fmaf((float)f13.x, dsc1[r], ndm1[r]),
                               __builtin_fmaf((float)f02.y, dsc1[r], ndm1[r]), __builtin_fmaf((float)f13.y, dsc1[r], ndm1[r])};
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    s0[r][b] = dot4_f(wl, xl[b], s0[r][b]);
                    s1[r][b] = dot4_f(wh, xh[b], s1[r][b]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[r][b] += s0[r][b] + s1[r][b];
    } else if constexpr (T == T_Q5_K) {
        // unit = (super-block, code group p = u % 4): sub-block 2p in the low
        // nibbles, 2p+1 in the high nibbles; bit 4 at bit 2p / 2p+1 of the
        // qh byte of its element
        const int p = u & 3;
        float dsc0[R], dsc1[R], ndm0[R], ndm1[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            uint32_t sc0, m0, sc1, m1;
            q4k_scale_min(raw[r].hd.y, raw[r].hd.z, raw[r].hd.w, 2 * p, sc0, m0);
            q4k_scale_min(raw[r].hd.y, raw[r].hd.z, raw[r].hd.w, 2 * p + 1, sc1, m1);
            const float d = h2f(raw[r].hd.x & 0xffffu), dmin = h2f(raw[r].hd.x >> 16);
            dsc0[r] = d * (float)sc0;
            dsc1[r] = d * (float)sc1;
            ndm0[r] = -(dmin * (float)m0);
            ndm1[r] = -(dmin * (float)m1);
        }
        AccT s0[R][B], s1[R][B];
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int r = 0; r < R; ++r) s0[r][b] = s1[r][b] = zero_acc<AccT>();
        const uint32_t sh0 = 2u * (uint32_t)p;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            f32x4 xl[B], xh[B];
#pragma unroll
            for (int b = 0; b < B; ++b) {
                xl[b] = xg(i, b);
                xh[b] = xg(8 + i, b);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t c = raw[r].c[i], hb = raw[r].h[i];
                const uint32_t lo = opaque((c & 0x0f0f0f0fu) | (((hb >> sh0) & 0x01010101u) << 4));
                const uint32_t hi = opaque(((c >> 4) & 0x0f0f0f0fu) | (((hb >> (sh0 + 1u)) & 0x01010101u) << 4));
                const f32x4 wl = wts4(lo, dsc0[r], ndm0[r]), wh = wts4(hi, dsc1[r], ndm1[r]);
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    s0[r][b] = dot4_f(wl, xl[b], s0[r][b]);
                    s1[r][b] = dot4_f(wh, xh[b], s1[r][b]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b) acc[r][b] += fin(s0[r][b]) + fin(s1[r][b]);
    } else {  // Q6_K
        // unit = (super-block, half h, l-range 16 hf .. 16 hf + 15): for each
        // g the 16 elements 128h + 32g + 16hf + i belong to sub-block
        // 8h + 2g + hf; low nibble in ql (g = 0/2 in qa, 1/3 in qb), high bits
        // at bit 2g of qh.  Bytes 4 (q - 32): the low 4 bits of q at bits 2..5,
        // the high 2 bits at 6..7 with bit 5 of q flipped (qh XOR 0b10 per
        // 2-bit field)
        const int hf = u & 1;
        float dsc[R][4];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float d = h2f(raw[r].d) * 0.25f;
            const uint32_t sh = 8u * hf;
            dsc[r][0] = d * (float)(int8_t)(raw[r].sc[0] >> sh);          // scale 8h + hf
            dsc[r][1] = d * (float)(int8_t)(raw[r].sc[0] >> (16 + sh));   // scale 8h + 2 + hf
            dsc[r][2] = d * (float)(int8_t)(raw[r].sc[1] >> sh);          // scale 8h + 4 + hf
            dsc[r][3] = d * (float)(int8_t)(raw[r].sc[1] >> (16 + sh));   // scale 8h + 6 + hf
        }
        // one scalar chain per (row, batch, group): the four groups already
        // give four independent chains of 16 fmas per unit
        float s[R][B][4];
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int r = 0; r < R; ++r) s[r][b][g] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 xv[B];
#pragma unroll
                for (int b = 0; b < B; ++b) xv[b] = xg(4 * g + i, b);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint32_t a = raw[r].qa[i], bq = raw[r].qb[i], hx = raw[r].qh[i] ^ 0xaaaaaaaau;
                    // high bits at 6..7 alone (zeros elsewhere), then one
                    // v_and_or_b32 with the shifted nibbles
                    const uint32_t hb = opaque((hx << (6 - 2 * g)) & 0xc0c0c0c0u);
                    const uint32_t lo = g == 0 ? a << 2 : g == 1 ? bq << 2 : g == 2 ? a >> 2 : bq >> 2;
                    const uint32_t q = opaque((lo & 0x3c3c3c3cu) | hb);
#pragma unroll
                    for (int b = 0; b < B; ++b) s[r][b][g] = dot4_s(q, xv[b], s[r][b][g]);
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
                    t = __builtin_fmaf(dsc[r][g], fin(s[r][b][g]), t);
                acc[r][b] += t;
            }
    }
}

// ------------------------------------------------- row-segment staging --

// Prefetch of R row segments into registers (16-byte chunks, unconditional:
// chunks past the data read offset 0 of w instead) and their store to LDS.
// NT: non-temporal loads.  Each weight byte is read once, and in the decode
// passes streaming past the caches is faster (Q4_K_M-style mix at batch 1:
// 1.50 -> 1.46 ms; Llama-3-8B Q4_K: 1.32 -> 1.27 ms; TinyLlama Q4_0: 0.46
// -> 0.42 ms); single small launches at batch 2 are 2-12% slower with them.
template <int T, int R, bool NT = true>
struct SegStage {
    static constexpr int UE = GemvUnit<T>::UE;
    static constexpr int SEGE = 64 * UE;
    static constexpr int SEGB = SEGE / Fmt<T>::BE * Fmt<T>::BB;
    static constexpr int CPR = SEGB / 16;                  // chunks per full row segment
    static constexpr int RS = SEGB / 4 + 4;                // LDS row stride (dwords)
    static constexpr int NCH = (R * CPR + 63) / 64;        // chunks per lane
    static constexpr int LDS_DW = R * RS + 256;            // + 64 dummy 16-byte slots
    u32x4 pf[NCH];

    __device__ __forceinline__ void load(const uint8_t *w, int64_t rb, int n, int row0, int seg, int cpr, int lane)
    {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = lane + 64 * i;
            const int jr = c / CPR, off = c - jr * CPR;
            const int row = row0 + jr;
            const bool ok = jr < R && off < cpr && row < n;
            const int64_t o = ok ? (int64_t)row * rb + (int64_t)seg * SEGB + 16 * off : 0;
            pf[i] = NT ? __builtin_nontemporal_load((const u32x4 *)(w + o)) : *(const u32x4 *)(w + o);
        }
    }
    // One row (R = 1) through a buffer resource: the segment is the first
    // nbytes bytes at base (a wave-uniform address; nbytes 0 for an item
    // past the wave's last).  Loads past nbytes return zero without a memory
    // access, and each lane's offsets are constants: no per-lane address
    // arithmetic per item (Q4_K loop 234 -> 215 VALU instructions per item,
    // Q4_0 115 -> 97).  Used with the non-temporal loads of the large
    // matrices: single launches on small ones were slower with it (Q8_0
    // 2048 x 2048 2.89 -> 3.37 us).
    __device__ __forceinline__ void load_row(const uint8_t *base, uint32_t nbytes, int lane)
    {
        static_assert(R == 1, "one row per item");
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)nbytes, 0x00020000);
#pragma unroll
        for (int i = 0; i < NCH; ++i)
            pf[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * (lane + 64 * i), 0,
                                                                                    NT ? 2 : 0));
    }
    __device__ __forceinline__ void store(uint32_t *ws, int lane) const
    {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = lane + 64 * i;
            const int jr = c / CPR, off = c - jr * CPR;
            const int idx = jr < R ? jr * RS + 4 * off : R * RS + 4 * lane;
            *(u32x4 *)(ws + idx) = pf[i];
        }
    }
};

template <int R>
__device__ __forceinline__ void reduce_store(float (&acc)[R][1], int row0, int n, int lane, float *y)
{
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float v = wave_sum(acc[r][0]);
        const int row = row0 + r;
        if (lane == 0 && row < n)
            y[row] = v;
        acc[r][0] = 0.f;
    }
}

}  // namespace qmm
