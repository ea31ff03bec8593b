// qmm_gemv.hip -- decode GEMV y[b] = W x[b] straight from quantized blocks.
//
// dotLLM "GPU Inference", cuBLAS GEMM/GEMV and Custom Kernels table: at
// seqLen = 1 every projection is a quantized GEMV that operates directly on
// the quantized weights and is memory-bandwidth bound; shimmy "Airframe GPU
// pipeline" (decode) says the same: reading the weight tensors dominates.
//
// gfx950 design
//   - Work is split into lane-units: one Q8_0 / Q4_0 block (32 elements) or a
//     64-element quarter of a Q4_K / Q6_K super-block.  A segment is 64
//     consecutive units of a row, i.e. one unit per lane of a wavefront.
//   - Weights are read with 16-byte loads.  Q4_K blocks (144 B) keep 16-byte
//     alignment, so each lane loads its unit straight into registers.  Blocks
//     of 34, 18, 22 and 210 bytes are only 2-byte aligned (and the 176-byte
//     Q5_K blocks take the same path): the wavefront copies the
//     row segment into LDS with fully coalesced loads (64 lanes x 16 B
//     contiguous) and each lane reads its unit back with aligned dword reads,
//     realigned in registers with v_alignbyte_b32.
//   - Codes are converted with a few bit operations per dword plus the byte
//     converts (v_cvt_f32_ubyteN, or the sign-extending SDWA convert), and
//     every product uses the element's own weight: integer code offsets
//     (-8, -16, -32) become signed bytes before the convert, the K-quant
//     weights d sc q - dmin m are formed per element with one fma.  Sums are
//     fp32 per block or sub-block; integer-code scales are applied once per
//     (sub-)block.
//   - Per-lane partial sums are reduced across the wavefront with cross-lane
//     shuffles; lane 0 writes y.
//   - Loads are issued without branches (out-of-range lanes read a valid
//     address and discard it): the compiler otherwise sinks a predicated load
//     into its branch and waits for it at once, serializing the memory
//     round trips.
//
// Kernels
//   gemv3_kernel  batch 1, k <= one segment (every projection except the
//                 wide-k down ones): x staged once per workgroup in LDS
//                 (padded against bank conflicts) while the first weight
//                 loads are in flight, each lane then holds its slice of x in
//                 registers; waves are independent and persistent, one row
//                 per item, and the weight bytes of the next items are in
//                 flight while the current one is decoded; 8 or 16 waves
//                 per compute unit.
//   gemv2m_kernel the same loop (gemv2_body) over a table of up to 8
//                 problems sharing k (the grouped entry point), x read by
//                 each wave from L2: one launch instead of one per matrix.
//   gemv3m_kernel the table with one x shared by every problem (q / k / v,
//                 gate / up): x staged in LDS as in gemv3.
//   gemv1_kernel  batch 1, k spanning several segments: x is staged in LDS
//                 once per workgroup; otherwise as gemv3 (two rows per item,
//                 one when there are too few rows to give every CU a
//                 workgroup).
//   gemv_kernel   batch 2..8 of Q8_0 / Q4_0 / Q5_0 / Q5_K (and unaligned
//                 batch-1 rows): x
//                 segment and weight segments staged in LDS per workgroup.
//   Batch 2..8 of Q4_K / Q6_K runs on the matrix cores (qmm_gemv_mfma.hip).
#include "qmm_device.h"
#include "qmm_launch.h"

#include <type_traits>

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

// Q4_K unit u straight from global memory (super-blocks are 16-byte aligned).
__device__ __forceinline__ void raw_from_global_q4k(const uint8_t *seg, int u, URaw<T_Q4_K> &r)
{
    const uint8_t *blk = seg + 144 * (u >> 2);
    const int p = u & 3;
    r.hd = *(const u32x4 *)blk;
    const u32x4 c0 = *(const u32x4 *)(blk + 16 + 32 * p);
    const u32x4 c1 = *(const u32x4 *)(blk + 32 + 32 * p);
    r.c[0] = c0.x; r.c[1] = c0.y; r.c[2] = c0.z; r.c[3] = c0.w;
    r.c[4] = c1.x; r.c[5] = c1.y; r.c[6] = c1.z; r.c[7] = c1.w;
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
    } else if constexpr (T == T_Q4_K || T == T_Q5_K) {
        // unit = (super-block, code group p = u % 4): sub-block 2p in the low
        // nibbles, 2p+1 in the high nibbles (Q5_K: bit 4 at bit 2p / 2p+1 of
        // the qh byte of its element)
        const int p = u & 3;
        float dsc0[R], dsc1[R], ndm0[R], ndm1[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            uint32_t sc0, m0, sc1, m1;
            q4k_scale_min(raw[r].hd.y, raw[r].hd.z, raw[r].hd.w, 2 * p, sc0, m0);
            q4k_scale_min(raw[r].hd.y, raw[r].hd.z, raw[r].hd.w, 2 * p + 1, sc1, m1);
            const float d = h2f(raw[r].hd.x & 0xffffu), dmin = h2f(raw[r].hd.x >> 16);
            dsc0[r] = d * (float)sc0;
            // Q4_K high nibbles convert as 16 q
            dsc1[r] = T == T_Q4_K ? d * (float)sc1 * 0.0625f : d * (float)sc1;
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
                uint32_t lo, hi;
                if constexpr (T == T_Q4_K) {
                    lo = opaque(raw[r].c[i] & 0x0f0f0f0fu);
                    hi = opaque(raw[r].c[i] & 0xf0f0f0f0u);
                } else {
                    const uint32_t c = raw[r].c[i], hb = raw[r].h[i];
                    lo = opaque((c & 0x0f0f0f0fu) | (((hb >> sh0) & 0x01010101u) << 4));
                    hi = opaque(((c >> 4) & 0x0f0f0f0fu) | (((hb >> (sh0 + 1u)) & 0x01010101u) << 4));
                }
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
        AccT s[R][B][4];
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int r = 0; r < R; ++r) s[r][b][g] = zero_acc<AccT>();
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
                    uint32_t q;
                    if (g == 0) q = ((a << 2) & 0x3c3c3c3cu) | ((hx << 6) & 0xc0c0c0c0u);
                    else if (g == 1) q = ((bq << 2) & 0x3c3c3c3cu) | ((hx << 4) & 0xc0c0c0c0u);
                    else if (g == 2) q = ((a >> 2) & 0x3c3c3c3cu) | ((hx << 2) & 0xc0c0c0c0u);
                    else q = ((bq >> 2) & 0x3c3c3c3cu) | (hx & 0xc0c0c0c0u);
                    q = opaque(q);
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
template <int T, int R>
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
            pf[i] = *(const u32x4 *)(w + o);
        }
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

// --------------------------------------------------------------- gemv2 --
// Batch 1, k <= one segment, x in registers, independent persistent waves.
// One launch serves up to MAXP problems with the same type and k (e.g. the
// q / k / v or gate / up projections of a layer): row groups are numbered
// across the problems and each wave walks them with a stride.
constexpr int GEMV_MAXP = 8;
struct GemvProbs {
    const uint8_t *w[GEMV_MAXP];
    const float *x[GEMV_MAXP];
    float *y[GEMV_MAXP];
    int n[GEMV_MAXP];
    int rg0[GEMV_MAXP + 1];   // first row group of each problem; rg0[np] = total
    int np;
};

// Problem sources: one problem passed as plain kernel arguments (held in
// SGPRs from the start), or a table of problems (its entries are scalar loads
// whose latency shows in small launches, so single problems avoid it).
struct OneProb {
    const uint8_t *w;
    const float *x;
    float *y;
    int n;
    __device__ __forceinline__ int total_rg(int R) const { return (n + R - 1) / R; }
    __device__ __forceinline__ int find(int) const { return 0; }
    __device__ __forceinline__ int rg_begin(int) const { return 0; }
    __device__ __forceinline__ const uint8_t *W(int) const { return w; }
    __device__ __forceinline__ const float *X(int) const { return x; }
    __device__ __forceinline__ float *Y(int) const { return y; }
    __device__ __forceinline__ int N(int) const { return n; }
};
struct TableProbs {
    const GemvProbs &P;
    __device__ __forceinline__ int total_rg(int) const { return P.rg0[P.np]; }
    __device__ __forceinline__ int find(int rg) const
    {
        int pp = 0;
        for (int q = 1; q < P.np; ++q)
            if (rg >= P.rg0[q]) pp = q;
        return pp;
    }
    __device__ __forceinline__ int rg_begin(int pp) const { return P.rg0[pp]; }
    __device__ __forceinline__ const uint8_t *W(int pp) const { return P.w[pp]; }
    __device__ __forceinline__ const float *X(int pp) const { return P.x[pp]; }
    __device__ __forceinline__ float *Y(int pp) const { return P.y[pp]; }
    __device__ __forceinline__ int N(int pp) const { return P.n[pp]; }
};

// NW wavefronts per workgroup.  xl (X_LDS): the workgroup first copies the
// single problem's x into LDS, and each wave takes its lane slice from there
// (instead of every wave reading all of x from L2, which with many waves
// costs more L2 traffic than the weights).
template <int T, int R, class PS, int NW = 4, bool X_LDS = false>
__device__ __forceinline__ void gemv2_body(const PS &P, int k, int64_t rb, uint32_t *ws, float *xl = nullptr)
{
    constexpr int UE = GemvUnit<T>::UE, NRUN = GemvUnit<T>::NRUN;
    using S = SegStage<T, R>;
    constexpr bool DIRECT = (T == T_Q4_K);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int gw = blockIdx.x * NW + wave, tw = gridDim.x * NW;
    // X_LDS: this thread's share of x is loaded into registers first, so
    // that it is in flight together with the first weight loads (issued
    // next), and written to LDS after them (stage_x).  Positions past k
    // read x[0..3] and are not stored.
    constexpr int XV = X_LDS ? (64 * UE + 4 * 64 * NW - 1) / (4 * 64 * NW) : 1;
    f32x4 xst[XV];
    if constexpr (X_LDS) {
        const float *x = P.X(0);
#pragma unroll
        for (int j = 0; j < XV; ++j) {
            const int e = 4 * ((int)threadIdx.x + 64 * NW * j);
            xst[j] = *(const f32x4 *)(x + (e < k ? e : 0));
        }
        // keep these loads ahead of the weight loads: the wait for them
        // before the LDS writes then leaves the weight loads in flight
        __builtin_amdgcn_sched_barrier(0);
    }
    // padded layout (4 floats per unit): lanes read their unit slices at a
    // stride of UE + 4 floats, which keeps the 128-bit reads off a single
    // bank group.  The barrier is a raw one after this wave's LDS writes
    // complete: a full __syncthreads() would also wait for the weight loads.
    auto stage_x = [&]() __attribute__((always_inline)) {
        if constexpr (X_LDS) {
#pragma unroll
            for (int j = 0; j < XV; ++j) {
                const int e = 4 * ((int)threadIdx.x + 64 * NW * j);
                if (e < k)
                    *(f32x4 *)(xl + xpad<UE>(e)) = xst[j];
            }
            lds_barrier();
        }
    };
    // each wave takes a contiguous run of row groups (run lengths differ by
    // at most one, so every wave has work when there are enough), so that
    // its results form contiguous runs of y (stored 64 at a time, below)
    const int nrg = P.total_rg(R);
    const int q = nrg / tw, rem = nrg - q * tw;    // one 32-bit division
    const int rgs = gw * q + min(gw, rem);
    const int nit = q + (gw < rem ? 1 : 0);
    const bool active = lane < k / UE;
    const int cpr = k / Fmt<T>::BE * Fmt<T>::BB / 16;

    // problem and first row of item it (past the end: the last item)
    auto locate = [&](int it, int &pp, int &row0) __attribute__((always_inline)) {
        it = min(it, max(nit - 1, 0));
        const int rg = min(rgs + it, nrg - 1);   // a wave with no item: the last row group
        pp = P.find(rg);
        row0 = (rg - P.rg_begin(pp)) * R;
    };

    // this lane's slice of x for the current problem
    f32x4 xr[NRUN];
    auto load_x = [&](int pp) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NRUN; ++j) {
            const int e = active ? run_elem<T>(lane, j) : 0;
            xr[j] = X_LDS ? *(const f32x4 *)(xl + xpad<UE>(e)) : *(const f32x4 *)(P.X(pp) + e);
        }
    };
    const XFromRegs<T> xg{xr};

    float acc[R][1];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r][0] = 0.f;

    int p0, r0;
    locate(0, p0, r0);
    int xp = p0;
    if constexpr (!X_LDS)
        load_x(xp);

    // Two items of weight bytes in flight while an item computes: three
    // prefetch register sets, the loop unrolled by three so that each has a
    // fixed place.  An item computes in place and its set is reloaded (for
    // item it + 3) only after its last use, with a scheduling barrier in
    // between: a reload scheduled above the use would need other registers
    // and a copy back at the loop edge, which waits for the load.  Prefetches
    // past the wave's last item read offset 0 in every lane (one cache line,
    // no branch: a load under a branch is waited for at once).  Lanes past k
    // compute on offset-0 bytes and contribute 0 (select, not branch).
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    // Row results collect in lane (row - blk_row) of res and leave as one
    // coalesced store per 64 rows (or at a problem change / the end); a
    // one-lane store per row costs a divergent branch and a store each.
    float res = 0.f;
    int blk_row = 0, blk_cnt = 0, blk_pp = 0;
    auto flush = [&]() __attribute__((always_inline)) {
        if (blk_cnt > 0) {
            const int row = blk_row + lane;
            if (lane < blk_cnt && row < P.N(blk_pp))
                P.Y(blk_pp)[row] = res;
        }
        blk_cnt = 0;
    };
    auto finish = [&](int pp, int row0) __attribute__((always_inline)) {
        if (blk_cnt + R > 64 || (blk_cnt > 0 && pp != blk_pp))
            flush();
        if (blk_cnt == 0) {
            blk_row = row0;
            blk_pp = pp;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float v = wave_sum_hi(active ? acc[r][0] : 0.f);
            const float tot = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
            res = lane == blk_cnt + r ? tot : res;
            acc[r][0] = 0.f;
        }
        blk_cnt += R;
    };
    if constexpr (DIRECT) {
        URaw<T> pr[3][R];
        auto load = [&](int it, URaw<T> (&dst)[R]) __attribute__((always_inline)) {
            int pp, row0;
            locate(it, pp, row0);
            const uint8_t *w = P.W(pp);
            const int n = P.N(pp);
            const bool live = it < nit;   // past the wave's last item: a dummy load of offset 0
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const bool ok = live && active && row0 + r < n;
                raw_from_global_q4k(w + (ok ? (int64_t)(row0 + r) * rb : 0), ok ? lane : 0, dst[r]);
            }
        };
        load(0, pr[0]);
        load(1, pr[1]);
        load(2, pr[2]);
        if constexpr (X_LDS) {
            stage_x();
            load_x(xp);
        }
        auto step = [&](auto bc, int it) __attribute__((always_inline)) {
            constexpr int B = decltype(bc)::value;
            int pp, row0;
            locate(it, pp, row0);
            if (pp != xp) {   // wave-uniform: the next problem's x
                xp = pp;
                load_x(xp);
            }
            unit_dot<T, 1, R>(pr[B], lane, xg, acc);
            __builtin_amdgcn_sched_barrier(0);
            load(it + 3, pr[B]);
            finish(pp, row0);
        };
        int it = 0;
        for (; it + 2 < nit; it += 3) {
            step(I0{}, it);
            step(I1{}, it + 1);
            step(I2{}, it + 2);
        }
        if (it < nit)
            step(I0{}, it);
        if (it + 1 < nit)
            step(I1{}, it + 1);
        flush();
    } else {
        // LDS-staged rows: one prefetch register set suffices, since it is
        // emptied into LDS before being refilled (no copy of an in-flight
        // load); measured faster than three sets for these types
        uint32_t *mw = ws + wave * S::LDS_DW;
        S st;
        auto load = [&](int it) __attribute__((always_inline)) {
            int pp, row0;
            locate(it, pp, row0);
            // past the wave's last item: no row is in range, every chunk reads offset 0
            st.load(P.W(pp), rb, it < nit ? P.N(pp) : 0, row0, 0, cpr, lane);
        };
        load(0);
        if constexpr (X_LDS) {
            stage_x();
            load_x(xp);
        }
        for (int it = 0; it < nit; ++it) {
            int pp, row0;
            locate(it, pp, row0);
            if (pp != xp) {
                xp = pp;
                load_x(xp);
            }
            st.store(mw, lane);
            wave_lds_sync();
            load(it + 1);
            URaw<T> cur[R];
#pragma unroll
            for (int r = 0; r < R; ++r) raw_from_lds<T>(mw + r * S::RS, lane, cur[r]);
            unit_dot<T, 1, R>(cur, lane, xg, acc);
            finish(pp, row0);
            wave_lds_sync();
        }
        flush();
    }
}

// Batch 1, one problem, x staged in LDS, NW wavefronts per workgroup (one
// workgroup per CU: 16 waves, 4 per SIMD, hide the weight latency).
template <int T, int R, int NW>
__global__ void __launch_bounds__(64 * NW)
gemv3_kernel(const uint8_t *__restrict__ w, int n, int k, int64_t rb, const float *__restrict__ x,
             float *__restrict__ y)
{
    __shared__ __attribute__((aligned(16))) float xl[64 * (GemvUnit<T>::UE + 4)];
    __shared__ __attribute__((aligned(16))) uint32_t ws[T == T_Q4_K ? 4 : NW * SegStage<T, R>::LDS_DW];
    const OneProb P{w, x, y, n};
    gemv2_body<T, R, OneProb, NW, true>(P, k, rb, ws, xl);
}

template <int T, int R>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 4)))
gemv2m_kernel(const GemvProbs Pt, int k, int64_t rb)
{
    __shared__ __attribute__((aligned(16))) uint32_t ws[T == T_Q4_K ? 4 : 4 * SegStage<T, R>::LDS_DW];
    const TableProbs P{Pt};
    gemv2_body<T, R>(P, k, rb, ws);
}

// The table of problems with one x shared by all of them (the q / k / v or
// gate / up projections of a layer read the same activation): x staged in
// LDS as in gemv3, one row per item.
template <int T, int R, int NW>
__global__ void __launch_bounds__(64 * NW)
gemv3m_kernel(const GemvProbs Pt, int k, int64_t rb)
{
    __shared__ __attribute__((aligned(16))) float xl[64 * (GemvUnit<T>::UE + 4)];
    __shared__ __attribute__((aligned(16))) uint32_t ws[T == T_Q4_K ? 4 : NW * SegStage<T, R>::LDS_DW];
    const TableProbs P{Pt};
    gemv2_body<T, R, TableProbs, NW, true>(P, k, rb, ws, xl);
}

// --------------------------------------------------------------- gemv1 --
// Batch 1, k spanning several segments: x staged in LDS once per workgroup;
// each wave walks items (R rows x one segment) with the weight bytes of the
// next D items in flight (a ring of D register stages, so a row's segments
// are fetched together rather than one round trip after another).
template <int T, int R, int NW, int XK, int D>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 4)))
gemv1_kernel(const uint8_t *__restrict__ w, int n, int k, int64_t rb, const float *__restrict__ x,
             float *__restrict__ y)
{
    using F = Fmt<T>;
    constexpr int UE = GemvUnit<T>::UE;
    using S = SegStage<T, R>;
    constexpr int SEGE = S::SEGE;
    constexpr int XS = XK + (XK / UE) * 4;
    constexpr int XV = XK / (4 * 64 * NW);          // 4-float vectors per thread for x
    __shared__ __attribute__((aligned(16))) float xs[XS];
    __shared__ __attribute__((aligned(16))) uint32_t ws[NW * S::LDS_DW];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gw = blockIdx.x * NW + wave, tw = gridDim.x * NW;
    const int nrg = (n + R - 1) / R;
    const int nseg = (k + SEGE - 1) / SEGE;
    const int my_rg = gw < nrg ? (nrg - gw + tw - 1) / tw : 0;
    const int nitems = my_rg * nseg;
    uint32_t *mw = ws + wave * S::LDS_DW;

    S st[D];
    auto load = [&](S &dst, int it) __attribute__((always_inline)) {
        it = min(it, max(nitems - 1, 0));   // past the end: reload the last item
        const int rg = gw + tw * (it / nseg), seg = it % nseg;
        const int segE = min(SEGE, k - seg * SEGE);
        dst.load(w, rb, n, rg * R, seg, segE / F::BE * F::BB / 16, lane);
    };

#pragma unroll
    for (int i = 0; i < D; ++i)
        load(st[i], i);
    {   // stage x; positions >= k hold copies of x[0..3], which no active lane reads
        f32x4 xv[XV];
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            const int e = 4 * (threadIdx.x + 64 * NW * i);
            xv[i] = *(const f32x4 *)(x + (e < k ? e : 0));
        }
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            const int e = 4 * (threadIdx.x + 64 * NW * i);
            *(f32x4 *)(xs + xpad<UE>(e)) = xv[i];
        }
    }
    __syncthreads();

    float acc[R][1];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r][0] = 0.f;
    for (int it0 = 0; it0 < nitems; it0 += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            const int it = it0 + i;
            st[i].store(mw, lane);
            wave_lds_sync();
            // no refill past the wave's last item (wave-uniform): a wave does
            // not end before its loads land, and the refill's data is unused
            // (2048 x 5632 Q4_0: 5.55 -> 5.42 us)
            if (it + D < nitems)
                load(st[i], it + D);
            if (it < nitems) {     // the ring runs in whole rounds; the surplus items are reloads
                const int rg = gw + tw * (it / nseg), seg = it % nseg;
                const int segE = min(SEGE, k - seg * SEGE);
                if (lane < segE / UE) {
                    URaw<T> cur[R];
#pragma unroll
                    for (int r = 0; r < R; ++r) raw_from_lds<T>(mw + r * S::RS, lane, cur[r]);
                    const XFromLds<T, XS> xg{xs + xpad<UE>(seg * SEGE), lane};
                    unit_dot<T, 1, R>(cur, lane, xg, acc);
                }
                if (seg == nseg - 1)
                    reduce_store<R>(acc, rg * R, n, lane, y);
            }
            wave_lds_sync();
        }
    }
}

// ---------------------------------------------------------------- gemv --
// Batch 1..8, any row alignment: per segment, the workgroup stages x (all
// batches) and each wave its R row segments in LDS.
template <int T, int B, int R, bool A16>
__global__ void __launch_bounds__(256)
gemv_kernel(const uint8_t *__restrict__ w, int n, int k, int64_t rb, const float *__restrict__ x,
            float *__restrict__ y)
{
    using F = Fmt<T>;
    constexpr int UE = GemvUnit<T>::UE;
    using S = SegStage<T, R>;
    constexpr int SEGE = S::SEGE, SEGB = S::SEGB;
    constexpr int XS = SEGE + (SEGE / UE) * 4;    // padded floats per batch
    __shared__ __attribute__((aligned(16))) float xs[B * XS];
    __shared__ __attribute__((aligned(16))) uint32_t ws[4 * S::LDS_DW];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row0 = (blockIdx.x * 4 + wave) * R;
    uint32_t *mw = ws + wave * S::LDS_DW;
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
        S st;
        if constexpr (A16)
            st.load(w, rb, n, row0, seg, segBytes >> 4, lane);
        // stage x[b][e0 .. e0+segE): XB vectors per thread per batch of loads
        {
            constexpr int XB = 8;
            const int nx4 = B * (segE >> 2);
            for (int base = 0; base < nx4; base += 256 * XB) {
                f32x4 v[XB];
#pragma unroll
                for (int j = 0; j < XB; ++j) {
                    const int i4 = base + threadIdx.x + 256 * j;
                    const int ic = i4 < nx4 ? i4 : 0;
                    const int b = ic / (segE >> 2), e = 4 * (ic - b * (segE >> 2));
                    v[j] = *(const f32x4 *)(x + (int64_t)b * k + e0 + e);
                }
#pragma unroll
                for (int j = 0; j < XB; ++j) {
                    const int i4 = base + threadIdx.x + 256 * j;
                    if (i4 < nx4) {
                        const int b = i4 / (segE >> 2), e = 4 * (i4 - b * (segE >> 2));
                        *(f32x4 *)(xs + b * XS + xpad<UE>(e)) = v[j];
                    }
                }
            }
        }
        if constexpr (A16) {
            st.store(mw, lane);
        } else {
            // rows not 16-byte aligned: 2-byte copies
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int row = row0 + r;
                if (row < n) {
                    const uint8_t *src = w + (int64_t)row * rb + (int64_t)seg * SEGB;
                    uint16_t *dst = (uint16_t *)(mw + r * S::RS);
                    for (int c = lane; c < (segBytes >> 1); c += 64)
                        dst[c] = ((const uint16_t *)src)[c];
                }
            }
        }
        __syncthreads();
        if (lane < segE / UE) {
            URaw<T> cur[R];
#pragma unroll
            for (int r = 0; r < R; ++r) raw_from_lds<T>(mw + r * S::RS, lane, cur[r]);
            const XFromLds<T, XS> xg{xs, lane};
            unit_dot<T, B, R>(cur, lane, xg, acc);
        }
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

// ------------------------------------------------------------- launchers --

// Persistent launches: at most as many workgroups as fit on the device at once.
template <class K>
static int resident_wgs(K kernel, int block)
{
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess || per_cu < 1)
        return 0;
    return per_cu * cus;
}

// at most 2 workgroups (8 waves) per CU: each wave then walks several row
// groups, which amortizes its x slice and keeps a load in flight
template <class K>
static int gemv2_cap(K kernel)
{
    int dev = 0, cus = 0;
    const int res = resident_wgs(kernel, 256);
    if (res == 0 || hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return res < 2 * cus ? res : 2 * cus;
}

// Batch 1 through gemv3 (x staged in LDS, 8 waves per workgroup): at most
// one workgroup per CU, each wave a contiguous run of rows.
template <int T, int R, int NW>
static hipError_t launch_b1_xlds(const uint8_t *w, int64_t n, int64_t k, size_t rb, const float *x, float *y,
                                 hipStream_t s)
{
    const int cus = device_cu_count();
    if (cus == 0)
        return hipErrorInvalidValue;
    const int64_t want = ((n + R - 1) / R + NW - 1) / NW;
    const dim3 grid((unsigned)(want < cus ? want : cus)), block(64 * NW);
    hipLaunchKernelGGL((gemv3_kernel<T, R, NW>), grid, block, 0, s, w, (int)n, (int)k, (int64_t)rb, x, y);
    return hipGetLastError();
}

template <int T, int R>
static hipError_t launch_b1_table(const GemvProbs &P, int64_t k, size_t rb, hipStream_t s)
{
    static std::atomic<int> slot[64];
    const int cap = per_device_cached(slot, [] { return gemv2_cap(gemv2m_kernel<T, R>); });
    if (cap == 0)
        return hipErrorInvalidValue;
    const int64_t want = ((int64_t)P.rg0[P.np] + 3) / 4;
    if (want == 0)
        return hipSuccess;
    const dim3 grid((unsigned)(want < cap ? want : cap)), block(256);
    hipLaunchKernelGGL((gemv2m_kernel<T, R>), grid, block, 0, s, P, (int)k, (int64_t)rb);
    return hipGetLastError();
}

// Shared-x table through gemv3m: at most one workgroup per CU.
template <int T, int NW>
static hipError_t launch_b1_table_xlds(const GemvProbs &P, int64_t k, size_t rb, hipStream_t s)
{
    const int cus = device_cu_count();
    if (cus == 0)
        return hipErrorInvalidValue;
    const int64_t want = ((int64_t)P.rg0[P.np] + NW - 1) / NW;
    if (want == 0)
        return hipSuccess;
    const dim3 grid((unsigned)(want < cus ? want : cus)), block(64 * NW);
    hipLaunchKernelGGL((gemv3m_kernel<T, 1, NW>), grid, block, 0, s, P, (int)k, (int64_t)rb);
    return hipGetLastError();
}

template <int T, int R, int NW, int XK, int D>
static hipError_t launch_b1_lds(const uint8_t *w, int64_t n, int64_t k, size_t rb, const float *x, float *y,
                                hipStream_t s)
{
    static std::atomic<int> slot[64];
    const int cap = per_device_cached(slot, [] { return resident_wgs(gemv1_kernel<T, R, NW, XK, D>, 64 * NW); });
    if (cap == 0)
        return hipErrorInvalidValue;
    const int64_t want = ((n + R - 1) / R + NW - 1) / NW;
    const dim3 grid((unsigned)(want < cap ? want : cap)), block(64 * NW);
    hipLaunchKernelGGL((gemv1_kernel<T, R, NW, XK, D>), grid, block, 0, s, w, (int)n, (int)k, (int64_t)rb, x, y);
    return hipGetLastError();
}

template <int T, int B, int R>
static hipError_t launch_tbr(const uint8_t *w, int64_t n, int64_t k, size_t rb, const float *x, float *y,
                             hipStream_t s)
{
    const dim3 grid((unsigned)((n + 4 * R - 1) / (4 * R))), block(256);
    if (rb % 16 == 0)
        hipLaunchKernelGGL((gemv_kernel<T, B, R, true>), grid, block, 0, s, w, (int)n, (int)k, (int64_t)rb, x, y);
    else
        hipLaunchKernelGGL((gemv_kernel<T, B, R, false>), grid, block, 0, s, w, (int)n, (int)k, (int64_t)rb, x, y);
    return hipGetLastError();
}

template <int T>
static hipError_t launch_t(const uint8_t *w, int64_t n, int64_t k, size_t rb, const float *x, int batch, float *y,
                           hipStream_t s)
{
    if (batch == 1 && rb % 16 == 0) {
        if (k <= 64 * GemvUnit<T>::UE) {
            // x staged once per workgroup in LDS (while the first weight
            // loads are in flight), one row per item: 8 waves per CU, 16 for
            // the 32-element types with at least 4096 rows.  Measured on
            // MI355X against the same loop with x read by every wave from L2:
            // Q4_0 256 / 2048 / 5632 x 2048: 2.64 / 3.48 / 4.46 -> 2.21 /
            // 2.78 / 4.01 us; Q8_0 2048 x 2048 3.57 -> 3.10 us; Q6_K 1024 x
            // 4096 and 128256 x 4096: 3.81 -> 3.67 us and 81.0 -> 78.1 us;
            // Q5_K 1024 / 4096 / 14336 x 4096: 4.44 / 6.69 / 13.5 -> 3.49 /
            // 4.87 / 11.2 us.
            if constexpr (T == T_Q4_0 || T == T_Q8_0 || T == T_Q5_0) {
                if (n >= 4096)
                    return launch_b1_xlds<T, 1, 16>(w, n, k, rb, x, y, s);
                return launch_b1_xlds<T, 1, 8>(w, n, k, rb, x, y, s);
            }
            return launch_b1_xlds<T, 1, 8>(w, n, k, rb, x, y, s);
        }
        if (k <= 16384) {
            // two rows per item, unless that leaves compute units without a
            // workgroup (e.g. 2048 rows: 128 workgroups of 8 waves); then one
            // (measured on MI355X: 2048 x 5632 Q4_0 5.95 -> 5.23 us)
            const int cus = device_cu_count();
            if (cus == 0)
                return hipErrorInvalidValue;
            if (((n + 1) / 2 + 7) / 8 < cus)
                return launch_b1_lds<T, 1, 8, 16384, 1>(w, n, k, rb, x, y, s);
            return launch_b1_lds<T, 2, 8, 16384, 1>(w, n, k, rb, x, y, s);
        }
    }
    if (gemv_mfma_supported(T, batch))
        return launch_gemv_mfma(T, w, n, k, rb, x, batch, y, s);
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
    const uint8_t *wb = (const uint8_t *)w;
    switch (type) {
    case T_Q4_0: return launch_t<T_Q4_0>(wb, n, k, rb, x, batch, y, s);
    case T_Q8_0: return launch_t<T_Q8_0>(wb, n, k, rb, x, batch, y, s);
    case T_Q4_K: return launch_t<T_Q4_K>(wb, n, k, rb, x, batch, y, s);
    case T_Q6_K: return launch_t<T_Q6_K>(wb, n, k, rb, x, batch, y, s);
    case T_Q5_0: return launch_t<T_Q5_0>(wb, n, k, rb, x, batch, y, s);
    case T_Q5_K: return launch_t<T_Q5_K>(wb, n, k, rb, x, batch, y, s);
    default: return hipErrorInvalidValue;
    }
}

template <int T>
static hipError_t launch_multi_t(int np, const void *const *w, const int64_t *n, int64_t k, size_t rb,
                                 const float *const *x, int batch, float *const *y, hipStream_t s)
{
    if (batch == 1 && rb % 16 == 0 && k <= 64 * GemvUnit<T>::UE) {
        // empty problems are left out of the tables: every table entry then
        // has rows (and a weight pointer), so a wave with no item of its own,
        // whose dummy loads read the first bytes of the last problem, never
        // meets an empty one (whose w may be NULL)
        int live[GEMV_MAXP];
        int i0 = 0;
        while (i0 < np) {
            int cnt = 0;
            for (; i0 < np && cnt < GEMV_MAXP; ++i0)
                if (n[i0] > 0)
                    live[cnt++] = i0;
            if (cnt == 0)
                break;
            GemvProbs P{};
            P.np = cnt;
            // one x for every problem of this launch: x staged once in LDS
            // per workgroup (gemv3m), one row per item; else gemv2m
            bool shared = true;
            int64_t rows = 0;
            for (int i = 0; i < P.np; ++i) {
                shared = shared && x[live[i]] == x[live[0]];
                rows += n[live[i]];
            }
            const int R = shared ? 1 : 2;
            P.rg0[0] = 0;
            for (int i = 0; i < P.np; ++i) {
                const int j = live[i];
                P.w[i] = (const uint8_t *)w[j];
                P.x[i] = x[j];
                P.y[i] = y[j];
                P.n[i] = (int)n[j];
                P.rg0[i + 1] = P.rg0[i] + (int)((n[j] + R - 1) / R);
            }
            constexpr bool small_blocks = GemvUnit<T>::UE == 32;
            const hipError_t e = !shared ? launch_b1_table<T, 2>(P, k, rb, s)
                                 : small_blocks && rows >= 4096 ? launch_b1_table_xlds<T, 16>(P, k, rb, s)
                                                                : launch_b1_table_xlds<T, 8>(P, k, rb, s);
            if (e != hipSuccess)
                return e;
        }
        return hipSuccess;
    }
    // other shapes: one launch per problem
    for (int i = 0; i < np; ++i) {
        if (n[i] == 0)
            continue;
        const hipError_t e = launch_t<T>((const uint8_t *)w[i], n[i], k, rb, x[i], batch, y[i], s);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

hipError_t launch_gemv_multi(int type, int np, const void *const *w, const int64_t *n, int64_t k, size_t rb,
                             const float *const *x, int batch, float *const *y, hipStream_t s)
{
    switch (type) {
    case T_Q4_0: return launch_multi_t<T_Q4_0>(np, w, n, k, rb, x, batch, y, s);
    case T_Q8_0: return launch_multi_t<T_Q8_0>(np, w, n, k, rb, x, batch, y, s);
    case T_Q4_K: return launch_multi_t<T_Q4_K>(np, w, n, k, rb, x, batch, y, s);
    case T_Q6_K: return launch_multi_t<T_Q6_K>(np, w, n, k, rb, x, batch, y, s);
    case T_Q5_0: return launch_multi_t<T_Q5_0>(np, w, n, k, rb, x, batch, y, s);
    case T_Q5_K: return launch_multi_t<T_Q5_K>(np, w, n, k, rb, x, batch, y, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
