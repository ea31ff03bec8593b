// qmm_gemv_mfma.hip -- decode GEMV for small batches (2..8 activation rows)
// on the fp16 matrix cores, for the K-quant formats Q4_K and Q6_K.
//
// At batch 1 the decode GEMV is a pure weight stream (qmm_gemv.hip).  With a
// few activation rows the same weight bytes feed B dot products each, and the
// fp32 vector ALU would need 2B flops per weight on top of the decode; the
// matrix cores take that work instead.  The contraction per super-block of
// 256 weights is one 16 x 16 x 256 product:
//
//   A (16 x 256, fp16): activation rows.  Row 2b holds the high part of
//     x[b] * 2^sh, row 2b+1 the remainder times 2^11 (both fp16, round to
//     nearest even), so hi + 2^-11 lo carries about 22 significant bits of
//     the fp32 input.  sh is a power of two per (row b, super-block) that puts
//     the block's largest |x| in [2^14, 2^15): no fp16 overflow, and both
//     parts stay normal for every element down to 2^-29 of the largest.
//   B (256 x 16, fp16): 16 weight rows, two operands whose sum is the
//     weight, so that every product is taken with the element's own weight.
//     Q6_K: (q - 32)(sc - b) and (q - 32) b, b = sc & 1: an even integer of
//     magnitude at most 4096 and one of at most 32, both exact in fp16, each
//     formed by one fused fp16 multiply-add from a biased code (256 + q); the
//     super-block scale d is applied to the fp32 sums.  Q4_K: the weight
//     d sc q - dmin m itself, formed per element in fp32 exactly as the
//     dequantizer forms it (after a power of two 2^s per super-block that
//     keeps it below 2^15), and split into hi = fp16(w) and the remainder
//     fp16(w - hi), which holds it to 22 bits (a subnormal, 2^-25 absolute,
//     only for weights below 2^-18 of the block's scale).  No cancellation
//     happens after a rounding: a row of zero weights gives exactly 0.
//   C (16 x 16, fp32): the sum over the super-block of both weight parts;
//     then, per row j and batch b, y[b][j] += 2^-sh (C_hi + 2^-11 C_lo)
//     (Q6_K: times d; Q4_K: times 2^-s) in fp32, C_hi and C_lo being the
//     rows of x's two fp16 parts.
//
// Block layouts: Q4_K fp16 d, fp16 dmin, 12 bytes of packed 6-bit scales and
// mins, 128 code bytes (sub-block j of 32: nibble j%2 of bytes 32(j/2)..+31);
// Q6_K 128 bytes of low nibbles, 64 bytes of 2-bit high parts, 16 int8
// scales (one per 16 weights), fp16 d (shimmy "Architecture", Quantization
// table; dotLLM "GPU Inference", Quantization on GPU table, as read with the
// Llama-3-8B Q4_K and Q4_K_M-mix workloads).
//
// Work split.  One workgroup of 8 waves per compute unit, persistent over a
// contiguous range of 16-row tiles.  The waves split K: wave w owns a
// contiguous run of super-blocks and keeps their A fragments in registers
// (converted once, reused for every tile), streams the B bytes of its run for
// each tile (the next tile's bytes in flight while the current one is decoded)
// and leaves a partial sum per tile in LDS; after every 8 tiles the partials
// are added in a fixed order and stored, so results do not depend on timing.
// When a wave's run is longer than two super-blocks, it is taken two at a time
// (fragments converted again per 8 tiles) and the partials accumulate in LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "qmm_device.h"
#include "qmm_launch.h"

namespace qmm {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float fl2 __attribute__((ext_vector_type(2)));
typedef float fl4 __attribute__((ext_vector_type(4)));

constexpr int GB_W = 8;    // waves per workgroup
constexpr int GB_TC = 8;   // tiles between cross-wave reductions
constexpr int GB_C = 2;    // super-blocks per wave held in registers at a time

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ uint32_t as_u(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// fp16 round-to-nearest-even of two fp32 values, packed (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pk_rne(float a, float b)
{
    return as_u(__builtin_convertvector((fl2){a, b}, h2));
}

// Bytes i and j of v as the fp16 pair (bias + byte_i, bias + byte_j), bias
// given by the high byte hb: 0x64 -> 1024 (spacing 1), 0x60 -> 512 (the byte
// is then twice the value added).
__device__ __forceinline__ uint32_t byte_pair(uint32_t hb4, uint32_t v, uint32_t sel)
{
    return __builtin_amdgcn_perm(hb4, v, sel);
}

// ------------------------------------------------------------- A fragments --
// The k order inside a super-block.  MFMA i (0..7) of a super-block takes, in
// lane group G = lane/16, the 8 elements with lane-local index
// 8i + {0, 2, 1, 3, 4, 6, 5, 7} of the 64 elements that group owns: pairs of
// elements two apart share one packed register on the weight side, where a
// dword holds 4 code bytes and one mask takes bytes 0 and 2.
//   Q4_K: group G owns elements 64G .. 64G+63 (sub-blocks 2G, 2G+1).
//   Q6_K: group G owns, for g' = 0..3, the 16 elements
//         128(G/2) + 32g' + 16(G%2) + 0..15 (lane-local index 16g' + l).
struct XFrag {
    h8 a[8];      // A operands of the 8 MFMAs of the super-block
    float xs0;    // 2^-sh of batch rows 2G and 2G+1 (C layout of this lane)
    float xs1;
};

// Element offset of the q-th group of 4 activations of lane group G in a
// 256-element block (the k order above).
template <int T>
__device__ __forceinline__ int xgroup_off(int G, int q)
{
    return T == T_Q4_K ? 64 * G + 4 * q : 128 * (G >> 1) + 16 * (G & 1) + 32 * (q >> 2) + 4 * (q & 3);
}

// The two lanes of a batch row (rows 2b and 2b+1 of A, lanes l and l ^ 1)
// split its 64 activations of a block: fragment i takes groups 2i and 2i+1,
// and the lane of parity p loads group 2i + p.
template <int T>
__device__ __forceinline__ void load_x(const float *__restrict__ xb, int G, fl4 v[8])
{
    const int p = threadIdx.x & 1;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        v[i] = *(const fl4 *)(xb + xgroup_off<T>(G, 2 * i + p));
}

// The partner lane's value of v (lanes l and l ^ 1 swap, DPP quad_perm 1,0,3,2).
__device__ __forceinline__ uint32_t swap_pair(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xf, 0xf, false);
}

// A fragments of one block from this lane's half of its row's activations.
// Row 2b keeps hi = fp16(x 2^sh), row 2b+1 the fp16 of the remainder times
// 2^11 (exact in fp32, at most 16 in magnitude).  Each lane forms hi and lo
// of its own groups and takes the other half of its fragment from the
// partner lane: 22 instead of 32 operations per fragment.
template <int T>
__device__ __forceinline__ void convert_x(fl4 v[8], XFrag &f)
{
    const int lane = threadIdx.x & 63, G = lane >> 4;
    const bool odd = (lane & 1) != 0;
    float m = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q)
        m = fmaxf(fmaxf(m, fmaxf(fabsf(v[q][0]), fabsf(v[q][1]))), fmaxf(fabsf(v[q][2]), fabsf(v[q][3])));
    m = fmaxf(m, __builtin_bit_cast(float, swap_pair(__builtin_bit_cast(uint32_t, m))));
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    // m in [2^(e-1), 2^e): scale the block so that it lands in [2^14, 2^15)
    const int e = __builtin_amdgcn_frexp_expf(m);
    const int sh = min(max(15 - e, -128), 126);
    // -1 the optimizer cannot see: a + (-1) hi stays one v_fma_mix_f32 that
    // reads hi in place (not a convert and a subtract)
    const float n1 = __builtin_bit_cast(float, opaque(0xbf800000u));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float a0 = __builtin_amdgcn_ldexpf(v[i][0], sh), a1 = __builtin_amdgcn_ldexpf(v[i][1], sh);
        const float a2 = __builtin_amdgcn_ldexpf(v[i][2], sh), a3 = __builtin_amdgcn_ldexpf(v[i][3], sh);
        // element pairs (0, 2) and (1, 3) of the group
        const uint32_t H0 = pk_rne(a0, a2), H1 = pk_rne(a1, a3);
        const h2 h0 = as_h2(H0), h1 = as_h2(H1);
        const uint32_t L0 = pk_rne(fmaf(n1, (float)h0[0], a0) * 2048.f, fmaf(n1, (float)h0[1], a2) * 2048.f);
        const uint32_t L1 = pk_rne(fmaf(n1, (float)h1[0], a1) * 2048.f, fmaf(n1, (float)h1[1], a3) * 2048.f);
        // the partner needs lo of an even lane's group, hi of an odd lane's
        const uint32_t R0 = swap_pair(odd ? H0 : L0), R1 = swap_pair(odd ? H1 : L1);
        // even lane (hi row): own group first; odd lane (lo row): own second
        const uint32_t o0 = odd ? R0 : H0, o1 = odd ? R1 : H1, o2 = odd ? L0 : R0, o3 = odd ? L1 : R1;
        f.a[i] = __builtin_bit_cast(h8, (u32x4){o0, o1, o2, o3});
    }
    const float xs = __builtin_amdgcn_ldexpf(1.f, -sh);
    f.xs0 = __shfl(xs, 4 * G);        // row 4G   = batch 2G
    f.xs1 = __shfl(xs, 4 * G + 2);    // row 4G+2 = batch 2G+1
}

// ------------------------------------------------------------- B operands --
template <int T> struct WRawB;

// Q4_K, lane (n, g): header (d, dmin, 12 scale bytes) and code bytes
// 32g .. 32g+31 (sub-blocks 2g and 2g+1).
template <> struct WRawB<T_Q4_K> {
    u32x4 hd, c0, c1;
};

// Q6_K, lane (n, g), h = g/2, l = g%2: ql bytes 64h+16l (+16) and 64h+32+16l
// (+16), qh bytes 32h+16l (+16), scale bytes 8h..8h+7, d.  Super-blocks are
// only 2-byte aligned (210 bytes): every run is read as aligned dwords plus a
// trailing 16-bit word and realigned at decode time.
template <> struct WRawB<T_Q6_K> {
    u32x4 q0, q1, qh;
    uint32_t q0t, q1t, qht;
    uint32_t s0, s1, st;
    uint32_t d;
    uint32_t sh;
};

template <int T>
__device__ __forceinline__ void load_b(const uint8_t *__restrict__ p, int64_t off, int g, WRawB<T> &r);

template <>
__device__ __forceinline__ void load_b<T_Q4_K>(const uint8_t *__restrict__ p, int64_t off, int g, WRawB<T_Q4_K> &r)
{
    const uint8_t *b = p + off;
    r.hd = *(const u32x4 *)b;
    r.c0 = *(const u32x4 *)(b + 16 + 32 * g);
    r.c1 = *(const u32x4 *)(b + 32 + 32 * g);
}

template <>
__device__ __forceinline__ void load_b<T_Q6_K>(const uint8_t *__restrict__ p, int64_t off, int g, WRawB<T_Q6_K> &r)
{
    const uint32_t sh = (uint32_t)off & 2u;        // p is 16-byte aligned
    const uint8_t *a = p + (off - sh);             // dword aligned
    const int h = g >> 1, l = g & 1;
    const int o0 = 64 * h + 16 * l, o1 = o0 + 32, oh = 128 + 32 * h + 16 * l, os = 192 + 8 * h;
    r.q0 = *(const u32x4 *)(a + o0);
    r.q0t = *(const uint16_t *)(a + o0 + 16);
    r.q1 = *(const u32x4 *)(a + o1);
    r.q1t = *(const uint16_t *)(a + o1 + 16);
    r.qh = *(const u32x4 *)(a + oh);
    r.qht = *(const uint16_t *)(a + oh + 16);
    const uint32_t *sp = (const uint32_t *)(a + os);
    r.s0 = sp[0];
    r.s1 = sp[1];
    r.st = *(const uint16_t *)(a + os + 8);
    r.d = *(const uint16_t *)(p + off + 208);
    r.sh = sh;
}

// Keep every loaded dword live up to the decode, so that no register of a
// load in flight is reused as a temporary (the write-after-write would wait
// for all outstanding loads).
template <int T>
__device__ __forceinline__ void keep(const WRawB<T> &r)
{
    constexpr int N = sizeof(WRawB<T>) / 4;
    const uint32_t *v = (const uint32_t *)&r;
#pragma unroll
    for (int i = 0; i < N; ++i)
        asm volatile("" : : "v"(v[i]));
}

__device__ __forceinline__ h2 h2c(float v) { return (h2){(_Float16)v, (_Float16)v}; }

// One super-block of one 16-row tile: 8 (+1) MFMAs and the fp32 scaling into
// acc0 / acc1 (batch rows 2g, 2g+1 of weight row n of the tile).
template <int T>
__device__ __forceinline__ void sb_dot(const WRawB<T> &r, const XFrag &f, int g, float &acc0, float &acc1);

template <>
__device__ __forceinline__ void sb_dot<T_Q4_K>(const WRawB<T_Q4_K> &r, const XFrag &f, int g, float &acc0,
                                               float &acc1)
{
    keep(r);
    const uint32_t hy = r.hd.y, hz = r.hd.z, hw = r.hd.w;
    // 6-bit scales / mins of sub-blocks 0..3 (lo) and 4..7 (hi), one per byte
    const uint32_t sclo = hy & 0x3f3f3f3fu;
    const uint32_t schi = (hw & 0x0f0f0f0fu) | ((hy >> 2) & 0x30303030u);
    const uint32_t mlo = hz & 0x3f3f3f3fu;
    const uint32_t mhi = ((hw >> 4) & 0x0f0f0f0fu) | ((hz >> 2) & 0x30303030u);
    const uint32_t sc = (g >= 2 ? schi : sclo) >> (16 * (g & 1));   // bytes: sc_2g, sc_2g+1
    const uint32_t mm = (g >= 2 ? mhi : mlo) >> (16 * (g & 1));     // bytes: m_2g, m_2g+1
    // 2^s with |w| 2^s < 1024 max(|d|, |dmin|) 2^s <= 2^15
    const float d = h2f(r.hd.x & 0xffffu), dmin = h2f(r.hd.x >> 16);
    const int s = 5 - __builtin_amdgcn_frexp_expf(fmaxf(fabsf(d), fabsf(dmin)));
    const float ds = __builtin_amdgcn_ldexpf(d, s), dms = __builtin_amdgcn_ldexpf(dmin, s);
    // A code masked in place is an fp16 subnormal: q 2^-24 for a low nibble,
    // q 2^-20 for a high one.  The scales carry the inverse power of two and
    // 2^11: W = 2^11 2^s w, one rounding of the exact q d sc - dmin m.
    const float dsc0 = ds * ub0(sc) * 0x1p35f, dsc1 = ds * ub1(sc) * 0x1p31f;
    const float ndm0 = -(dms * ub0(mm)) * 0x1p11f, ndm1 = -(dms * ub1(mm)) * 0x1p11f;
    const uint32_t D[8] = {r.c0.x, r.c0.y, r.c0.z, r.c0.w, r.c1.x, r.c1.y, r.c1.z, r.c1.w};
    uint32_t D8[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
        D8[t] = D[t] >> 8;
    fl4 ch = {0.f, 0.f, 0.f, 0.f}, cl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int t0 = 2 * (i & 3);
        const bool hn = i >= 4;
        const uint32_t msk = hn ? 0x00f000f0u : 0x000f000fu;      // codes of bytes 0, 2
        const float dsc = hn ? dsc1 : dsc0, ndm = hn ? ndm1 : ndm0;
        uint32_t oh[4], ol[4];
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) {
            const uint32_t v = (pr & 1) ? D8[t0 + (pr >> 1)] : D[t0 + (pr >> 1)];
            const h2 e = as_h2(opaque(v & msk));
            // W (v_fma_mix_f32 reads the fp16 code), hi = fp16(2^s w) and
            // lo = fp16(W - 2^11 hi), the remainder times 2^11 (exact in
            // fp32, one rounding).  Full-rate operations only: the fused
            // converts v_fma_mixlo/mixhi_f16 issue at about half the rate of
            // an fma on this chip, v_cvt_pk_f16_f32 at the full rate.
            const float W0 = fmaf((float)e[0], dsc, ndm), W1 = fmaf((float)e[1], dsc, ndm);
            oh[pr] = pk_rne(W0 * 0x1p-11f, W1 * 0x1p-11f);
            const h2 h = as_h2(oh[pr]);
            ol[pr] = pk_rne(fmaf((float)h[0], -2048.f, W0), fmaf((float)h[1], -2048.f, W1));
        }
        ch = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.a[i], __builtin_bit_cast(h8, (u32x4){oh[0], oh[1], oh[2], oh[3]}),
                                                    ch, 0, 0, 0);
        cl = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.a[i], __builtin_bit_cast(h8, (u32x4){ol[0], ol[1], ol[2], ol[3]}),
                                                    cl, 0, 0, 0);
    }
    const float u = __builtin_amdgcn_ldexpf(1.f, -s);
    acc0 = fmaf(f.xs0 * u, fmaf(0x1p-11f, fmaf(0x1p-11f, cl[1], cl[0]), fmaf(0x1p-11f, ch[1], ch[0])), acc0);
    acc1 = fmaf(f.xs1 * u, fmaf(0x1p-11f, fmaf(0x1p-11f, cl[3], cl[2]), fmaf(0x1p-11f, ch[3], ch[2])), acc1);
}

template <>
__device__ __forceinline__ void sb_dot<T_Q6_K>(const WRawB<T_Q6_K> &r, const XFrag &f, int g, float &acc0,
                                               float &acc1)
{
    keep(r);
    const uint32_t sh = r.sh;
    const uint32_t Q0[4] = {align_bytes(r.q0.y, r.q0.x, sh), align_bytes(r.q0.z, r.q0.y, sh),
                            align_bytes(r.q0.w, r.q0.z, sh), align_bytes(r.q0t, r.q0.w, sh)};
    const uint32_t Q1[4] = {align_bytes(r.q1.y, r.q1.x, sh), align_bytes(r.q1.z, r.q1.y, sh),
                            align_bytes(r.q1.w, r.q1.z, sh), align_bytes(r.q1t, r.q1.w, sh)};
    const uint32_t H[4] = {align_bytes(r.qh.y, r.qh.x, sh), align_bytes(r.qh.z, r.qh.y, sh),
                           align_bytes(r.qh.w, r.qh.z, sh), align_bytes(r.qht, r.qh.w, sh)};
    // int8 scales 8h + l + 2g' (g' = 0..3): bytes l, l+2 of the two dwords,
    // biased to sc + 128 and split into the even part sc - b and the low bit b
    const uint32_t S0 = align_bytes(r.s1, r.s0, sh) ^ 0x80808080u, S1 = align_bytes(r.st, r.s1, sh) ^ 0x80808080u;
    const uint32_t l = (uint32_t)(g & 1);
    const uint32_t sel0 = 0x04000400u + l * 0x00010001u, sel1 = sel0 + 0x00020002u;
    const h2 k1152 = h2c(1152.f), k1024 = h2c(1024.f), kn288 = h2c(-288.f);
    h2 se[4], ne[4], sb[4], nb[4];
#pragma unroll
    for (int gp = 0; gp < 4; ++gp) {
        const uint32_t S = gp < 2 ? S0 : S1, sel = (gp & 1) ? sel1 : sel0;
        se[gp] = as_h2(byte_pair(0x64646464u, S & 0xfefefefeu, sel)) - k1152;   // sc - b, even
        sb[gp] = as_h2(byte_pair(0x64646464u, S & 0x01010101u, sel)) - k1024;   // b = sc & 1
        ne[gp] = se[gp] * kn288;
        nb[gp] = sb[gp] * kn288;
    }
    fl4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int gp = i >> 1, t0 = 2 * (i & 1);
        uint32_t oe[4], ob[4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const uint32_t ql = (gp & 1) ? Q1[t0 + tt] : Q0[t0 + tt];
            // 4q per byte: low 4 bits from ql (nibble gp/2) to bits 2-5, bits
            // 4-5 of q from qh (bits 2gp..2gp+1) to bits 6-7
            const uint32_t lo4 = gp < 2 ? (ql << 2) & 0x3c3c3c3cu : (ql >> 2) & 0x3c3c3c3cu;
            const uint32_t q4 = lo4 | ((H[t0 + tt] << (6 - 2 * gp)) & 0xc0c0c0c0u);
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                // bytes (pp, pp+2) -> fp16 256 + q
                const h2 code = as_h2(byte_pair(0x5c5c5c5cu, q4, pp ? 0x04030401u : 0x04020400u));
                // (q - 32)(sc - b): even, at most 4096 in magnitude; (q - 32) b:
                // both exact in fp16, each from one fused multiply-add
                oe[2 * tt + pp] = as_u(__builtin_elementwise_fma(code, se[gp], ne[gp]));
                ob[2 * tt + pp] = as_u(__builtin_elementwise_fma(code, sb[gp], nb[gp]));
            }
        }
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.a[i], __builtin_bit_cast(h8, (u32x4){oe[0], oe[1], oe[2], oe[3]}),
                                                   c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.a[i], __builtin_bit_cast(h8, (u32x4){ob[0], ob[1], ob[2], ob[3]}),
                                                   c, 0, 0, 0);
    }
    const float d = h2f(r.d);
    acc0 = fmaf(f.xs0 * d, fmaf(0x1p-11f, c[1], c[0]), acc0);
    acc1 = fmaf(f.xs1 * d, fmaf(0x1p-11f, c[3], c[2]), acc1);
}

// ------------------------------------------------------------------ kernel --
// One run of up to two super-blocks (sa, sa+1 if TWO) over cnt tiles from
// tile0: fragments (if convert), then the tiles with the next tile's bytes in
// flight; each tile's partial goes to slot[tile][wave][lane] (added to what is
// there if accumulate).
template <int T, bool TWO>
__device__ __forceinline__ void run_piece(const uint8_t *__restrict__ w, int64_t rb, int n, int tile0, int cnt,
                                          int sa, bool convert, const float *__restrict__ xrow, XFrag (&xf)[GB_C],
                                          fl2 (*slot)[GB_W][64], bool accumulate)
{
    using F = Fmt<T>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nl = lane & 15, g = lane >> 4;
    auto off = [&](int tt, int s) -> int64_t {
        const int row = min((tile0 + tt) * 16 + nl, n - 1);
        return (int64_t)row * rb + (int64_t)s * F::BB;
    };
    WRawB<T> A0, A1, B0, B1;
    if (convert) {
        // activations of both super-blocks first: the waits for them then
        // leave the weight loads below in flight (loads complete in order)
        fl4 v[8], v2[8];
        load_x<T>(xrow + 256 * sa, g, v);
        if (TWO)
            load_x<T>(xrow + 256 * (sa + 1), g, v2);
        load_b<T>(w, off(0, sa), g, A0);
        if (TWO)
            load_b<T>(w, off(0, sa + 1), g, A1);
        convert_x<T>(v, xf[0]);
        if (TWO)
            convert_x<T>(v2, xf[1]);
    } else {
        load_b<T>(w, off(0, sa), g, A0);
        if (TWO)
            load_b<T>(w, off(0, sa + 1), g, A1);
    }
    auto tile = [&](const WRawB<T> &r0, const WRawB<T> &r1, int tt) {
        float a0 = 0.f, a1 = 0.f;
        sb_dot<T>(r0, xf[0], g, a0, a1);
        if (TWO)
            sb_dot<T>(r1, xf[1], g, a0, a1);
        fl2 part = {a0, a1};
        if (accumulate)
            part += slot[tt][wave][lane];
        slot[tt][wave][lane] = part;
    };
    int tt = 0;
    for (; tt + 2 <= cnt; tt += 2) {
        load_b<T>(w, off(tt + 1, sa), g, B0);
        if (TWO)
            load_b<T>(w, off(tt + 1, sa + 1), g, B1);
        tile(A0, A1, tt);
        const int tn = min(tt + 2, cnt - 1);   // past the end: a harmless re-read
        load_b<T>(w, off(tn, sa), g, A0);
        if (TWO)
            load_b<T>(w, off(tn, sa + 1), g, A1);
        tile(B0, B1, tt + 1);
    }
    if (tt < cnt)
        tile(A0, A1, tt);
}

template <int T>
__global__ void __launch_bounds__(64 * GB_W)
gemvb_kernel(const uint8_t *__restrict__ w, int n, int k, int64_t rb, const float *__restrict__ x, int batch,
             float *__restrict__ y)
{
    __shared__ fl2 red[2][GB_TC][GB_W][64];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int S = k / 256;
    const int s_begin = wave * S / GB_W, s_end = (wave + 1) * S / GB_W;
    const int npc = (s_end - s_begin + GB_C - 1) / GB_C;
    const bool multi = S > GB_C * GB_W;       // the same for every wave
    const int ntiles = (n + 15) >> 4;
    const int per = ntiles / (int)gridDim.x, rem = ntiles - per * (int)gridDim.x;
    const int t_begin = (int)blockIdx.x * per + min((int)blockIdx.x, rem);
    const int t_count = per + ((int)blockIdx.x < rem ? 1 : 0);
    // activation row of this lane's A rows (rows past the batch repeat the
    // last one; their outputs are never stored)
    const float *xrow = x + (int64_t)min((lane & 15) >> 1, batch - 1) * k;

    XFrag xf[GB_C];
    int buf = 0;
    for (int c0 = 0; c0 < t_count; c0 += GB_TC, buf ^= 1) {
        const int cnt = min(GB_TC, t_count - c0);
        const int tile0 = t_begin + c0;
        for (int p = 0; p < npc; ++p) {
            const int sa = s_begin + GB_C * p;
            const bool convert = multi || c0 == 0;
            if (sa + 1 < s_end)
                run_piece<T, true>(w, rb, n, tile0, cnt, sa, convert, xrow, xf, red[buf], p > 0);
            else
                run_piece<T, false>(w, rb, n, tile0, cnt, sa, convert, xrow, xf, red[buf], p > 0);
        }
        if (npc == 0) {
            for (int tt = 0; tt < cnt; ++tt)
                red[buf][tt][wave][lane] = (fl2){0.f, 0.f};
        }
        __syncthreads();
        // fixed-order sum over the waves, one (tile, lane) pair per thread
        for (int j = threadIdx.x; j < cnt * 64; j += 64 * GB_W) {
            const int tt = j >> 6, ln = j & 63;
            fl2 s = red[buf][tt][0][ln];
#pragma unroll
            for (int ww = 1; ww < GB_W; ++ww)
                s += red[buf][tt][ww][ln];
            const int row = (tile0 + tt) * 16 + (ln & 15), b0 = 2 * (ln >> 4);
            if (row < n) {
                if (b0 < batch)
                    y[(int64_t)b0 * n + row] = s[0];
                if (b0 + 1 < batch)
                    y[(int64_t)(b0 + 1) * n + row] = s[1];
            }
        }
        // red is double-buffered: the next chunk writes the other half, and
        // this half is written again only after the next chunk's barrier
    }
}

// ----------------------------------------------------- single-run kernel --
// K of at most 16 super-blocks (every wave owns at most two): the A fragments
// are converted once per workgroup and the weight stream runs through a ring
// of D tiles per wave (D - 1 tiles of bytes in flight while one is decoded;
// a workgroup with t tiles takes D = min(t + 1, the type's depth)).  The
// activations reach LDS by direct global->LDS loads, issued before the first
// weight loads: waiting for them (the memory counter completes in order)
// leaves those weight loads in flight while the fragments are built.
template <int T> struct RingDepth { static constexpr int D = 3; };
template <> struct RingDepth<T_Q4_K> { static constexpr int D = 4; };

constexpr int XROW = 256 + 4;    // floats per staged activation row (16-byte pad: fewer bank conflicts)

// Loads per WRawB<T> (each counts once in the vector memory counter).
template <int T> struct RawLoads { static constexpr int N = 3; };
template <> struct RawLoads<T_Q6_K> { static constexpr int N = 9; };

// s_waitcnt with only the vector memory counter limited to n (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
#define QMM_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8)))

// Up to MP_MAX problems of one type and k sharing x (q / k, gate / up of a
// layer): their 16-row tiles are numbered one after another (tile0), and a
// workgroup's run of tiles may cross from one problem into the next.
constexpr int MP_MAX = 8;
struct MProbs {
    const uint8_t *w[MP_MAX];
    float *y[MP_MAX];
    int n[MP_MAX];
    int tile0[MP_MAX + 1];   // first tile of each problem; tile0[np] = all tiles
    int np;
};

struct TileRef {
    const uint8_t *w;
    float *y;
    int n, row0;             // the problem's rows, the tile's first row in it
};

// Tile ti's problem (wave-uniform): the number of problem starts past the
// first at or below ti (the starts never decrease).  The starts are read at
// constant indices, so that they are loaded once, ahead of the tile loop, as
// independent scalar loads; the problem's fields are then one round of loads
// (a scan bounded by np would chain one load round trip per problem).
__device__ __forceinline__ TileRef tile_ref(const MProbs &P, int ti)
{
    int t0[MP_MAX];
#pragma unroll
    for (int q = 0; q < MP_MAX; ++q)
        t0[q] = P.tile0[q];
    const int np = P.np;
    int p = 0;
#pragma unroll
    for (int q = 1; q < MP_MAX; ++q)
        p += (int)(q < np) & (int)(ti >= t0[q]);
    return TileRef{P.w[p], P.y[p], P.n[p], (ti - P.tile0[p]) * 16};
}

// Cross-wave sum of tile j (red[j]) stored to its problem's y: one
// (row, batch pair) per thread of the first 64 j + 64.
__device__ __forceinline__ void store_tile(const MProbs &P, int ti, const fl2 (*redj)[64], int ln, int batch)
{
    fl2 s = redj[0][ln];
#pragma unroll
    for (int ww = 1; ww < GB_W; ++ww)
        s += redj[ww][ln];
    const TileRef R = tile_ref(P, ti);
    const int row = R.row0 + (ln & 15), b0 = 2 * (ln >> 4);
    if (row < R.n) {
        if (b0 < batch)
            R.y[(int64_t)b0 * R.n + row] = s[0];
        if (b0 + 1 < batch)
            R.y[(int64_t)(b0 + 1) * R.n + row] = s[1];
    }
}

template <int T, bool TWO, int D>
__device__ __forceinline__ void single_run(const MProbs &P, int k, int64_t rb, const float *__restrict__ x,
                                           int batch, int t_begin, int t_count, int sa, float (*xs)[8][XROW],
                                           fl2 (*red)[GB_W][64])
{
    using F = Fmt<T>;
    constexpr int NC = TWO ? 2 : 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nl = lane & 15, g = lane >> 4;
    // this wave's activations, 1 KB per (row, super-block), 16 bytes per lane;
    // rows past the batch repeat the last one (never stored)
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int b = 0; b < 8; ++b)
            __builtin_amdgcn_global_load_lds(
                (const void *)(x + (int64_t)min(b, batch - 1) * k + 256 * (sa + c) + 4 * lane),
                (__attribute__((address_space(3))) void *)&xs[c][b][0], 16, 0, 0);

    struct Slot {
        WRawB<T> r[NC];
    };
    Slot ring[D];
    auto load_tile = [&](Slot &sl, int t) {
        const TileRef R = tile_ref(P, t_begin + min(t, t_count - 1));
        const int row = min(R.row0 + nl, R.n - 1);
        const int64_t base = (int64_t)row * rb + (int64_t)sa * F::BB;
#pragma unroll
        for (int c = 0; c < NC; ++c)
            load_b<T>(R.w, base + c * F::BB, g, sl.r[c]);
    };
#pragma unroll
    for (int d = 0; d < D - 1; ++d)
        load_tile(ring[d], d);
    __builtin_amdgcn_sched_barrier(0);
    // the activation loads were issued before the ring: wait for them only
    // (the first D - 1 tiles stay in flight while the fragments are built)
    QMM_WAIT_VMCNT((D - 1) * NC * RawLoads<T>::N);
    __builtin_amdgcn_sched_barrier(0);
    XFrag xf[NC];
    {
        const int r = lane & 15, b = min(r >> 1, batch - 1);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            fl4 v[8];
            load_x<T>(xs[c][b], g, v);   // b: this lane's row (min(r/2, batch - 1))
            convert_x<T>(v, xf[c]);
        }
    }
    for (int t = 0; t < t_count; t += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            // past the workgroup's last tile: a re-read of that tile
            // (unconditional: a branch around the loads makes the compiler
            // wait for every load in flight)
            load_tile(ring[(j + D - 1) % D], t + j + D - 1);
            if (t + j < t_count) {
                float a0 = 0.f, a1 = 0.f;
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    sb_dot<T>(ring[j].r[c], xf[c], g, a0, a1);
                red[j][wave][lane] = (fl2){a0, a1};
            }
        }
        // cross-wave sum of these D tiles (raw barriers: no wait for the
        // weight loads in flight)
        lds_barrier();
        const int nt = min(D, t_count - t);
        if ((int)threadIdx.x < nt * 64)
            store_tile(P, t_begin + t + (threadIdx.x >> 6), red[threadIdx.x >> 6], threadIdx.x & 63, batch);
        lds_barrier();
    }
}

// ------------------------------------------------ staged Q6_K tiles --
// Q6_K rows of 4096 weights (16 super-blocks, 3360 bytes, 16-byte aligned):
// the workgroup moves each 16-row tile (16 x 3360 contiguous bytes) with
// coalesced 16-byte loads, 7 per thread, into LDS, and every wave reads its
// two super-blocks of the 16 rows back from there.  Per-lane loads of the
// scattered Q6_K fields (nine per super-block, five of them 2-byte tails)
// cost more than the bytes they bring: the 128256 x 4096 LM head at batch 8
// runs 130 us with them, 113 us staged (and 94 us with tile-contiguous loads
// decoding nothing meaningful: the loads alone).  The tile
// buffers (two, double buffered) overlay the activation staging, which is
// dead once the fragments are built.
constexpr int ST_RB = 16 * 210;                                    // bytes per row
constexpr int ST_CH = ST_RB;                                       // 16-byte chunks per 16-row tile
constexpr int ST_CPT = (ST_CH + 64 * GB_W - 1) / (64 * GB_W);     // chunks per thread (the last partial)

// Super-block sb of row nl of a staged tile (dword array): the fields of
// lane group g as load_b<T_Q6_K> reads them from global memory, here from
// dword-aligned LDS words (the block starts 2-byte aligned; each field run
// is read as aligned dwords plus the next one, realigned at decode time).
// Every word lies inside the tile: the last block of the last row starts
// 2 bytes past a dword boundary, so its last word ends on the tile's end.
__device__ __forceinline__ void lds_load_b_q6k(const uint32_t *tb, int nl, int sb, int g, WRawB<T_Q6_K> &r)
{
    const int off = nl * ST_RB + sb * 210;
    const uint32_t sh = (uint32_t)off & 2u;
    const uint32_t *a = tb + ((off - (int)sh) >> 2);
    const int h = g >> 1, l = g & 1;
    const int o0 = 16 * h + 4 * l, o1 = o0 + 8, oh = 32 + 8 * h + 4 * l, os = 48 + 2 * h;   // dwords
    r.q0 = (u32x4){a[o0], a[o0 + 1], a[o0 + 2], a[o0 + 3]};
    r.q0t = a[o0 + 4];
    r.q1 = (u32x4){a[o1], a[o1 + 1], a[o1 + 2], a[o1 + 3]};
    r.q1t = a[o1 + 4];
    r.qh = (u32x4){a[oh], a[oh + 1], a[oh + 2], a[oh + 3]};
    r.qht = a[oh + 4];
    r.s0 = a[os];
    r.s1 = a[os + 1];
    r.st = a[os + 2];
    r.d = (a[52] >> (8u * sh)) & 0xffffu;
    r.sh = sh;
}

template <int D>
__device__ __forceinline__ void staged_run_q6k(const MProbs &P, const float *__restrict__ x, int batch, int t_begin,
                                               int t_count, int sa, float (*xs)[8][XROW], uint32_t *tbuf,
                                               fl2 (*red)[GB_W][64])
{
    constexpr int T = T_Q6_K, NC = 2, k = 4096;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nl = lane & 15, g = lane >> 4;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int b = 0; b < 8; ++b)
            __builtin_amdgcn_global_load_lds(
                (const void *)(x + (int64_t)min(b, batch - 1) * k + 256 * (sa + c) + 4 * lane),
                (__attribute__((address_space(3))) void *)&xs[c][b][0], 16, 0, 0);

    struct Slot {
        u32x4 v[ST_CPT];
    };
    Slot ring[D];
    // chunk c of tile t: bytes 16 c of its 16 rows; past its problem's
    // matrix the last chunk of that matrix (rows past n are never stored).
    // Whole lines, each read once: non-temporal loads (128256 x 4096 at
    // batch 4 / 8: 114 / 116 -> 111 / 113 us; the per-lane field loads of
    // the other paths share lines between instructions and are 15% slower
    // with them)
    auto load_tile = [&](Slot &sl, int t) {
        const TileRef R = tile_ref(P, t_begin + min(t, t_count - 1));
        const int64_t base = (int64_t)R.row0 * ST_RB, last = (int64_t)R.n * ST_RB - 16;
#pragma unroll
        for (int i = 0; i < ST_CPT; ++i) {
            const int c = min(tid + 64 * GB_W * i, ST_CH - 1);
            sl.v[i] = __builtin_nontemporal_load((const u32x4 *)(R.w + min(base + 16 * c, last)));
        }
    };
#pragma unroll
    for (int d = 0; d < D - 1; ++d)
        load_tile(ring[d], d);
    __builtin_amdgcn_sched_barrier(0);
    QMM_WAIT_VMCNT((D - 1) * ST_CPT);
    __builtin_amdgcn_sched_barrier(0);
    XFrag xf[NC];
    {
        const int r = lane & 15, b = min(r >> 1, batch - 1);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            fl4 v[8];
            load_x<T>(xs[c][b], g, v);
            convert_x<T>(v, xf[c]);
        }
    }
    lds_barrier();   // every wave is done with the activation staging
    for (int t = 0; t < t_count; t += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int tt = t + j;
            // past the workgroup's last tile: a re-read of that tile
            // (unconditional: a branch around the loads makes the compiler
            // wait for every load in flight)
            load_tile(ring[(j + D - 1) % D], tt + D - 1);
            // buffer tt & 1 was last read for tile tt - 2, before the barrier of tile tt - 1
            uint32_t *buf = tbuf + (tt & 1) * (4 * ST_CH);
#pragma unroll
            for (int i = 0; i < ST_CPT; ++i) {
                const int c = tid + 64 * GB_W * i;
                if (c < ST_CH)
                    *(u32x4 *)(buf + 4 * c) = ring[j].v[i];
            }
            lds_barrier();
            if (tt < t_count) {
                float a0 = 0.f, a1 = 0.f;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    WRawB<T> r;
                    lds_load_b_q6k(buf, nl, sa + c, g, r);
                    sb_dot<T>(r, xf[c], g, a0, a1);
                }
                red[j][wave][lane] = (fl2){a0, a1};
            }
        }
        lds_barrier();
        const int nt = min(D, t_count - t);
        if ((int)threadIdx.x < nt * 64)
            store_tile(P, t_begin + t + (threadIdx.x >> 6), red[threadIdx.x >> 6], threadIdx.x & 63, batch);
        lds_barrier();
    }
}

template <int T>
__global__ void __launch_bounds__(64 * GB_W)
gemvb1_kernel(const float *__restrict__ x, int k, int64_t rb, int batch, int ntiles, int grid, const MProbs P)
{
    constexpr int DM = RingDepth<T>::D;
    // activation staging; for staged Q6_K tiles also the two tile buffers
    constexpr int XS_BYTES = GB_W * 2 * 8 * XROW * 4, TB_BYTES = 2 * 16 * ST_CH;
    static_assert(TB_BYTES <= XS_BYTES, "tile buffers overlay the activation staging");
    __shared__ __attribute__((aligned(16))) uint32_t lds_x[XS_BYTES / 4];
    __shared__ __attribute__((aligned(16))) fl2 red[DM][GB_W][64];
    float(*const xs)[2][8][XROW] = (float(*)[2][8][XROW])lds_x;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int S = k / 256;
    const int sa = wave * S / GB_W, ns = (wave + 1) * S / GB_W - sa;   // 0, 1 or 2 super-blocks
    // ntiles (all tiles of the table) and grid (gridDim.x) arrive as plain
    // arguments, preloaded into SGPRs, not read from the table or the
    // dispatch's implicit arguments
    const int per = ntiles / grid, rem = ntiles - per * grid;
    const int t_begin = (int)blockIdx.x * per + min((int)blockIdx.x, rem);
    const int t_count = per + ((int)blockIdx.x < rem ? 1 : 0);

    // ring depth: one tile per lane group of loads in flight per tile the
    // workgroup still has (no prefetch of tiles that do not exist)
    auto run = [&](auto two_c, auto d_c) {
        single_run<T, decltype(two_c)::value, decltype(d_c)::value>(P, k, rb, x, batch, t_begin, t_count, sa,
                                                                      xs[wave], red);
    };
    using std_true = std::integral_constant<bool, true>;
    using std_false = std::integral_constant<bool, false>;
    if constexpr (T == T_Q6_K) {
        // every wave owns two super-blocks; at least 4 tiles per workgroup
        // (with fewer, the per-tile barriers cost more than the scattered
        // loads: 1024 x 4096 at batch 8, 8.1 -> 9.8 us)
        if (k == 4096 && rb == ST_RB && t_count >= 4) {
            staged_run_q6k<DM>(P, x, batch, t_begin, t_count, sa, xs[wave], lds_x, red);
            return;
        }
    }
    if (ns > 0) {
        // D - 1 tiles in flight, at most one past the workgroup's last
        const int dsel = min(t_count + 1, DM);
        auto by_depth = [&](auto two_c) {
            if (dsel >= DM) run(two_c, std::integral_constant<int, DM>{});
            else if constexpr (DM > 3) {
                if (dsel == 3) run(two_c, std::integral_constant<int, 3>{});
                else if (dsel == 2) run(two_c, std::integral_constant<int, 2>{});
                else run(two_c, std::integral_constant<int, 1>{});
            } else if constexpr (DM > 2) {
                if (dsel == 2) run(two_c, std::integral_constant<int, 2>{});
                else run(two_c, std::integral_constant<int, 1>{});
            } else {
                run(two_c, std::integral_constant<int, 1>{});
            }
        };
        if (ns == 2)
            by_depth(std_true{});
        else
            by_depth(std_false{});
    }
    else {
        // no super-block: zero partials, same barriers as the others
        const int D = min(t_count, DM);
        for (int t = 0; t < t_count; t += D) {
            for (int j = 0; j < D; ++j)
                red[j][wave][lane] = (fl2){0.f, 0.f};
            lds_barrier();
            const int nt = min(D, t_count - t);
            if ((int)threadIdx.x < nt * 64)
                store_tile(P, t_begin + t + (threadIdx.x >> 6), red[threadIdx.x >> 6], threadIdx.x & 63, batch);
            lds_barrier();
        }
    }
}

int cu_count_cached()
{
    const int v = device_cu_count();
    return v > 0 ? v : 256;
}

template <int T>
hipError_t launch_b(const uint8_t *w, int64_t n, int64_t k, size_t rb, const float *x, int batch, float *y,
                    hipStream_t s)
{
    const int64_t ntiles = (n + 15) / 16;
    const int grid = (int)(ntiles < cu_count_cached() ? ntiles : cu_count_cached());
    if (k <= 256 * 2 * GB_W) {
        MProbs P{};
        P.w[0] = w;
        P.y[0] = y;
        P.n[0] = (int)n;
        P.tile0[1] = (int)ntiles;
        P.np = 1;
        hipLaunchKernelGGL(gemvb1_kernel<T>, dim3(grid), dim3(64 * GB_W), 0, s, x, (int)k, (int64_t)rb, batch,
                           (int)ntiles, grid, P);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(gemvb_kernel<T>, dim3(grid), dim3(64 * GB_W), 0, s, w, (int)n, (int)k, (int64_t)rb, x,
                       batch, y);
    return hipGetLastError();
}

// Problems of one type and k <= 4096 reading one x: one launch over all their
// tiles (empty problems left out of the table).
template <int T>
hipError_t launch_b_multi(int np, const void *const *w, const int64_t *n, int64_t k, size_t rb, const float *x,
                          int batch, float *const *y, hipStream_t s)
{
    for (int i0 = 0; i0 < np;) {
        MProbs P{};
        int c = 0;
        for (; i0 < np && c < MP_MAX; ++i0) {
            if (n[i0] == 0)
                continue;
            P.w[c] = (const uint8_t *)w[i0];
            P.y[c] = y[i0];
            P.n[c] = (int)n[i0];
            P.tile0[c + 1] = P.tile0[c] + (int)((n[i0] + 15) / 16);
            ++c;
        }
        if (c == 0)
            break;
        P.np = c;
        const int ntiles = P.tile0[c];
        const int grid = ntiles < cu_count_cached() ? ntiles : cu_count_cached();
        hipLaunchKernelGGL(gemvb1_kernel<T>, dim3(grid), dim3(64 * GB_W), 0, s, x, (int)k, (int64_t)rb, batch,
                           ntiles, grid, P);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace

bool gemv_mfma_supported(int type, int batch)
{
    return batch >= 2 && batch <= 8 && (type == T_Q4_K || type == T_Q6_K);
}

hipError_t launch_gemv_mfma(int type, const void *w, int64_t n, int64_t k, size_t rb, const float *x, int batch,
                            float *y, hipStream_t s)
{
    const uint8_t *wb = (const uint8_t *)w;
    switch (type) {
    case T_Q4_K: return launch_b<T_Q4_K>(wb, n, k, rb, x, batch, y, s);
    case T_Q6_K: return launch_b<T_Q6_K>(wb, n, k, rb, x, batch, y, s);
    default: return hipErrorInvalidValue;
    }
}

bool gemv_mfma_multi_supported(int type, int batch, int64_t k)
{
    return gemv_mfma_supported(type, batch) && k <= 256 * 2 * GB_W;
}

hipError_t launch_gemv_mfma_multi(int type, int np, const void *const *w, const int64_t *n, int64_t k, size_t rb,
                                  const float *x, int batch, float *const *y, hipStream_t s)
{
    switch (type) {
    case T_Q4_K: return launch_b_multi<T_Q4_K>(np, w, n, k, rb, x, batch, y, s);
    case T_Q6_K: return launch_b_multi<T_Q6_K>(np, w, n, k, rb, x, batch, y, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
