// qmm_gemm.hip -- prefill GEMM Y[m][n] = sum_k X[m][k] W[n][k] with W in
// quantized blocks, X in fp16, Y in fp32, on gfx950 matrix cores.
//
// dotLLM "GPU Inference", Weight Strategy / Future Work: prefill needs a dense
// FP16 contraction; instead of dequantizing a whole projection to an FP16
// scratch buffer and calling a library HGEMM, a fused kernel decodes the
// weights as it goes.  shimmy "Airframe GPU pipeline" prefills prompts in
// 512-token chunks; dequantization happens inline inside each matmul.  Each
// weight enters the contraction as fp16_RNE(w), w being its exact fp32
// dequantized value.
//
// gfx950 design
//   Measured on MI355X: v_mfma_f32_16x16x32_f16 sustains ~2.0-2.2 PFLOP/s;
//   VALU work co-issues with MFMA only up to ~3-4 wave instructions per MFMA
//   before it becomes the limit, and LDS delivers 256 B/clk per CU to
//   conflict-free 128-bit reads and 128 B/clk to stores.  So:
//   - Workgroup tile BM (m) x BN (n) = 256 x 128 with 8 wavefronts stacked
//     along m, each owning 32 x 128 = 2 x 8 MFMA blocks (256 x 112 when that
//     tile count fills the CUs better, 128 x 64 with 8 waves of 16 x 64 when
//     256 x 128 tiles would leave half the CUs idle, 128 x 128 for
//     m <= 128).  Every wave loads only its own X rows (two waves loading the
//     same X lines doubled the L2 traffic and was 2.5x slower); all share the
//     weight tile.  The decode of a weight element is shared by BM rows of X.
//   - Only the weight tile goes through LDS: it is decoded once per workgroup
//     into fp16 [n][k] (16-byte chunks XOR-swizzled within each row so that
//     the 128-bit fragment reads and decode stores are bank-conflict free),
//     double buffered, K step 128.  The decode of tile t+1
//     runs between the MFMAs of tile t; one barrier per K step.
//   - X fragments are loaded straight from global memory into the MFMA
//     operand registers (16 bytes per lane; L2-resident), one K step ahead in
//     a rolling window.  The raw weight bytes of tile t+2 are requested at the
//     start of tile t, right after the first X load of the next tile, so the
//     in-order vmcnt waits for X cover them only a tile later.
//   - Weight decode to fp16: Q8_0 / Q4_0 / Q5_0 codes become exact fp16 integers
//     (byte permute into 0x64xx = 1024 + byte, then subtract the bias) and one
//     v_pk_mul_f16 by d rounds d*q exactly once: d*q is exact in fp32, so this
//     equals fp16_RNE(fp32 w).  Q4_K / Q5_K / Q6_K values are formed in fp32 with one
//     fma (the exact dequantized fp32 value) and packed with v_cvt_pk_f16_f32.
//   - Workgroups are remapped so that each XCD (dispatched round-robin) owns a
//     contiguous run of tiles along n with one X slice, which stays in its L2.
//   - Ragged m / n: loads clamp to the last valid row, stores are masked (row
//     r of Y depends only on row r of X and column j only on row j of W).
//     Ragged K (32-element blocks, K a multiple of 32): 32-wide K sub-steps past K
//     are skipped.
#include "qmm_device.h"
#include "qmm_launch.h"

#include <type_traits>

namespace qmm {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int GKT = 128;            // K step
#ifndef QMM_GEMM_SCHED
#define QMM_GEMM_SCHED 1
#endif
constexpr bool SCHED = QMM_GEMM_SCHED;   // explicit MFMA / VALU interleave

// Unaligned byte runs: NDW dwords starting at an even byte address p are
// fetched as the NDW aligned dwords at or below p plus a 2-byte tail, reading
// only bytes in [p - 2, p + 4*NDW); the realignment (v_alignbyte_b32 by
// sh = p % 4, 0 or 2) happens at decode time, so the loads are not waited for
// where they are issued.  When p is 4-byte aligned the tail load reads the
// run's last two bytes instead (unused): it is unconditional -- a load under a
// branch is waited for at once -- and never touches memory past the run.
template <int NDW>
struct URun {
    uint32_t d[NDW + 1];
};

template <int NDW>
__device__ __forceinline__ uint32_t gload_run(const uint8_t *p, URun<NDW> &r)
{
    // pointer arithmetic, not an integer round trip: the pointer keeps its
    // global address space and the loads stay global_load, not flat_load
    // (which would also count against the LDS wait counter)
    const uint32_t sh = (uint32_t)((uintptr_t)p & 3u);
    const uint32_t *q = (const uint32_t *)(p - sh);
#pragma unroll
    for (int i = 0; i < NDW; ++i)
        r.d[i] = q[i];
    r.d[NDW] = *(const uint16_t *)((const uint8_t *)(q + NDW) - (2u - sh));
    return sh;
}

template <int NDW>
__device__ __forceinline__ void realign(const URun<NDW> &r, uint32_t sh, uint32_t *out)
{
#pragma unroll
    for (int i = 0; i < NDW; ++i)
        out[i] = align_bytes(r.d[i + 1], r.d[i], sh);
}

// ------------------------------------------------------- decode units --
// A unit is 32 weights of one row inside K step t, quarter q (0..3):
//   Q8_0 / Q4_0 / Q5_0  block 4 t + q of the row (one run of 32 elements at
//                32 q; Q5_0 reads its high-bit word with the codes);
//   Q4_K         16 code bytes of super-block t / 2: low nibbles are 16
//                elements of sub-block 2p, high nibbles the same 16 of
//                sub-block 2p + 1 (p = 2 (t % 2) + q / 2);
//   Q5_K         as Q4_K, plus the 16 qh bytes of the same elements l;
//   Q6_K         16 ql bytes and 16 qh bytes of super-block t / 2, half
//                h = t % 2: 16 elements (l = 16 (q % 2) + i) of each of the
//                groups g = q / 2 (low nibble) and g + 2 (high nibble).
template <int T> struct WRaw;
template <> struct WRaw<T_Q8_0> { uint32_t d; URun<8> c; uint32_t sh; };
template <> struct WRaw<T_Q4_0> { uint32_t d; URun<4> c; uint32_t sh; };
template <> struct WRaw<T_Q4_K> { u32x4 hd; u32x4 c; };
template <> struct WRaw<T_Q6_K> { URun<4> ql; URun<4> qh; uint32_t sc; uint32_t d; uint32_t sh; };
template <> struct WRaw<T_Q5_0> { uint32_t d; URun<5> c; uint32_t sh; };   // c: high-bit word, 4 code dwords
template <> struct WRaw<T_Q5_K> { u32x4 hd; u32x4 c; u32x4 h; };

template <int T>
__device__ __forceinline__ void load_unit(const uint8_t *row, int t, int q, WRaw<T> &r)
{
    if constexpr (T == T_Q8_0) {
        const uint8_t *blk = row + (int64_t)(4 * t + q) * 34;
        r.d = *(const uint16_t *)blk;
        r.sh = gload_run<8>(blk + 2, r.c);
    } else if constexpr (T == T_Q4_0) {
        const uint8_t *blk = row + (int64_t)(4 * t + q) * 18;
        r.d = *(const uint16_t *)blk;
        r.sh = gload_run<4>(blk + 2, r.c);
    } else if constexpr (T == T_Q5_0) {
        const uint8_t *blk = row + (int64_t)(4 * t + q) * 22;
        r.d = *(const uint16_t *)blk;
        r.sh = gload_run<5>(blk + 2, r.c);
    } else if constexpr (T == T_Q5_K) {
        const uint8_t *blk = row + (int64_t)(t >> 1) * 176;    // 16-byte aligned
        r.hd = *(const u32x4 *)blk;
        r.h = *(const u32x4 *)(blk + 16 + 16 * (q & 1));      // qh of the unit's 16 elements l
        r.c = *(const u32x4 *)(blk + 48 + 64 * (t & 1) + 16 * q);
    } else if constexpr (T == T_Q4_K) {
        const uint8_t *blk = row + (int64_t)(t >> 1) * 144;    // 16-byte aligned
        r.hd = *(const u32x4 *)blk;
        r.c = *(const u32x4 *)(blk + 16 + 64 * (t & 1) + 16 * q);
    } else {
        const uint8_t *blk = row + (int64_t)(t >> 1) * 210;
        const int h = t & 1, gp = q >> 1, lq = q & 1;
        // both runs start at the same offset mod 4 as the block
        r.sh = gload_run<4>(blk + 64 * h + 32 * gp + 16 * lq, r.ql);
        gload_run<4>(blk + 128 + 32 * h + 16 * lq, r.qh);
        const uint32_t s0 = blk[192 + 8 * h + 2 * gp + lq];        // scale of group g = gp
        const uint32_t s1 = blk[192 + 8 * h + 2 * gp + 4 + lq];    // scale of group g = gp + 2
        r.sc = s0 | (s1 << 8);
        r.d = *(const uint16_t *)(blk + 208);
    }
}

__device__ __forceinline__ uint32_t h2_bits(half2v v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ half2v bits_h2(uint32_t v) { return __builtin_bit_cast(half2v, v); }

// fp16_RNE of two fp32 values, packed (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_rne(float a, float b)
{
    return h2_bits(__builtin_convertvector((float2v){a, b}, half2v));
}

// Bytes 2j and 2j+1 of c (j = 0, 1) as the fp16 values 1024 + byte.
__device__ __forceinline__ uint32_t bytes_1024(uint32_t c, int j)
{
    return __builtin_amdgcn_perm(0x64646464u, c, j ? 0x04030402u : 0x04010400u);
}

// Decode unit (t, q) to fp16 and store its runs into weight tile row ws
// (tile-local element offsets).
// Keep every loaded dword live up to the decode: a dword the decode does not
// need (e.g. the third Q4_K scale dword in even K steps) would otherwise be
// reused as a temporary while its load is in flight, and the write-after-write
// forces a wait for all outstanding loads.
template <int T>
__device__ __forceinline__ void keep_raw(const WRaw<T> &r)
{
    constexpr int N = sizeof(WRaw<T>) / 4;
    const uint32_t *v = (const uint32_t *)&r;
#pragma unroll
    for (int i = 0; i < N; ++i)
        asm volatile("" : : "v"(v[i]));
}

// Weight tile layout in LDS: row r holds the 128 K-step weights of output
// column r as fp16; its 16-byte chunk c (weights 8c .. 8c+7) is stored at
// chunk c ^ ((c >> 1) & 6) ^ (r % 16) of the row (no padding).  Measured on
// gfx950 (LDS bank-conflict counters): a 16-byte read serves 16 lanes per
// cycle from 64 banks, in lane quads grouped by half-wave and by the parity
// of the quad index, and a 16-byte store serves 8 consecutive lanes from 32
// banks.  Under this swizzle both the MFMA fragment reads (lane l: row l % 16,
// chunk 4 s + l / 16) and the decode stores (lane l: row l / 4, the chunk of
// quarter l % 4 and part i) hit distinct banks; a row pitch padded by 8 halves
// conflicted 2-way on the reads and 2- to 4-way on the stores.
__device__ __forceinline__ int tile_off(int r, int c)
{
    return r * GKT + 8 * ((c ^ ((c >> 1) & 6) ^ r) & 15);
}

// The swizzle is linear over GF(2): for a chunk c ^ d whose set bits do not
// meet those of c, tile_off(r, c ^ d) = tile_off(r, c) ^ tile_xor(d).
__host__ __device__ constexpr int tile_xor(int d)
{
    return 8 * ((d ^ ((d >> 1) & 6)) & 15);
}

// Decoder of one unit, in four parts of 8 consecutive weights (one 16-byte
// store each), so that the decode can be spread between the MFMAs of the four
// 32-wide sub-steps of a K step.  setup() prepares the scales; part(i, dst)
// stores its 8 fp16 weights at dst.  chunk(q, i) = chunk(q, 0) ^ delta(i):
// the row chunk (8 weights) that part i of quarter q covers (delta(i) shares
// no set bit with chunk(q, 0)).
template <int T> struct Dec;

__device__ __forceinline__ uint32_t dw(const u32x4 &v, int k)
{
    return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

__device__ __forceinline__ void st128(_Float16 *dst, const uint32_t (&o)[4])
{
    *(u32x4 *)dst = u32x4{o[0], o[1], o[2], o[3]};
}

template <> struct Dec<T_Q8_0> {
    half2v d2;
    static constexpr int delta(int i) { return i; }
    static __device__ __forceinline__ int chunk(int q, int i) { return 4 * q + delta(i); }
    __device__ __forceinline__ void setup(const WRaw<T_Q8_0> &r, int, int)
    {
        keep_raw(r);
        d2 = bits_h2(r.d | (r.d << 16));
    }
    __device__ __forceinline__ void part(const WRaw<T_Q8_0> &r, int i, _Float16 *dst) const
    {
        const half2v bias = {(_Float16)1152.f, (_Float16)1152.f};
        uint32_t o[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t c = align_bytes(r.c.d[2 * i + h + 1], r.c.d[2 * i + h], r.sh) ^ 0x80808080u;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                o[2 * h + j] = h2_bits((bits_h2(bytes_1024(c, j)) - bias) * d2);   // q exact, one rounding
        }
        st128(dst, o);
    }
};

// Q4_0 / Q5_0 part i: the low (i even: elements 8 (i / 2) + 0..7) or high
// (i odd: elements 16 + 8 (i / 2) + 0..7) nibbles of code dwords 2 (i / 2) and
// 2 (i / 2) + 1, so that each code dword is needed by two consecutive parts.
template <> struct Dec<T_Q4_0> {
    half2v d2;
    static constexpr int delta(int i) { return (i >> 1) + 2 * (i & 1); }
    static __device__ __forceinline__ int chunk(int q, int i) { return 4 * q + delta(i); }
    __device__ __forceinline__ void setup(const WRaw<T_Q4_0> &r, int, int)
    {
        keep_raw(r);
        d2 = bits_h2(r.d | (r.d << 16));
    }
    __device__ __forceinline__ void part(const WRaw<T_Q4_0> &r, int i, _Float16 *dst) const
    {
        const half2v bias = {(_Float16)1032.f, (_Float16)1032.f};
        uint32_t o[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = 2 * (i >> 1) + h;
            const uint32_t c = align_bytes(r.c.d[k + 1], r.c.d[k], r.sh);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint32_t b = bytes_1024(c, j);                   // [c, 0x64, c', 0x64]
                const uint32_t v = (i & 1) == 0 ? (b & 0x640f640fu) : (((b >> 4) & 0x000f000fu) | 0x64006400u);
                o[2 * h + j] = h2_bits((bits_h2(v) - bias) * d2);
            }
        }
        st128(dst, o);
    }
};

// Q4_K / Q5_K part i: the low (i even, sub-block 2p) or high (i odd, sub-block
// 2p + 1) nibbles of code dwords 2 (i / 2) and 2 (i / 2) + 1 of the unit.
template <> struct Dec<T_Q4_K> {
    float dsc0, dm0, dsc1, dm1;
    static constexpr int delta(int i) { return (i >> 1) + 4 * (i & 1); }
    static __device__ __forceinline__ int chunk(int q, int i) { return 8 * (q >> 1) + 2 * (q & 1) + delta(i); }
    __device__ __forceinline__ void setup(const WRaw<T_Q4_K> &r, int t, int q)
    {
        keep_raw(r);
        const int p = 2 * (t & 1) + (q >> 1);
        uint32_t sc0, m0, sc1, m1;
        q4k_scale_min(r.hd.y, r.hd.z, r.hd.w, 2 * p, sc0, m0);
        q4k_scale_min(r.hd.y, r.hd.z, r.hd.w, 2 * p + 1, sc1, m1);
        const float d = h2f(r.hd.x & 0xffffu), dmin = h2f(r.hd.x >> 16);
        // high nibbles convert as 16 q: the 1/16 goes into their scale (exact,
        // so the fma still yields the exact fp32 value, rounded once)
        dsc0 = d * (float)sc0;
        dm0 = dmin * (float)m0;
        dsc1 = d * (float)sc1 * 0.0625f;
        dm1 = dmin * (float)m1;
    }
    __device__ __forceinline__ void part(const WRaw<T_Q4_K> &r, int i, _Float16 *dst) const
    {
        const bool lo = (i & 1) == 0;
        const float ds = lo ? dsc0 : dsc1, dm = lo ? dm0 : dm1;
        uint32_t o[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t c = dw(r.c, 2 * (i >> 1) + h);
            const uint32_t v = opaque(c & (lo ? 0x0f0f0f0fu : 0xf0f0f0f0u));
            o[2 * h] = pack_rne(__builtin_fmaf(ub0(v), ds, -dm), __builtin_fmaf(ub1(v), ds, -dm));
            o[2 * h + 1] = pack_rne(__builtin_fmaf(ub2(v), ds, -dm), __builtin_fmaf(ub3(v), ds, -dm));
        }
        st128(dst, o);
    }
};

template <> struct Dec<T_Q5_0> {
    half2v d2;
    static constexpr int delta(int i) { return Dec<T_Q4_0>::delta(i); }
    static __device__ __forceinline__ int chunk(int q, int i) { return 4 * q + delta(i); }
    __device__ __forceinline__ void setup(const WRaw<T_Q5_0> &r, int, int)
    {
        keep_raw(r);
        d2 = bits_h2(r.d | (r.d << 16));
    }
    __device__ __forceinline__ void part(const WRaw<T_Q5_0> &r, int i, _Float16 *dst) const
    {
        const half2v bias = {(_Float16)1040.f, (_Float16)1040.f};
        const uint32_t hb = align_bytes(r.c.d[1], r.c.d[0], r.sh);
        uint32_t o[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = 2 * (i >> 1) + h;
            const uint32_t c = align_bytes(r.c.d[k + 2], r.c.d[k + 1], r.sh);
            // element e of the block takes bit e of the high-bit word
            const uint32_t q5 = (i & 1) == 0 ? (c & 0x0f0f0f0fu) | bits_to_byte_bit4(hb >> (4 * k))
                                      : ((c >> 4) & 0x0f0f0f0fu) | bits_to_byte_bit4(hb >> (16 + 4 * k));
#pragma unroll
            for (int j = 0; j < 2; ++j)   // 1024 + q exactly, minus 1040: q - 16, then one rounding of d (q - 16)
                o[2 * h + j] = h2_bits((bits_h2(bytes_1024(q5, j)) - bias) * d2);
        }
        st128(dst, o);
    }
};

template <> struct Dec<T_Q5_K> {
    float dsc0, dm0, dsc1, dm1;
    uint32_t hs;
    static constexpr int delta(int i) { return Dec<T_Q4_K>::delta(i); }
    static __device__ __forceinline__ int chunk(int q, int i) { return Dec<T_Q4_K>::chunk(q, i); }
    __device__ __forceinline__ void setup(const WRaw<T_Q5_K> &r, int t, int q)
    {
        keep_raw(r);
        const int p = 2 * (t & 1) + (q >> 1);
        uint32_t sc0, m0, sc1, m1;
        q4k_scale_min(r.hd.y, r.hd.z, r.hd.w, 2 * p, sc0, m0);
        q4k_scale_min(r.hd.y, r.hd.z, r.hd.w, 2 * p + 1, sc1, m1);
        const float d = h2f(r.hd.x & 0xffffu), dmin = h2f(r.hd.x >> 16);
        dsc0 = d * (float)sc0;
        dm0 = dmin * (float)m0;
        dsc1 = d * (float)sc1;
        dm1 = dmin * (float)m1;
        hs = 2u * (uint32_t)p;      // qh bit of sub-block 2p; 2p + 1 for the high nibbles
    }
    __device__ __forceinline__ void part(const WRaw<T_Q5_K> &r, int i, _Float16 *dst) const
    {
        const bool lo = (i & 1) == 0;
        const float ds = lo ? dsc0 : dsc1, dm = lo ? dm0 : dm1;
        uint32_t o[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = 2 * (i >> 1) + h;
            const uint32_t c = dw(r.c, k), hq = dw(r.h, k);
            const uint32_t v = lo ? opaque((c & 0x0f0f0f0fu) | (((hq >> hs) & 0x01010101u) << 4))
                                     : opaque(((c >> 4) & 0x0f0f0f0fu) | (((hq >> (hs + 1u)) & 0x01010101u) << 4));
            o[2 * h] = pack_rne(__builtin_fmaf(ub0(v), ds, -dm), __builtin_fmaf(ub1(v), ds, -dm));
            o[2 * h + 1] = pack_rne(__builtin_fmaf(ub2(v), ds, -dm), __builtin_fmaf(ub3(v), ds, -dm));
        }
        st128(dst, o);
    }
};

// Q6_K part i: group g = q / 2 (low nibbles, i even) or g + 2 (high nibbles,
// i odd) of ql / qh dwords 2 (i / 2) and 2 (i / 2) + 1 of the unit.
template <> struct Dec<T_Q6_K> {
    float ds0, nb0, ds1, nb1;
    uint32_t hs0;
    static constexpr int delta(int i) { return (i >> 1) + 8 * (i & 1); }
    static __device__ __forceinline__ int chunk(int q, int i) { return 4 * (q >> 1) + 2 * (q & 1) + delta(i); }
    __device__ __forceinline__ void setup(const WRaw<T_Q6_K> &r, int, int q)
    {
        keep_raw(r);
        const int gp = q >> 1;
        const float d = h2f(r.d);
        ds0 = d * (float)(int8_t)(r.sc & 0xffu);          // group gp
        ds1 = d * (float)(int8_t)((r.sc >> 8) & 0xffu);   // group gp + 2
        nb0 = -32.f * ds0;                                // fma(q, ds, -32 ds) = ds (q - 32), rounded once
        nb1 = -32.f * ds1;
        hs0 = 2u * (uint32_t)gp;
    }
    __device__ __forceinline__ void part(const WRaw<T_Q6_K> &r, int i, _Float16 *dst) const
    {
        const bool lo = (i & 1) == 0;
        const float ds = lo ? ds0 : ds1, nb = lo ? nb0 : nb1;
        uint32_t o[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = 2 * (i >> 1) + h;
            const uint32_t l = align_bytes(r.ql.d[k + 1], r.ql.d[k], r.sh);
            const uint32_t hb = align_bytes(r.qh.d[k + 1], r.qh.d[k], r.sh);
            const uint32_t v = lo ? opaque((l & 0x0f0f0f0fu) | (((hb >> hs0) & 0x03030303u) << 4))
                                     : opaque(((l >> 4) & 0x0f0f0f0fu) | (((hb >> (hs0 + 4u)) & 0x03030303u) << 4));
            o[2 * h] = pack_rne(__builtin_fmaf(ub0(v), ds, nb), __builtin_fmaf(ub1(v), ds, nb));
            o[2 * h + 1] = pack_rne(__builtin_fmaf(ub2(v), ds, nb), __builtin_fmaf(ub3(v), ds, nb));
        }
        st128(dst, o);
    }
};

// ---------------------------------------------------------------- kernel --
// FM x FN MFMA blocks per wave, WM x WN waves; BM = 16 FM WM, BN = 16 FN WN.
template <int T, int FM, int FN, int WM, int WN, int XD>
struct GemmCfg {
    static constexpr int MW = 16 * FM, NW = 16 * FN;
    static constexpr int BM = MW * WM, BN = NW * WN;
    static constexpr int NT = 64 * WM * WN;
    static constexpr int UNITS = 4 * BN;              // decode units per K step
    static constexpr int UPT = (UNITS + NT - 1) / NT; // per thread
    // units split evenly over the threads, or (e.g. 112-column tiles) the
    // last wavefronts have none in the last slot
    static constexpr bool EVEN = UNITS % NT == 0;
    static_assert(EVEN || (UNITS % 64 == 0 && UNITS > NT * (UPT - 1)), "decode units per wavefront");
    static constexpr int LDS_HALVES = 2 * BN * GKT;
};

template <int T, int FM, int FN, int WM, int WN, int XD>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_kernel(const uint8_t *__restrict__ w, int n, int k, int64_t rb, const uint16_t *__restrict__ x, int m,
            float *__restrict__ y, int nnt, int tiles, int ksplit, int remap)
{
    using C = GemmCfg<T, FM, FN, WM, WN, XD>;
    __shared__ __attribute__((aligned(16))) _Float16 Ws[C::LDS_HALVES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    // Workgroup b = kc * tiles + tile: K chunk kc of the tile (split K adds
    // the chunks into a zeroed Y).  XCD-aware tile order: workgroup b runs on
    // XCD b % 8; give each XCD a contiguous range of tile ids (m-major), i.e.
    // one X slice and a run of n.
    const int kc = (int)blockIdx.x / tiles;
    int b = (int)blockIdx.x - kc * tiles;
    if (remap) {
        const int per = tiles >> 3;
        b = (b & 7) * per + (b >> 3);
    }
    const int mt = b / nnt, nt = b - mt * nnt;
    const int m0 = mt * C::BM, n0 = nt * C::BN;
    const int nkt_all = (k + GKT - 1) / GKT;
    const int chunk = (nkt_all + ksplit - 1) / ksplit;
    const int kt0 = kc * chunk;
    const int nkt = min(kt0 + chunk, nkt_all);   // end of this chunk's steps

    // ---- X fragment addressing (A operand: row lane%16, k 8*(lane/16)..+7)
    const uint16_t *xrow[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int r = min(m0 + wm * C::MW + 16 * i + (lane & 15), m - 1);
        xrow[i] = x + (int64_t)r * k + 8 * (lane >> 4);
    }
    // rolling window of XD sub-steps: sub-step (t, s) lives in slot (4t + s) % XD
    static_assert(XD == 2 || XD == 4, "X prefetch distance");
    half8 xa[XD][FM];
    auto load_x = [&](int t, int s) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
            xa[s % XD][i] = *(const half8 *)(xrow[i] + GKT * t + 32 * s);
    };

    // ---- weight units of this thread
    const uint8_t *wrow[C::UPT];
    int uq[C::UPT], woff[C::UPT];
#pragma unroll
    for (int u = 0; u < C::UPT; ++u) {
        const int id = tid + C::NT * u;
        const int col = id >> 2;
        uq[u] = id & 3;
        wrow[u] = w + (int64_t)min(n0 + col, n - 1) * rb;
        woff[u] = tile_off(col, Dec<T>::chunk(uq[u], 0));   // part i: ^ tile_xor(delta(i))
    }
    // slot u of this thread holds a unit (wave-uniform: units come in whole wavefronts)
    auto has = [&](int u) __attribute__((always_inline)) {
        return C::EVEN || u < C::UPT - 1 || __builtin_amdgcn_readfirstlane(tid) + C::NT * u < C::UNITS;
    };
    WRaw<T> wr[2][C::UPT];
    // (full: step t lies wholly inside K, which always holds for 256-element
    // super-blocks since K is then a multiple of 256)
    auto load_w = [&](int par, int t, bool full) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < C::UPT; ++u)
            if (has(u) && (full || Fmt<T>::BE == 256 || 4 * t + uq[u] < (k >> 5)))
                load_unit<T>(wrow[u], t, uq[u], wr[par][u]);
    };
    // decode of step t in four parts (part i between the MFMAs of sub-step i)
    Dec<T> dec[C::UPT];
    auto decode_w = [&](int par, int t, _Float16 *dst, bool full, int i) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < C::UPT; ++u)
            if (has(u) && (full || Fmt<T>::BE == 256 || 4 * t + uq[u] < (k >> 5))) {
                if (i == 0)
                    dec[u].setup(wr[par][u], t, uq[u]);
                int wo = woff[u];
                asm volatile("" : "+v"(wo));   // keep the XOR in the loop: hoisted, the 4 offsets pin 4 VGPRs
                dec[u].part(wr[par][u], i, dst + (wo ^ tile_xor(Dec<T>::delta(i))));
            }
    };

    float4v acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = float4v{0.f, 0.f, 0.f, 0.f};

    // B fragment of sub-step s, block j: row wn NW + 16 j + lane % 16, chunk
    // 4 s + lane / 16 (the swizzle depends on the row only through lane % 16)
    const int bro = tile_off(wn * C::NW + (lane & 15), lane >> 4);   // sub-step s: ^ tile_xor(4 s)

    // One K step t with compile-time buffer parity PAR (= t % 2).  FULL: t is
    // not among the last three steps, so every step, load and decode of the
    // body is in range and the body has no branches (a branch around a load
    // makes the compiler wait for it at once).
    auto tile = [&](auto par_c, auto full_c, int t) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par_c)::value;
        constexpr bool FULL = decltype(full_c)::value;
        const _Float16 *wcur = Ws + PAR * C::BN * GKT;
        _Float16 *wnext = Ws + (1 - PAR) * C::BN * GKT;
        const bool nx = FULL || t + 1 < nkt;
        // weight fragments of step s + 1 are read from LDS while the MFMAs of
        // step s run (two register sets)
        half8 bf[2][FN];
        auto read_b = [&](int s, half8 *dst) __attribute__((always_inline)) {
            int b = bro;
            asm volatile("" : "+v"(b));        // as for the decode stores
            const _Float16 *src = wcur + (b ^ tile_xor(4 * s));
#pragma unroll
            for (int j = 0; j < FN; ++j)
                dst[j] = *(const half8 *)(src + 16 * j * GKT);
        };
        if (FULL || GKT * t < k)
            read_b(0, bf[0]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s < 3 && (FULL || GKT * t + 32 * (s + 1) < k))
                read_b(s + 1, bf[(s + 1) & 1]);
            if (FULL || GKT * t + 32 * s < k) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[s % XD][i], bf[s & 1][j], acc[i][j], 0, 0, 0);
            }
            // FULL: a load past the last step re-reads the last step instead
            // (in range, never used), so the body stays free of branches
            {   // X of sub-step s + XD into the slot just consumed
                const int tn = t + (s + XD) / 4, sn = (s + XD) % 4;
                if (FULL)
                    load_x(min(tn, nkt - 1), sn);
                else if (tn < nkt && GKT * tn + 32 * sn < k)
                    load_x(tn, sn);
            }
            if (s == 0 && (FULL || t + 2 < nkt))
                load_w(PAR, FULL ? min(t + 2, nkt - 1) : t + 2, FULL);
            if (nx)
                decode_w(1 - PAR, FULL ? min(t + 1, nkt - 1) : t + 1, wnext, FULL, s);
            if constexpr (FULL && SCHED) {
                // interleave: the next sub-step's LDS reads and the X loads
                // first, then each MFMA followed by ~2 VALU instructions of
                // the decode, then its LDS writes
                __builtin_amdgcn_sched_group_barrier(0x100, FN, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, FM, 0);
#pragma unroll
                for (int g = 0; g < FM * FN; ++g) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x200, C::UPT, 0);
            }
        }
        __syncthreads();
    };

    // prologue: X of the first step, raw weights of the first two, decode the first
#pragma unroll
    for (int s = 0; s < XD; ++s)
        if (GKT * kt0 + 32 * s < k)
            load_x(kt0, s);
    load_w(0, kt0, false);
    if (kt0 + 1 < nkt)
        load_w(1, kt0 + 1, false);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        decode_w(0, kt0, Ws, false, i);
    __syncthreads();

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using BT = std::integral_constant<bool, true>;
    using BF = std::integral_constant<bool, false>;
    // A step is FULL when it and every step it loads or decodes lie wholly
    // inside K, loads past the last step being clamped to it.  When K is a
    // multiple of 128 (always for 256-element super-blocks) every step is;
    // otherwise only the last one is partial and the last pairs take the
    // general path.
    const bool whole = (k % GKT) == 0 || nkt < nkt_all;
    const int full_pairs_end = whole ? nkt - 1 : nkt - 4;
    int t = kt0;
    for (; t < full_pairs_end; t += 2) {
        tile(I0{}, BT{}, t);
        tile(I1{}, BT{}, t + 1);
    }
    if (whole && t < nkt) {   // odd number of steps: the last one alone
        tile(I0{}, BT{}, t);
        ++t;
    }
    while (t < nkt) {
        tile(I0{}, BF{}, t);
        if (++t < nkt)
            tile(I1{}, BF{}, t);
        ++t;
    }

    // C fragment: lane holds rows 4*(lane/16) + 0..3 (of X), column lane%16 (of W)
    const int cr = 4 * (lane >> 4), cc = lane & 15;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int gn = n0 + wn * C::NW + 16 * j + cc;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int gm = m0 + wm * C::MW + 16 * i + cr + r;
                if (gm < m && gn < n) {
                    if (ksplit > 1)
                        unsafeAtomicAdd(y + (int64_t)gm * n + gn, acc[i][j][r]);   // global_atomic_add_f32
                    else
                        y[(int64_t)gm * n + gn] = acc[i][j][r];
                }
            }
        }
}

// Compute units of the current device (256, the MI355X count, if the runtime
// cannot tell: only the tile choice depends on it).
static int cu_count()
{
    const int v = device_cu_count();
    return v > 0 ? v : 256;
}

hipError_t launch_fill_zero(float *p, int64_t count, hipStream_t s);

template <int BM, int BN>
static int64_t tile_count(int64_t m, int64_t n)
{
    return ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
}

template <int T, int FM, int FN, int WM, int WN, int XD>
hipError_t launch_cfg(const uint8_t *w, int64_t n, int64_t k, size_t rb, const uint16_t *x, int64_t m, float *y,
                      hipStream_t s)
{
    using C = GemmCfg<T, FM, FN, WM, WN, XD>;
    const int nmt = (int)((m + C::BM - 1) / C::BM), nnt = (int)((n + C::BN - 1) / C::BN);
    const int tiles = nmt * nnt;
    const int remap = (tiles % 8 == 0) ? 1 : 0;
    // Split K when the tiles alone leave most CUs idle (e.g. 512 x 4096: 64
    // tiles): up to 4 chunks of at least 8 K steps, added with fp32 atomics
    // into a zeroed Y (the order of the additions is not fixed).
    const int nkt = (int)((k + GKT - 1) / GKT);
    int ksplit = 1;
    while (ksplit < 4 && tiles * ksplit * 2 <= cu_count() && nkt / (ksplit * 2) >= 8)
        ksplit *= 2;
    if (ksplit > 1) {
        const hipError_t e = launch_fill_zero(y, m * n, s);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((gemm_kernel<T, FM, FN, WM, WN, XD>), dim3((unsigned)(tiles * ksplit)), dim3(C::NT), 0, s, w,
                       (int)n, (int)k, (int64_t)rb, x, (int)m, y, nnt, tiles, ksplit, remap);
    return hipGetLastError();
}

template <int T>
hipError_t launch_gemm_t(const uint8_t *w, int64_t n, int64_t k, size_t rb, const uint16_t *x, int64_t m,
                         float *y, hipStream_t s)
{
    // Wavefronts stacked along m, each 16 FM x 16 FN: every wave reads its own
    // X rows (no wave loads X another wave loads), all share the weight tile.
    // 256 x 128 tiles (8 waves) when they fill at least half the CUs; else
    // 128 x 64 tiles before splitting K: on 512 x 4096 these give 256 tiles
    // and ran 25% faster than 64 tiles split 4 ways, whose fp32 atomics and
    // zero fill cost more than the smaller tiles' extra decode.  Those tiles
    // use 8 waves of 16 x 64 (two per SIMD, the first four decode the weight
    // tile): measured 3-10% faster than 4 waves of 32 x 64.
    // Of 128- and 112-column tiles, 112 when they keep clearly more CUs busy
    // in the last round (512 x 14336: 224 tiles of 128 leave 32 of 256 CUs
    // idle, 256 tiles of 112 none; measured 4-5% faster).
    if (m <= 128)
        return launch_cfg<T, 1, 8, 8, 1, 4>(w, n, k, rb, x, m, y, s);   // 128 x 128
    const int64_t cus = cu_count();
    const int64_t t128 = tile_count<256, 128>(m, n);
    if (2 * t128 > cus) {
        const int64_t t112 = tile_count<256, 112>(m, n);
        // busy fraction of the last round, compared as t / rounds (cross-multiplied)
        const int64_t r128 = (t128 + cus - 1) / cus, r112 = (t112 + cus - 1) / cus;
        if (100 * t112 * r128 > 105 * t128 * r112)
            return launch_cfg<T, 2, 7, 8, 1, 4>(w, n, k, rb, x, m, y, s);   // 256 x 112
        // Q6_K: X two sub-steps ahead, not four (16 VGPRs; four spill)
        return launch_cfg<T, 2, 8, 8, 1, T == T_Q6_K ? 2 : 4>(w, n, k, rb, x, m, y, s);   // 256 x 128
    }
    return launch_cfg<T, 1, 4, 8, 1, 4>(w, n, k, rb, x, m, y, s);       // 128 x 64, 8 waves
}

hipError_t launch_gemm(int type, const void *w, int64_t n, int64_t k, size_t rb, const uint16_t *x, int64_t m,
                       float *y, hipStream_t s)
{
    const uint8_t *wb = (const uint8_t *)w;
    switch (type) {
    case T_Q4_0: return launch_gemm_t<T_Q4_0>(wb, n, k, rb, x, m, y, s);
    case T_Q8_0: return launch_gemm_t<T_Q8_0>(wb, n, k, rb, x, m, y, s);
    case T_Q4_K: return launch_gemm_t<T_Q4_K>(wb, n, k, rb, x, m, y, s);
    case T_Q6_K: return launch_gemm_t<T_Q6_K>(wb, n, k, rb, x, m, y, s);
    case T_Q5_0: return launch_gemm_t<T_Q5_0>(wb, n, k, rb, x, m, y, s);
    case T_Q5_K: return launch_gemm_t<T_Q5_K>(wb, n, k, rb, x, m, y, s);
    default: return hipErrorInvalidValue;
    }
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
