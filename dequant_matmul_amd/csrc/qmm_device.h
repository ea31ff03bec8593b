// qmm_device.h -- device-side helpers shared by the gfx950 kernels of libqmm.
//
// Block formats decoded here (shimmy "Architecture", Quantization table;
// dotLLM "GPU Inference", Quantization on GPU table):
//   Q4_0  32 el / 18 B : fp16 d | 16 B codes (el i<16 low nibble of byte i,
//                        el i>=16 high nibble of byte i-16)   w = d (q - 8)
//   Q8_0  32 el / 34 B : fp16 d | 32 int8                      w = d q
//   Q4_K 256 el / 144 B: fp16 d | fp16 dmin | 12 B 6-bit scale/min |
//                        128 B codes; w = d sc_j q - dmin m_j, j = e / 32
//   Q6_K 256 el / 210 B: 128 B ql | 64 B qh | 16 int8 scales | fp16 d;
//                        w = d scale[e/16] (q - 32)
//   Q5_0  32 el / 22 B : fp16 d | 32 high bits | 16 B codes as Q4_0;
//                        w = d (q - 16)
//   Q5_K 256 el / 176 B: as Q4_K with 32 B qh between the scales and the
//                        codes (bit j of qh[l]: bit 4 of element (j, l))
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

enum : int { T_Q4_0 = 0, T_Q8_0 = 1, T_Q4_K = 2, T_Q6_K = 3, T_Q5_0 = 4, T_Q5_K = 5 };

// Native 128-bit vectors.  (HIP's uint4 / float4 are structs whose copies
// lower to memcpy, which can keep arrays of them in scratch memory.)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));

template <int T> struct Fmt;
template <> struct Fmt<T_Q4_0> { static constexpr int BE = 32, BB = 18; };
template <> struct Fmt<T_Q8_0> { static constexpr int BE = 32, BB = 34; };
template <> struct Fmt<T_Q4_K> { static constexpr int BE = 256, BB = 144; };
template <> struct Fmt<T_Q6_K> { static constexpr int BE = 256, BB = 210; };
template <> struct Fmt<T_Q5_0> { static constexpr int BE = 32, BB = 22; };
template <> struct Fmt<T_Q5_K> { static constexpr int BE = 256, BB = 176; };

// IEEE binary16 bits -> fp32 (exact; v_cvt_f32_f16).
__device__ __forceinline__ float h2f(uint32_t bits16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// Hide a value from the optimizer so that a whole-dword mask stays one
// v_and_b32 followed by per-byte converts (v_cvt_f32_ubyteN), instead of being
// folded into one bit-field extract per element.
__device__ __forceinline__ uint32_t opaque(uint32_t v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// Bytes [s, s+4) of the 8-byte value (hi:lo), s in 0..3 (v_alignbyte_b32).
__device__ __forceinline__ uint32_t align_bytes(uint32_t hi, uint32_t lo, uint32_t s)
{
    return __builtin_amdgcn_alignbyte(hi, lo, s);
}

__device__ __forceinline__ float ub0(uint32_t v) { return (float)(v & 0xffu); }
__device__ __forceinline__ float ub1(uint32_t v) { return (float)((v >> 8) & 0xffu); }
__device__ __forceinline__ float ub2(uint32_t v) { return (float)((v >> 16) & 0xffu); }
__device__ __forceinline__ float ub3(uint32_t v) { return (float)(v >> 24); }
__device__ __forceinline__ float sb0(uint32_t v) { return (float)(int8_t)(v); }
__device__ __forceinline__ float sb1(uint32_t v) { return (float)(int8_t)(v >> 8); }
__device__ __forceinline__ float sb2(uint32_t v) { return (float)(int8_t)(v >> 16); }
__device__ __forceinline__ float sb3(uint32_t v) { return (float)(int8_t)(v >> 24); }

// Bits 0..3 of h moved to bit 4 of bytes 0..3 (the four partial products of
// the multiply land on disjoint bit ranges, so nothing carries): the high
// code bit of four consecutive Q5_0 elements.
__device__ __forceinline__ uint32_t bits_to_byte_bit4(uint32_t h)
{
    return ((h & 15u) * 0x02040810u) & 0x10101010u;
}

// Make this wave's LDS writes visible to the other lanes of the same wave.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroup barrier that waits only for this wave's LDS operations
// (lgkmcnt(0)), not for its global loads in flight (a __syncthreads() waits
// for those too).  The builtins alone carry no memory semantics for the
// compiler: the empty asm statements with a memory clobber keep LDS accesses
// on their side of the barrier.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0); vmcnt, expcnt untouched
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Sum over the 64 lanes of a wavefront; every lane receives the total.
// Within each 16-lane row: DPP swaps (quad_perm [1,0,3,2], [2,3,0,1],
// row_half_mirror, row_mirror) -- register-to-register, no LDS round trip;
// then the four row sums are read with v_readlane and added.
__device__ __forceinline__ float dpp_f(float v, int ctrl)
{
    return __builtin_bit_cast(float, ctrl == 0xB1 ? __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)
                                 : ctrl == 0x4E ? __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)
                                 : ctrl == 0x141 ? __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)
                                                 : __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp_f(v, 0xB1);    // lanes 1,0,3,2 of each quad
    v += dpp_f(v, 0x4E);    // lanes 2,3,0,1 of each quad
    v += dpp_f(v, 0x141);   // mirror within each half-row of 8
    v += dpp_f(v, 0x140);   // mirror within the row of 16
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (r0 + r1) + (r2 + r3);
}

// Sum over the 64 lanes, valid in lanes 48..63 only (read it from lane 63):
// the four row sums as in wave_sum, then row_bcast:15 adds row 0 into row 1
// and row 2 into row 3, and row_bcast:31 adds rows 0+1 into row 3.  The
// additions associate as (r2 + r3) + (r0 + r1), i.e. the same value as
// wave_sum, without the four v_readlane round trips.
__device__ __forceinline__ float wave_sum_hi(float v)
{
    v += dpp_f(v, 0xB1);
    v += dpp_f(v, 0x4E);
    v += dpp_f(v, 0x141);
    v += dpp_f(v, 0x140);
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xa, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xc, 0xf, false));
    return v;
}

// Q4_K: 6-bit scale and min of sub-block j from the 3 dwords holding the 12
// packed bytes (byte i of the 12 is byte i%4 of dword i/4).  For j < 4 the
// scale / min are the low 6 bits of bytes j and j+4; for j >= 4 they are the
// low / high nibble of byte j+4 with the top two bits of byte j-4 / j as bits
// 4-5 (packing given with the Llama-3-8B Q4_K workload).
__device__ __forceinline__ void q4k_scale_min(uint32_t s0, uint32_t s1, uint32_t s2, int j,
                                              uint32_t &sc, uint32_t &m)
{
    const uint32_t sh = 8u * (uint32_t)(j & 3);
    const uint32_t a = (s0 >> sh) & 0xffu;  // byte j   (j<4) or j-4 (j>=4)
    const uint32_t b = (s1 >> sh) & 0xffu;  // byte j+4 (j<4) or j   (j>=4)
    const uint32_t c = (s2 >> sh) & 0xffu;  // byte j+4 for j>=4
    if (j < 4) {
        sc = a & 63u;
        m = b & 63u;
    } else {
        sc = (c & 15u) | ((a >> 6) << 4);
        m = (c >> 4) | ((b >> 6) << 4);
    }
}

}  // namespace qmm
