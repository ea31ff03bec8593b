// qmm_quant.hip -- fp16 / fp32 values -> Q8_0 or Q4_0 blocks on gfx950 (the
// encoder of a quantized KV cache; decoding back is qmm_dequant_f16).
//
// dotLLM "GPU Inference", Implementation: the GPU KV-cache is kept in Q8_0 or
// Q4_0 blocks with an FP16 window of recent tokens.  The pages do not give
// the rounding rule; this is the GGUF one, every step in fp32:
//   Q8_0  d = amax / 127, id = 1 / d (0 if d == 0), q = x id rounded half
//         away from zero;
//   Q4_0  v = the value of largest magnitude (the first on a tie),
//         d = v / -8, id = 1 / d (0 if d == 0), q = min(15, trunc(x id + 8.5));
// the codes use the fp32 d, which is then stored rounded to fp16 (RNE).  Both
// divisions are the correctly rounded IEEE ones and no multiply-add is fused
// (contraction is off in the kernel), so the bytes are those of any exact
// fp32 evaluation of the rule.
//
// Work split: a workgroup of 256 lanes encodes 64 consecutive blocks (the
// input is [n][k] with k a multiple of 32, so blocks are contiguous across
// rows).  Four lanes share a block, 8 values each (one 16-byte load for fp16
// input); the block maximum is found with two quad DPP exchanges.  The encoded
// blocks are assembled in LDS and written as whole 16-byte stores (64 blocks
// are 2176 or 1152 bytes, a multiple of 16, so every full group starts
// 16-byte aligned).  Bound: HBM (2 or 4 bytes in, 1.06 or 0.56 bytes out per
// value).
#include "qmm_device.h"
#include "qmm_launch.h"

namespace qmm {

namespace {

constexpr int QBLK = 64;   // blocks per workgroup

__device__ __forceinline__ void load8(const uint16_t *p, float v[8])
{
    const uint4 r = *(const uint4 *)p;
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = h2f(w[i] & 0xffffu);
        v[2 * i + 1] = h2f(w[i] >> 16);
    }
}

__device__ __forceinline__ void load8(const float *p, float v[8])
{
    const float4 a = *(const float4 *)p, b = *(const float4 *)(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ uint32_t xch(uint32_t v, int ctrl)
{
    return __builtin_bit_cast(uint32_t, dpp_f(__builtin_bit_cast(float, v), ctrl));
}

__device__ __forceinline__ uint16_t half_bits(float d)
{
    return __builtin_bit_cast(uint16_t, (_Float16)d);
}

template <int T, typename I>
__global__ void __launch_bounds__(256)
quantize_kernel(const I *__restrict__ x, int64_t nblk, uint8_t *__restrict__ out)
{
#pragma clang fp contract(off)
    constexpr int BB = T == T_Q8_0 ? 34 : 18;
    constexpr int OUT16 = QBLK * BB / 16;          // 16-byte stores per full group
    __shared__ __align__(16) uint16_t st[QBLK * BB / 2];
    const int lane = threadIdx.x, j = lane & 3, bl = lane >> 2;

    for (int64_t grp = blockIdx.x; grp * QBLK < nblk; grp += gridDim.x) {
        const int64_t b = grp * QBLK + bl;
        const bool live = b < nblk;
        float v[8];
        if (live) {
            load8(x + b * 32 + 8 * j, v);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = 0.f;
        }
        uint16_t *sb = st + bl * (BB / 2);      // this block's bytes in LDS

        if constexpr (T == T_Q8_0) {
            float amax = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                amax = fmaxf(amax, fabsf(v[i]));
            amax = fmaxf(amax, dpp_f(amax, 0xB1));
            amax = fmaxf(amax, dpp_f(amax, 0x4E));
            const float d = amax / 127.f;
            const float id = d != 0.f ? 1.f / d : 0.f;
            uint32_t c[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                c[i] = (uint32_t)(int)roundf(v[i] * id) & 0xffu;
            if (live) {
                if (j == 0)
                    sb[0] = half_bits(d);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sb[1 + 4 * j + i] = (uint16_t)(c[2 * i] | (c[2 * i + 1] << 8));
            }
        } else {
            // first value of largest magnitude: lane-local scan in element
            // order, then the lower lane wins ties across lanes
            float amax = 0.f, vmax = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (fabsf(v[i]) > amax) {
                    amax = fabsf(v[i]);
                    vmax = v[i];
                }
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int ctrl = s == 0 ? 0xB1 : 0x4E;
                const float oa = dpp_f(amax, ctrl), ov = dpp_f(vmax, ctrl);
                const int other = j ^ (s == 0 ? 1 : 2);
                if (oa > amax || (oa == amax && other < j)) {
                    amax = oa;
                    vmax = ov;
                }
            }
            const float d = vmax / -8.f;
            const float id = d != 0.f ? 1.f / d : 0.f;
            uint32_t nib = 0;   // the lane's 8 codes, code i in bits 4i..4i+3
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float u = v[i] * id + 8.5f;
                const int c = (int)truncf(u);
                nib |= (uint32_t)(c < 15 ? c : 15) << (4 * i);
            }
            // byte i of the block holds element i (low nibble) and i + 16
            // (high): lanes 0 and 1 take the codes of lanes 2 and 3
            const uint32_t hi = xch(nib, 0x4E);
            if (live && j < 2) {
                if (j == 0)
                    sb[0] = half_bits(d);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t b0 = ((nib >> (8 * i)) & 15u) | (((hi >> (8 * i)) & 15u) << 4);
                    const uint32_t b1 = ((nib >> (8 * i + 4)) & 15u) | (((hi >> (8 * i + 4)) & 15u) << 4);
                    sb[1 + 4 * j + i] = (uint16_t)(b0 | (b1 << 8));
                }
            }
        }
        __syncthreads();
        const int64_t nb = nblk - grp * QBLK < QBLK ? nblk - grp * QBLK : QBLK;
        uint8_t *dst = out + grp * QBLK * BB;
        if (nb == QBLK) {
            if (lane < OUT16)
                ((uint4 *)dst)[lane] = ((const uint4 *)st)[lane];
        } else {
            // last, partial group: 2-byte stores of the bytes that exist
            for (int i = lane; i < nb * (BB / 2); i += 256)
                ((uint16_t *)dst)[i] = st[i];
        }
        __syncthreads();
    }
}

template <typename I>
hipError_t launch_q(int type, const I *x, int64_t n, int64_t k, uint8_t *out, hipStream_t s)
{
    const int64_t nblk = n * (k / 32);
    const int64_t groups = (nblk + QBLK - 1) / QBLK;
    const dim3 grid((unsigned)(groups < (1 << 20) ? groups : (1 << 20))), block(256);
    if (type == T_Q8_0)
        hipLaunchKernelGGL((quantize_kernel<T_Q8_0, I>), grid, block, 0, s, x, nblk, out);
    else if (type == T_Q4_0)
        hipLaunchKernelGGL((quantize_kernel<T_Q4_0, I>), grid, block, 0, s, x, nblk, out);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(int type, const float *x, int64_t n, int64_t k, void *out, hipStream_t s)
{
    return launch_q(type, x, n, k, (uint8_t *)out, s);
}

hipError_t launch_quantize_f16(int type, const uint16_t *x, int64_t n, int64_t k, void *out, hipStream_t s)
{
    return launch_q(type, x, n, k, (uint8_t *)out, s);
}

}  // namespace qmm
