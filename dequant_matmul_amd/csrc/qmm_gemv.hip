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
//   - Weights are read with fully coalesced 16-byte loads: the wavefront
//     copies each row segment (64 lanes x 16 B contiguous per load) into its
//     LDS area and each lane reads its unit back (aligned dword reads,
//     realigned in registers with v_alignbyte_b32 where blocks are only
//     2-byte aligned).  Measured on MI355X this beats per-lane loads of the
//     16-byte-aligned Q4_K units (three 16-byte loads per lane at a 144-byte
//     stride): 14336 x 4096 Q4_K 10.3 -> 8.9 us, 4096 x 4096 5.3 -> 4.3 us.
//   - Codes are converted with a few bit operations per dword plus the byte
//     converts (v_cvt_f32_ubyteN, or the sign-extending SDWA convert), or for
//     Q4_K straight inside the weight-forming fma (a nibble alone in a
//     16-bit half is an exact fp16 subnormal, read by v_fma_mix_f32), and
//     every product uses the element's own weight: integer code offsets
//     (-8, -16, -32) become signed bytes before the convert, the K-quant
//     weights d sc q - dmin m are formed per element with one fma.  Sums are
//     fp32 per block or sub-block; integer-code scales are applied once per
//     (sub-)block.
//   - Per-lane partial sums of 8 rows at a time are reduced together
//     through LDS (8 lanes per row), one store per 8 rows.
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
//   gemv3s_kernel the stage launch of the decode pass: up to three groups of
//                 problems of different block types (same lane-unit size)
//                 sharing one x, wave slots split by weight bytes.
//   gemv4_kernel  batch 1, k of two to eight segments (up to 16384): a
//                 workgroup owns a block of rows, its waves split the
//                 segments, x is staged whole in LDS once, and the partial
//                 sums meet in LDS.
//   gemv1_kernel  batch 1, longer k: x is staged in LDS per segment,
//                 otherwise as gemv3.
//   gemv_kernel   batch 2..8 of Q8_0 / Q4_0 / Q5_0 / Q5_K, batch 2 of Q4_K /
//                 Q6_K below 65536 rows (and unaligned batch-1 rows): x
//                 segment and weight segments staged in LDS per workgroup.
//   The other batches 2..8 of Q4_K / Q6_K run on the matrix cores
//   (qmm_gemv_mfma.hip).
#include "qmm_device.h"
#include "qmm_gemv_unit.h"
#include "qmm_launch.h"

#include <type_traits>

namespace qmm {

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

// A mixed-type launch (gemv3s): up to STAGE_MAXG groups, each a table of
// problems of one block type.  The groups' block types and wave-slot ranges
// travel as plain kernel arguments (preloaded into SGPRs), the tables here.
constexpr int STAGE_MAXG = 3;
struct StageGroups {
    GemvProbs P[STAGE_MAXG];
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
    __device__ __forceinline__ int rg_end(int, int R) const { return (n + R - 1) / R; }
    __device__ __forceinline__ const uint8_t *W(int) const { return w; }
    __device__ __forceinline__ const float *X(int) const { return x; }
    __device__ __forceinline__ float *Y(int) const { return y; }
    __device__ __forceinline__ int N(int) const { return n; }
};
// The table's row-group starts are read at constant indices, so that the
// reads are one batch of independent scalar loads (a loop bounded by np, or
// an index read from the table, chains one load round trip after another
// ahead of the first weight load).  The problem of a row group is the number
// of starts (past the first) at or below it: the starts never decrease.
struct TableProbs {
    const GemvProbs &P;
    __device__ __forceinline__ int total_rg(int) const
    {
        int r[GEMV_MAXP + 1];
#pragma unroll
        for (int q = 0; q <= GEMV_MAXP; ++q)
            r[q] = P.rg0[q];
        const int np = P.np;
        int t = 0;
#pragma unroll
        for (int q = 1; q <= GEMV_MAXP; ++q)
            t = q == np ? r[q] : t;
        return t;
    }
    __device__ __forceinline__ int find(int rg) const
    {
        int r[GEMV_MAXP];
#pragma unroll
        for (int q = 0; q < GEMV_MAXP; ++q)
            r[q] = P.rg0[q];
        const int np = P.np;
        int pp = 0;
#pragma unroll
        for (int q = 1; q < GEMV_MAXP; ++q)
            pp += (int)(q < np) & (int)(rg >= r[q]);
        return pp;
    }
    __device__ __forceinline__ int rg_begin(int pp) const { return P.rg0[pp]; }
    __device__ __forceinline__ int rg_end(int pp, int) const { return P.rg0[pp + 1]; }
    __device__ __forceinline__ const uint8_t *W(int pp) const { return P.w[pp]; }
    __device__ __forceinline__ const float *X(int pp) const { return P.x[pp]; }
    __device__ __forceinline__ float *Y(int pp) const { return P.y[pp]; }
    __device__ __forceinline__ int N(int pp) const { return P.n[pp]; }
};
// A table whose problems all read one x, passed as a kernel argument.
struct SharedXProbs : TableProbs {
    const float *xs;
    __device__ __forceinline__ const float *X(int) const { return xs; }
};

// NW wavefronts per workgroup.  xl (X_LDS): the workgroup first copies the
// single problem's x into LDS, and each wave takes its lane slice from there
// (instead of every wave reading all of x from L2, which with many waves
// costs more L2 traffic than the weights).
//
// gw / tw: this wave's index among the tw waves that share the rows (all
// waves of the grid, or the waves of one block type in a mixed launch).
//
// WSTRIDE: dwords of the LDS segment area per wave (0: this type's own size;
// a launch mixing block types passes the largest, so that the waves' areas
// do not overlap).
//
// X_LDS staging: by default the problem's x (k floats, one segment at most);
// a caller whose waves work on different column ranges of one row passes the
// whole x (xsrc, xn floats, at most XMAX) and this wave's offset xoff into
// the padded LDS copy.
template <int T, int R, class PS, int NW = 4, bool X_LDS = false, int WSTRIDE = 0, int XMAX = 0, bool NT = true>
__device__ __forceinline__ void gemv2_body(const PS &P, int k, int64_t rb, uint32_t *ws, float *xl, int gw, int tw,
                                           const float *xsrc = nullptr, int xn = 0, int xoff = 0)
{
    constexpr int UE = GemvUnit<T>::UE, NRUN = GemvUnit<T>::NRUN;
    using S = SegStage<T, R, NT>;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // X_LDS: this thread's share of x is loaded into registers first, so
    // that it is in flight together with the first weight loads (issued
    // next), and written to LDS after them (stage_x).  Positions past the
    // end read x[0..3] and are not stored.
    constexpr int XV = X_LDS ? ((XMAX ? XMAX : 64 * UE) + 4 * 64 * NW - 1) / (4 * 64 * NW) : 1;
    const int xcount = xsrc ? xn : k;
    f32x4 xst[XV];
    if constexpr (X_LDS) {
        const float *x = xsrc ? xsrc : P.X(0);
#pragma unroll
        for (int j = 0; j < XV; ++j) {
            const int e = 4 * ((int)threadIdx.x + 64 * NW * j);
            xst[j] = *(const f32x4 *)(x + (e < xcount ? e : 0));
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
                if (e < xcount)
                    *(f32x4 *)(xl + xpad<UE>(e)) = xst[j];
            }
            lds_barrier();
        }
    };
    // each wave takes a contiguous run of row groups (run lengths differ by
    // at most one, so every wave has work when there are enough)
    const int nrg = P.total_rg(R);
    const int q = nrg / tw, rem = nrg - q * tw;    // one 32-bit division
    const int rgs = gw * q + min(gw, rem);
    const int nit = q + (gw < rem ? 1 : 0);
    const bool active = lane < k / UE;
    const int cpr = k / Fmt<T>::BE * Fmt<T>::BB / 16;

    // Problem of an item: a cursor walks the problems as the items advance
    // (items are visited in increasing order), so that the problem's
    // pointers and sizes are read from the table only when it changes, not
    // per item (each such scalar read is a wait in the item loop).
    struct Cur {
        int pp, beg, end, n;
        const uint8_t *w;
    };
    auto cur_set = [&](Cur &c, int pp) __attribute__((always_inline)) {
        c.pp = pp;
        c.beg = P.rg_begin(pp);
        c.end = P.rg_end(pp, R);
        c.n = P.N(pp);
        c.w = P.W(pp);
    };
    // first row group of item it (past the end: the last item; a wave with
    // no item: the last row group)
    auto item_rg = [&](int it) __attribute__((always_inline)) {
        it = min(it, max(nit - 1, 0));
        return min(rgs + it, nrg - 1);
    };
    auto locate = [&](Cur &c, int it) __attribute__((always_inline)) {
        const int rg = item_rg(it);
        if (rg >= c.end)
            cur_set(c, P.find(rg));
        return (rg - c.beg) * R;   // first row of the item in its problem
    };
    Cur cl, cs;                    // the load and the compute cursors
    cur_set(cl, P.find(item_rg(0)));
    cs = cl;

    // this lane's slice of x for the current problem
    f32x4 xr[NRUN];
    auto load_x = [&](int pp) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NRUN; ++j) {
            const int e = active ? run_elem<T>(lane, j) : 0;
            xr[j] = X_LDS ? *(const f32x4 *)(xl + xoff + xpad<UE>(e)) : *(const f32x4 *)(P.X(pp) + e);
        }
    };
    const XFromRegs<T> xg{xr};

    float acc[R][1];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r][0] = 0.f;

    int xp = cs.pp;
    if constexpr (!X_LDS)
        load_x(xp);

    // Row results: each lane's partial sum of a row goes to LDS (one slot of
    // 64 floats per row, RG rows per group); a full group (or a problem
    // change, or the end) is reduced across lanes at once, 8 lanes per row
    // (two 128-bit reads, 7 adds and 3 DPP steps per 8 rows instead of a
    // full 64-lane reduction per row), and leaves as one store per 8 rows.
    constexpr int RG = 8;
    static_assert(R <= RG, "rows per item above the reduction group");
    __shared__ __attribute__((aligned(16))) float redbuf[NW * RG * 64];
    float *const red = redbuf + wave * (RG * 64);
    int blk_row = 0, blk_cnt = 0, blk_pp = -1, blk_n = 0;
    float *blk_y = nullptr;
    auto flush = [&]() __attribute__((always_inline)) {
        if (blk_cnt > 0) {
            wave_lds_sync();
            const int rr = lane >> 3, q8 = lane & 7;
            const f32x4 a = *(const f32x4 *)(red + 8 * lane), b = *(const f32x4 *)(red + 8 * lane + 4);
            float v = ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w));
            v += dpp_f(v, 0xB1);    // lanes 1,0,3,2 of each quad
            v += dpp_f(v, 0x4E);    // lanes 2,3,0,1 of each quad
            v += dpp_f(v, 0x141);   // the other quad of each 8 lanes
            const int row = blk_row + rr;
            if (q8 == 0 && rr < blk_cnt && row < blk_n)
                blk_y[row] = v;
            wave_lds_sync();
        }
        blk_cnt = 0;
    };
    auto finish = [&](int row0) __attribute__((always_inline)) {
        if (blk_cnt + R > RG || (blk_cnt > 0 && cs.pp != blk_pp))
            flush();
        if (blk_cnt == 0) {
            blk_row = row0;
            if (cs.pp != blk_pp) {
                blk_pp = cs.pp;
                blk_n = cs.n;
                blk_y = P.Y(blk_pp);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            red[(blk_cnt + r) * 64 + lane] = active ? acc[r][0] : 0.f;
            acc[r][0] = 0.f;
        }
        blk_cnt += R;
    };

    // Rows are staged through LDS: the wave loads an item's row segments
    // with fully coalesced 16-byte loads (64 lanes, contiguous), stores them
    // to its LDS area and each lane reads its unit back.  One prefetch
    // register set: it is emptied into LDS before being refilled (no copy of
    // an in-flight load).  Prefetches past the wave's last item read offset
    // 0 in every lane (one cache line, no branch: a load under a branch is
    // waited for at once).  Lanes past k compute on offset-0 bytes and
    // contribute 0 (select, not branch).
    static_assert(WSTRIDE == 0 || WSTRIDE >= S::LDS_DW, "LDS segment area too small");
    uint32_t *mw = ws + wave * (WSTRIDE ? WSTRIDE : S::LDS_DW);
    S st;
    auto load = [&](int it) __attribute__((always_inline)) {
        const int row0 = locate(cl, it);
        if constexpr (R == 1 && NT) {
            // past the wave's last item: an empty range, every chunk reads zero
            st.load_row(cl.w + (int64_t)row0 * rb, it < nit ? (uint32_t)(16 * cpr) : 0u, lane);
        } else {
            // past the wave's last item: no row is in range, every chunk reads offset 0
            st.load(cl.w, rb, it < nit ? cl.n : 0, row0, 0, cpr, lane);
        }
    };
    load(0);
    if constexpr (X_LDS) {
        stage_x();
        load_x(xp);
    }
    for (int it = 0; it < nit; ++it) {
        const int row0 = locate(cs, it);
        if (cs.pp != xp) {   // wave-uniform: the next problem's x
            xp = cs.pp;
            load_x(xp);
        }
        st.store(mw, lane);
        wave_lds_sync();
        load(it + 1);
        URaw<T> cur[R];
#pragma unroll
        for (int r = 0; r < R; ++r) raw_from_lds<T>(mw + r * S::RS, lane, cur[r]);
        unit_dot<T, 1, R>(cur, lane, xg, acc);
        finish(row0);
        wave_lds_sync();
    }
    flush();
}

// Batch 1, one problem, x staged in LDS, NW wavefronts per workgroup (one
// workgroup per CU: 16 waves, 4 per SIMD, hide the weight latency).
template <int T, int R, int NW, bool NT>
__global__ void __launch_bounds__(64 * NW)
gemv3_kernel(const uint8_t *__restrict__ w, int n, int k, int64_t rb, const float *__restrict__ x,
             float *__restrict__ y)
{
    __shared__ __attribute__((aligned(16))) float xl[64 * (GemvUnit<T>::UE + 4)];
    __shared__ __attribute__((aligned(16))) uint32_t ws[NW * SegStage<T, R>::LDS_DW];
    const OneProb P{w, x, y, n};
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    gemv2_body<T, R, OneProb, NW, true, 0, 0, NT>(P, k, rb, ws, xl, blockIdx.x * NW + wave, gridDim.x * NW);
}

template <int T, int R>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 4)))
gemv2m_kernel(const GemvProbs Pt, int k, int64_t rb)
{
    __shared__ __attribute__((aligned(16))) uint32_t ws[4 * SegStage<T, R>::LDS_DW];
    const TableProbs P{Pt};
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    gemv2_body<T, R>(P, k, rb, ws, nullptr, blockIdx.x * 4 + wave, gridDim.x * 4);
}

// The table of problems with one x shared by all of them (the q / k / v or
// gate / up projections of a layer read the same activation): x staged in
// LDS as in gemv3, one row per item.
template <int T, int R, int NW>
__global__ void __launch_bounds__(64 * NW)
gemv3m_kernel(const GemvProbs Pt, int k, int64_t rb)
{
    __shared__ __attribute__((aligned(16))) float xl[64 * (GemvUnit<T>::UE + 4)];
    __shared__ __attribute__((aligned(16))) uint32_t ws[NW * SegStage<T, R>::LDS_DW];
    const TableProbs P{Pt};
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    gemv2_body<T, R, TableProbs, NW, true>(P, k, rb, ws, xl, blockIdx.x * NW + wave, gridDim.x * NW);
}

// -------------------------------------------------------------- gemv3s --
// One stage of a decode pass: up to STAGE_MAXG groups of problems, each group
// one block type (all types of a launch share the lane-unit size UEK), every
// problem reading the same x of k <= one segment (q / k / v, gate / up of a
// layer).  x is staged in LDS once per workgroup; the waves are split between
// the groups in proportion to their weight bytes, numbered wave-major
// (slot = wave * grid + workgroup) so that every workgroup holds waves of
// every group, and each wave runs its group's table loop.
// Group g owns the wave slots [wb_g, wb_{g+1}) with wb_0 = 0, wb_1 = wb1,
// wb_2 = wb2 and wb_3 = all slots (a launch of fewer groups passes all slots
// for the missing boundaries); its block type is bits 4g..4g+3 of types.
// grid is gridDim.x, passed as an argument: the argument arrives in an SGPR,
// while gridDim.x is a read of the dispatch's implicit arguments.
template <int T, class PS, int NW, int WSDW>
__device__ __forceinline__ void stage_body(const PS &P, int k, uint32_t *ws, float *xl, int gw, int tw)
{
    const int64_t rb = (int64_t)(k / Fmt<T>::BE) * Fmt<T>::BB;
    gemv2_body<T, 1, PS, NW, true, WSDW>(P, k, rb, ws, xl, gw, tw);
}

template <int UEK, int NW>
__global__ void __launch_bounds__(64 * NW)
gemv3s_kernel(const float *__restrict__ x, int k, int grid, int wb1, int wb2, int types, const StageGroups G)
{
    constexpr int WSDW = UEK == 64 ? SegStage<T_Q6_K, 1>::LDS_DW : SegStage<T_Q8_0, 1>::LDS_DW;
    __shared__ __attribute__((aligned(16))) float xl[64 * (UEK + 4)];
    __shared__ __attribute__((aligned(16))) uint32_t ws[NW * WSDW];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slot = wave * grid + (int)blockIdx.x;
    const int g = (slot >= wb1 ? 1 : 0) + (slot >= wb2 ? 1 : 0);
    const int lo = g == 0 ? 0 : g == 1 ? wb1 : wb2;
    const int hi = g == 0 ? wb1 : g == 1 ? wb2 : grid * NW;
    const int gw = slot - lo, tw = hi - lo;
    const SharedXProbs P{{G.P[g]}, x};
    if constexpr (UEK == 64) {
        switch ((types >> (4 * g)) & 15) {
        case T_Q4_K: stage_body<T_Q4_K, SharedXProbs, NW, WSDW>(P, k, ws, xl, gw, tw); break;
        case T_Q6_K: stage_body<T_Q6_K, SharedXProbs, NW, WSDW>(P, k, ws, xl, gw, tw); break;
        default: stage_body<T_Q5_K, SharedXProbs, NW, WSDW>(P, k, ws, xl, gw, tw); break;
        }
    } else {
        switch ((types >> (4 * g)) & 15) {
        case T_Q4_0: stage_body<T_Q4_0, SharedXProbs, NW, WSDW>(P, k, ws, xl, gw, tw); break;
        case T_Q8_0: stage_body<T_Q8_0, SharedXProbs, NW, WSDW>(P, k, ws, xl, gw, tw); break;
        default: stage_body<T_Q5_0, SharedXProbs, NW, WSDW>(P, k, ws, xl, gw, tw); break;
        }
    }
}

// --------------------------------------------------------------- gemv4 --
// Batch 1, k spanning several segments: the workgroup owns rwg consecutive
// rows and its waves split k by segment -- wave w takes segment w % nseg,
// the waves of one segment split the rows, and each runs the one-segment
// loop (gemv2_body) on its segment's columns with that slice of x in its
// registers (the row pitch stays the full row).  Per-(segment, row) partial
// sums meet in LDS and are added in segment order, so the result does not
// depend on timing.
constexpr int GEMV4_XMAX = 16384;  // the longest x the kernel stages in LDS
constexpr int GEMV4_PART = 4096;   // LDS floats for the partial sums (nseg * rwg)

template <int T, int NW, bool NT>
__global__ void __launch_bounds__(64 * NW)
gemv4_kernel(const uint8_t *__restrict__ w, int n, int k, int64_t rb, const float *__restrict__ x,
             float *__restrict__ y, int rwg, int nseg)
{
    using S = SegStage<T, 1>;
    constexpr int UE = GemvUnit<T>::UE;
    constexpr int XMAX = GEMV4_XMAX;
    __shared__ __attribute__((aligned(16))) float xl[XMAX + XMAX / UE * 4];
    __shared__ __attribute__((aligned(16))) uint32_t ws[NW * S::LDS_DW];
    __shared__ float part[GEMV4_PART];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row0 = (int)blockIdx.x * rwg;
    const int nr = min(rwg, n - row0);
    const int wps = NW / nseg;                 // waves per segment
    const int seg = wave % nseg, sub = wave / nseg;
    // every wave stages its share of the whole x once (waves past wps * nseg
    // too) and takes its segment's slice from LDS
    const int kseg = min(S::SEGE, k - seg * S::SEGE);
    const OneProb P{w + (int64_t)row0 * rb + (int64_t)seg * S::SEGB, x, part + seg * rwg, sub < wps ? nr : 0};
    gemv2_body<T, 1, OneProb, NW, true, 0, XMAX, NT>(P, kseg, rb, ws, xl, sub < wps ? sub : 0, wps, x, k,
                                                    xpad<UE>(seg * S::SEGE));
    __syncthreads();
    for (int t = threadIdx.x; t < nr; t += 64 * NW) {
        float v = part[t];
        for (int g = 1; g < nseg; ++g)
            v += part[g * rwg + t];
        y[row0 + t] = v;
    }
}

// --------------------------------------------------------------- gemv1 --
// Batch 1, k spanning several segments: x staged in LDS once per workgroup;
// each wave walks items (R rows x one segment) with the weight bytes of the
// next D items in flight (a ring of D register stages, so a row's segments
// are fetched together rather than one round trip after another).
template <int T, int R, int NW, int XK, int D, bool NT>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 4)))
gemv1_kernel(const uint8_t *__restrict__ w, int n, int k, int64_t rb, const float *__restrict__ x,
             float *__restrict__ y)
{
    using F = Fmt<T>;
    constexpr int UE = GemvUnit<T>::UE;
    using S = SegStage<T, R, NT>;
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
    using S = SegStage<T, R, false>;
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

// Matrices of at least this many bytes stream their weights with
// non-temporal loads; smaller single launches are faster with plain ones
// (Q8_0 2048 x 2048, 4.5 MB, over rotating copies: 2.92 us plain, 3.35 us
// non-temporal), and the decode passes faster with non-temporal loads from
// the 4096 x 4096 Q4_K projection (9.4 MB) up.
constexpr int64_t NT_MIN_BYTES = 8 << 20;

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
    if (n * (int64_t)rb >= NT_MIN_BYTES)
        hipLaunchKernelGGL((gemv3_kernel<T, R, NW, true>), grid, block, 0, s, w, (int)n, (int)k, (int64_t)rb, x, y);
    else
        hipLaunchKernelGGL((gemv3_kernel<T, R, NW, false>), grid, block, 0, s, w, (int)n, (int)k, (int64_t)rb, x, y);
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

template <int UEK, int NW>
static hipError_t launch_stage_t(const StageGroups &G, int ng, const int *type, const int64_t *bytes, int64_t rows,
                                 int64_t k, const float *x, hipStream_t s)
{
    const int cus = device_cu_count();
    if (cus == 0)
        return hipErrorInvalidValue;
    const int64_t want = (rows + NW - 1) / NW;
    const int grid = (int)(want < cus ? want : cus);
    // wave slots in proportion to the groups' weighted bytes, at least one
    // and at most one per row for each group
    const int tot = grid * NW;
    int64_t btot = 0;
    for (int g = 0; g < ng; ++g)
        btot += bytes[g];
    int cnt[STAGE_MAXG], used = 0;
    for (int g = 0; g < ng; ++g) {
        const int64_t r = G.P[g].rg0[G.P[g].np];
        int64_t c = btot > 0 ? (tot * bytes[g] + btot / 2) / btot : 1;
        c = c < 1 ? 1 : c > r ? r : c;
        cnt[g] = (int)c;
        used += cnt[g];
    }
    // fix the sum: surplus slots go to (or are taken from) the largest groups
    while (used != tot) {
        int best = -1;
        for (int g = 0; g < ng; ++g) {
            const int64_t r = G.P[g].rg0[G.P[g].np];
            const bool can = used < tot ? cnt[g] < r : cnt[g] > 1;
            if (can && (best < 0 || bytes[g] > bytes[best]))
                best = g;
        }
        if (best < 0)
            break;
        cnt[best] += used < tot ? 1 : -1;
        used += used < tot ? 1 : -1;
    }
    // group boundaries; slots past the last group (when every group is
    // capped at its rows) fall into the last group and find no row there
    int wb[STAGE_MAXG] = {0, tot, tot}, types = 0;
    for (int g = 0; g < ng; ++g)
        types |= type[g] << (4 * g);
    for (int g = 1; g < ng; ++g)
        wb[g] = wb[g - 1] + cnt[g - 1];
    hipLaunchKernelGGL((gemv3s_kernel<UEK, NW>), dim3((unsigned)grid), dim3(64 * NW), 0, s, x, (int)k, grid, wb[1],
                       wb[2], types, G);
    return hipGetLastError();
}

hipError_t launch_gemv_stage(int ng, const int *type, const int *np, const void *const *w, const int64_t *n,
                             int64_t k, const float *x, float *const *y, hipStream_t s)
{
    StageGroups G{};
    int64_t bytes[STAGE_MAXG] = {0, 0, 0};
    int64_t rows = 0;
    int i = 0;
    int ue = 0;
    for (int g = 0; g < ng; ++g) {
        const int t = type[g];
        const int be = (t == T_Q4_K || t == T_Q6_K || t == T_Q5_K) ? 256 : 32;
        const int bb = t == T_Q4_0 ? 18 : t == T_Q8_0 ? 34 : t == T_Q4_K ? 144 : t == T_Q6_K ? 210 : t == T_Q5_0 ? 22 : 176;
        ue = be == 256 ? 64 : 32;
        const int64_t rb = k / be * bb;
        GemvProbs &P = G.P[g];
        P.np = np[g];
        P.rg0[0] = 0;
        for (int j = 0; j < np[g]; ++j, ++i) {
            P.w[j] = (const uint8_t *)w[i];
            P.x[j] = x;
            P.y[j] = y[i];
            P.n[j] = (int)n[i];
            P.rg0[j + 1] = P.rg0[j] + (int)n[i];
            // Q6_K rows take longer per byte than Q4_K rows (2-byte-aligned
            // blocks read back from LDS with realignment): they get 1.4x
            // their byte share of the waves (q|k|v of the Q4_K_M-style mix:
            // 8.2 -> 7.9 us; 0.6x / 2x / 3x: 9.0 / 8.2 / 8.5 us)
            bytes[g] += n[i] * rb * (t == T_Q6_K ? 14 : 10) / 10;
        }
        rows += P.rg0[P.np];
    }
    if (rows == 0)
        return hipSuccess;
    if (ue == 64)
        return launch_stage_t<64, 8>(G, ng, type, bytes, rows, k, x, s);
    // 16 waves per compute unit for the 32-element types with many rows (as gemv3)
    return rows >= 4096 ? launch_stage_t<32, 16>(G, ng, type, bytes, rows, k, x, s)
                        : launch_stage_t<32, 8>(G, ng, type, bytes, rows, k, x, s);
}

template <int T, int R, int NW, int XK, int D, bool NT>
static hipError_t launch_b1_lds_nt(const uint8_t *w, int64_t n, int64_t k, size_t rb, const float *x, float *y,
                                   hipStream_t s)
{
    static std::atomic<int> slot[64];
    const int cap = per_device_cached(slot, [] { return resident_wgs(gemv1_kernel<T, R, NW, XK, D, NT>, 64 * NW); });
    if (cap == 0)
        return hipErrorInvalidValue;
    const int64_t want = ((n + R - 1) / R + NW - 1) / NW;
    const dim3 grid((unsigned)(want < cap ? want : cap)), block(64 * NW);
    hipLaunchKernelGGL((gemv1_kernel<T, R, NW, XK, D, NT>), grid, block, 0, s, w, (int)n, (int)k, (int64_t)rb, x, y);
    return hipGetLastError();
}

template <int T, int R, int NW, int XK, int D>
static hipError_t launch_b1_lds(const uint8_t *w, int64_t n, int64_t k, size_t rb, const float *x, float *y,
                                hipStream_t s)
{
    if (n * (int64_t)rb >= NT_MIN_BYTES)
        return launch_b1_lds_nt<T, R, NW, XK, D, true>(w, n, k, rb, x, y, s);
    return launch_b1_lds_nt<T, R, NW, XK, D, false>(w, n, k, rb, x, y, s);
}

template <int T, int NW>
static hipError_t launch_b1_split(const uint8_t *w, int64_t n, int64_t k, size_t rb, const float *x, float *y,
                                  int nseg, hipStream_t s)
{
    const int cus = device_cu_count();
    if (cus == 0)
        return hipErrorInvalidValue;
    int64_t rwg = (n + cus - 1) / cus;
    const int64_t cap = GEMV4_PART / nseg;
    rwg = rwg < cap ? rwg : cap;
    const int64_t grid = (n + rwg - 1) / rwg;
    if (n * (int64_t)rb >= NT_MIN_BYTES)
        hipLaunchKernelGGL((gemv4_kernel<T, NW, true>), dim3((unsigned)grid), dim3(64 * NW), 0, s, w, (int)n,
                           (int)k, (int64_t)rb, x, y, (int)rwg, nseg);
    else
        hipLaunchKernelGGL((gemv4_kernel<T, NW, false>), dim3((unsigned)grid), dim3(64 * NW), 0, s, w, (int)n,
                           (int)k, (int64_t)rb, x, y, (int)rwg, nseg);
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
        const int nseg = (int)((k + 64 * GemvUnit<T>::UE - 1) / (64 * GemvUnit<T>::UE));
        if (nseg <= 8 && k <= GEMV4_XMAX) {
            // the segments split over the waves of a workgroup, the whole x
            // staged in LDS once (gemv4): as many waves per segment as fit in 8
            switch (nseg) {
            case 2: case 4: case 8: return launch_b1_split<T, 8>(w, n, k, rb, x, y, nseg, s);
            case 3: return launch_b1_split<T, 6>(w, n, k, rb, x, y, nseg, s);
            case 5: return launch_b1_split<T, 5>(w, n, k, rb, x, y, nseg, s);
            case 6: return launch_b1_split<T, 6>(w, n, k, rb, x, y, nseg, s);
            default: return launch_b1_split<T, 7>(w, n, k, rb, x, y, nseg, s);
            }
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
    // Batch 2 of the K-quants takes the fp32 vector kernel below (1 + 2
    // operations per weight, two rows per item) except on very tall matrices:
    // measured on MI355X at B = 2 against the matrix-core kernel, 14336 x
    // 4096 Q4_K 21.3 -> 17.7 us, 4096 x 14336 Q6_K 28.2 -> 21.3, 4096 x 4096
    // Q4_K 8.9 -> 6.7, 1024 x 4096 Q4_K 8.9 -> 4.8; the 128256 x 4096 Q6_K
    // head (128 -> 151 us) stays on the matrix cores, and so does every
    // batch from 3 on (the vector kernel's x staging then leaves one
    // workgroup per compute unit: 34 us for the 14336 x 4096 Q4_K at B = 3).
    if (gemv_mfma_supported(T, batch) && !(batch == 2 && n < 65536))
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
    // batch 3..8 of the K-quants, one x for every problem: one matrix-core
    // launch over all their tiles (x converted once per workgroup for more
    // tiles, one launch instead of one per matrix)
    if (batch >= 3 && gemv_mfma_multi_supported(T, batch, k)) {
        bool shared = true;
        for (int i = 1; i < np; ++i)
            shared = shared && x[i] == x[0];
        if (shared)
            return launch_gemv_mfma_multi(T, np, w, n, k, rb, x[0], batch, y, s);
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
