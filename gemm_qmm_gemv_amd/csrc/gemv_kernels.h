// gemv_kernels.h -- bandwidth-bound quantized GEMV kernels (decode, M = 1) and the
// multi-row variant used for small M and for mixture-of-experts rows.
//
// Pages: "BaseRT claims fastest Apple Silicon inference" (thetesserapress.com),
// section "What BaseRT does differently": a dedicated GEMV for decode (M = 1),
// dequantization inline, memory traffic proportional to the compressed size.
//
// Work decomposition (wave64):
//   A row of W is cut into units of UNIT codes (64, or 32 when the group size
//   is an odd multiple of 32); a unit always lies inside one quantization
//   group, so it needs one scale and one min.  LPR lanes cooperate on a row:
//   lane j of the row owns units j, j+LPR, ..., (XC of them per pass), so the
//   LPR lanes of a slot read LPR consecutive units -- contiguous memory.  A
//   wave holds 64/LPR such slots and handles U rows per slot per iteration,
//   issuing every weight load of the iteration before any arithmetic
//   (U*XC units in flight per lane).  The activation side of each owned unit
//   (pairs, offset constant, plain sum) is built once per wave and reused for
//   every row the wave visits.  Partial sums are reduced across the LPR lanes
//   with cross-lane shuffles; results are deterministic (the one exception is
//   the expert rows' weighted combine, which adds into token rows with float
//   atomics in no fixed order).
//
// Fused variants share these loops: the SiLU-gated product of two matrices
// and the residual add (decode), the gate/up product and the weighted
// combine (expert rows).
#pragma once

#include "qmm_device.h"
#include "qmm_kernels.h"

#include <type_traits>

namespace qmm {

// Weights of one row batch held in registers: U rows per slot, XC units per
// lane, with each unit's scale and min (fp16 bits).  On the wide path the
// scales and mins arrive instead as one 32-bit word per lane of the batch's
// contiguous scale block (and min block) and are handed out to the lanes
// that need them with cross-lane permutes.
// Every GEMV-family launch uses 256-thread work-groups (the launch bounds
// below); a compile-time count saves a kernel-argument load.
constexpr int GEMV_WAVES_PER_BLOCK = 4;

// Output staging.  Stores and loads share one in-order completion counter on
// this architecture, so a store issued inside the pipelined loop makes the
// next wait for a load also wait for that store's write to complete.  The
// row sums are therefore parked in LDS (a per-wave area of YSTAGE floats) and
// written out with coalesced stores once per run, or when the area is full.
// (Both the batched launch and the single GEMV run their rows this way.)
constexpr int YSTAGE = 256;

// XLDS: the activation units come from the work-group's LDS copy xl (see
// gemv_kernel) instead of every lane's registers.
template <int B, int UNIT, int LPR, int XC, int U, bool RES, bool XLDS = false>
__device__ __forceinline__ void gemv_run(const u32* W, const uint16_t* S, const uint16_t* Mn,
                                         const uint16_t* X, float* Y, int n, int k, int group, int b0,
                                         int b1, int lane, float* ystage, int base, int bstride,
                                         const float* R, const u32* xl = nullptr);

// Single GEMVs over quantized weights keep the row's activation units once
// per work-group in LDS: building them in every lane (a strided read of the
// whole of x per wave, and its conversion) costs more than reading them back
// from LDS for each row batch, most where a wave has few batches.  Measured
// (cache-busted, one launch, Q4 unless named): 3072 x 8192 8.1 -> 6.0 us
// (Q2 7.6 -> 5.5, Q8 9.8 -> 8.1), 2048 x 8192 7.9 -> 5.3, 8192 x 2048 5.95 ->
// 5.00, 4096 x 4096 5.91 -> 5.13, 3072 x 1024 3.97 -> 3.51, 1024 x 1024 3.82
// -> 3.35, 151936 x 1024 Q2 13.4 -> 12.6; the staged 64 x 1 rows of the
// larger matrices lose a little (8192 x 4096 6.6 -> 6.8, 65536 x 4096 27.2 ->
// 27.6).  fp16 weights keep their registers except in 16 x 3 rows (in LDS,
// 3072 x 3072 5.8 -> 6.1 us and 65536 x 3072 65.2 -> 66.6 at 64 x 2).
template <int B, int LPR, int XC>
constexpr bool xunits_in_lds() {
    return XC == 3 || B < 16;
}

// Work-group barrier for LDS data only: waits for this wave's LDS traffic,
// not for its vector-memory loads in flight (a __syncthreads also drains
// those).  The wait is the builtin, so the compiler's own bookkeeping knows
// of it; the barrier is an asm statement with a memory clobber, so no load
// or store moves across it.
__device__ __forceinline__ void lds_barrier() {
    // s_waitcnt fields: vmcnt bits 3:0 and 15:14 (63: no wait), expcnt 6:4
    // (7: no wait), lgkmcnt 11:8 (0).
    __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (7 << 4));
    asm volatile("s_barrier" ::: "memory");
}

// a / group for the group size, a wave-uniform kernel argument: a shift for
// the usual power-of-two sizes (a uniform branch), a division otherwise.
// The division's set-up had put dozens of instructions between the
// argument loads and the first weight load of every launch.
__device__ __forceinline__ int div_group(int a, int group) {
    if ((group & (group - 1)) == 0) return a >> __builtin_ctz((unsigned)group);
    return a / group;
}

template <int B, int UNIT, int XC, int U>
struct RowBatch {
    static constexpr int WPU = UNIT * B / 32;
    u32 w[U][XC][WPU];
    u32 s[U][XC], m[U][XC];
    u32 sblk, mblk;
};

// Scale/min loads: the rows of one iteration (rb .. rb + SLOTS*U - 1) are
// consecutive, so their scales form one contiguous block of SLOTS*U*gpr fp16
// values, and likewise their mins.  When that block fits one 32-bit word per
// lane (and the arrays are 4-byte aligned with an even group count per row)
// two dword loads per lane replace 2*U*XC two-byte loads: fewer memory
// instructions and whole cache lines.
template <int LPR, int U>
__device__ __forceinline__ bool wide_scales_ok(const uint16_t* S, const uint16_t* Mn, int gpr) {
    constexpr int SLOTS = 64 / LPR;
    return ((reinterpret_cast<uintptr_t>(S) | reinterpret_cast<uintptr_t>(Mn)) & 3u) == 0 &&
           (gpr & 1) == 0 && SLOTS * U * gpr <= 128;
}

// Buffer resources over one matrix: packed weights, scales, mins, with their
// byte sizes.  An offset equal to the size reads zeros, which is how lanes
// with nothing to load are handled without branches.
struct MatRsrc {
    rsrc_t w, s, m;
    uint32_t wbytes, sbytes;
};
// Formats without scales and mins get empty resources for them: every such
// load reads zero without touching memory, so those pointers may be null.
template <int B>
__device__ __forceinline__ MatRsrc mat_rsrc(const void* W, const void* S, const void* Mn, int n,
                                            int wpr, int gpr) {
    const uint32_t wb = (uint32_t)n * (uint32_t)wpr * 4u;
    const uint32_t sb = has_affine<B>() ? (uint32_t)n * (uint32_t)gpr * 2u : 0u;
    return {make_rsrc(W, wb), make_rsrc(S, sb), make_rsrc(Mn, sb), wb, sb};
}

// Issue every load of a row batch (rows rb + r*SLOTS + slot, r < U).  Rows
// past n read zeros (buffer range check); units past the row, and the whole
// batch when `batch_live` is false, read nothing: their offsets point at the
// end of the buffer.  The loads are unconditional and the scale layout is a
// compile-time choice, so a pipelined loop has no branches around loads and
// the compiler can wait for exactly the batch it is about to use (a load
// issued on only one side of a branch makes it drain the whole queue).
template <int B, int UNIT, int LPR, int XC, int U, bool WIDE>
__device__ __forceinline__ void load_batch(RowBatch<B, UNIT, XC, U>& bt, const MatRsrc& mr, int rb,
                                           bool batch_live, int wpr, int gpr, int slot,
                                           const int (&unit)[XC], const int (&gidx)[XC], int nu,
                                           int lane) {
    constexpr int SLOTS = 64 / LPR;
    constexpr int WPU = UNIT * B / 32;
    constexpr int ALIGN = unit_align(B, UNIT);
    if constexpr (WIDE && has_affine<B>()) {
        const int words = SLOTS * U * gpr / 2;
        const uint32_t off = (batch_live && lane < words)
                                 ? ((uint32_t)rb * (uint32_t)gpr + 2u * (uint32_t)lane) * 2u
                                 : mr.sbytes;
        bt.sblk = buffer_u32(mr.s, off);
        bt.mblk = buffer_u32(mr.m, off);
    }
#pragma unroll
    for (int r = 0; r < U; ++r) {
        const uint32_t row = (uint32_t)(rb + r * SLOTS + slot);
#pragma unroll
        for (int c = 0; c < XC; ++c) {
            const bool live = batch_live && unit[c] < nu;  // rows past n fall past the end by themselves
            const uint32_t woff = live ? (row * (uint32_t)wpr + (uint32_t)(unit[c] * WPU)) * 4u : mr.wbytes;
            buffer_words<WPU, ALIGN>(mr.w, woff, bt.w[r][c]);
            if constexpr (!WIDE && has_affine<B>()) {
                const uint32_t so = live ? (row * (uint32_t)gpr + (uint32_t)gidx[c]) * 2u : mr.sbytes;
                bt.s[r][c] = buffer_u16(mr.s, so);
                bt.m[r][c] = buffer_u16(mr.m, so);
            }
        }
    }
}

// Partial dot products of a loaded batch, added into yacc[r].
template <int B, int UNIT, int LPR, int XC, int U, bool WIDE>
__device__ __forceinline__ void accumulate_batch(const RowBatch<B, UNIT, XC, U>& bt,
                                                 const XUnit<B, UNIT> (&xu)[XC], float (&yacc)[U],
                                                 int slot, int gpr, const int (&gidx)[XC]) {
    constexpr int SLOTS = 64 / LPR;
#pragma unroll
    for (int r = 0; r < U; ++r)
#pragma unroll
        for (int c = 0; c < XC; ++c) {
            u32 sb = 0, mb = 0;
            if constexpr (!has_affine<B>()) {
            } else if constexpr (!WIDE) {
                sb = bt.s[r][c];
                mb = bt.m[r][c];
            } else {
                // fp16 value number off of the block lives in word off/2, half off%2.
                const int off = (r * SLOTS + slot) * gpr + gidx[c];
                const int src = (off >> 1) << 2;
                const u32 sw = (u32)__builtin_amdgcn_ds_bpermute(src, (int)bt.sblk);
                const u32 mw = (u32)__builtin_amdgcn_ds_bpermute(src, (int)bt.mblk);
                const u32 sh = (off & 1) << 4;
                sb = (sw >> sh) & 0xFFFFu;
                mb = (mw >> sh) & 0xFFFFu;
            }
            const float t = unit_qx<B, UNIT>(bt.w[r][c], xu[c]);
            if constexpr (has_affine<B>())
                yacc[r] = __builtin_fmaf(scale_value<B>(sb), t,
                                         __builtin_fmaf(half_bits_to_float((uint16_t)mb), xu[c].xsum, yacc[r]));
            else
                yacc[r] += t;
        }
}

// Activation units held once per work-group in LDS (XUNIT_LDS_WORDS words
// per unit: the UNIT/2 pair words, the offset constant, the plain sum, two
// words of padding).  A stride of 36 words puts the 16 units that the 16
// lanes of a slot read at distinct bank quadruples, so the 16-byte reads are
// conflict-free; the slots of a wave read the same units (broadcast).
constexpr int XUNIT_LDS_WORDS = 36;
template <int B, int UNIT>
__device__ __forceinline__ void store_xunit_lds(const XUnit<B, UNIT>& xu, u32* dst) {
    static_assert(UNIT / 2 + 2 <= XUNIT_LDS_WORDS, "unit layout");
#pragma unroll
    for (int i = 0; i < UNIT / 2; i += 4)
        *reinterpret_cast<u32x4*>(dst + i) = u32x4{as_u32(xu.xp[i]), as_u32(xu.xp[i + 1]), as_u32(xu.xp[i + 2]),
                                                    as_u32(xu.xp[i + 3])};
    *reinterpret_cast<u32x4*>(dst + UNIT / 2) =
        u32x4{__builtin_bit_cast(u32, xu.corr), __builtin_bit_cast(u32, xu.xsum), 0u, 0u};
}
template <int B, int UNIT>
__device__ __forceinline__ void load_xunit_lds(const u32* src, XUnit<B, UNIT>& xu) {
#pragma unroll
    for (int i = 0; i < UNIT / 2; i += 4) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + i);
        xu.xp[i] = as_h2(v[0]); xu.xp[i + 1] = as_h2(v[1]); xu.xp[i + 2] = as_h2(v[2]); xu.xp[i + 3] = as_h2(v[3]);
    }
    const u32x4 t = *reinterpret_cast<const u32x4*>(src + UNIT / 2);
    // Elements go through plain scalars: this compiler resolves a bit cast
    // of a vector element expression to element 0.
    const u32 c0 = t[0], c1 = t[1];
    xu.corr = __builtin_bit_cast(float, c0);
    xu.xsum = __builtin_bit_cast(float, c1);
}

// accumulate_batch with the lane's activation units read from LDS (xl: the
// work-group's units, unit u at xl + u * XUNIT_LDS_WORDS), one unit at a
// time, so a lane never holds more than one unit's pairs.
template <int B, int UNIT, int LPR, int XC, int U, bool WIDE>
__device__ __forceinline__ void accumulate_batch_lds(const RowBatch<B, UNIT, XC, U>& bt, const u32* xl,
                                                     const int (&unit)[XC], float (&yacc)[U], int slot, int gpr,
                                                     const int (&gidx)[XC]) {
    constexpr int SLOTS = 64 / LPR;
#pragma unroll
    for (int c = 0; c < XC; ++c) {
        XUnit<B, UNIT> xu;
        load_xunit_lds<B, UNIT>(xl + unit[c] * XUNIT_LDS_WORDS, xu);
#pragma unroll
        for (int r = 0; r < U; ++r) {
            u32 sb = 0, mb = 0;
            if constexpr (!has_affine<B>()) {
            } else if constexpr (!WIDE) {
                sb = bt.s[r][c];
                mb = bt.m[r][c];
            } else {
                const int off = (r * SLOTS + slot) * gpr + gidx[c];
                const int src = (off >> 1) << 2;
                const u32 sw = (u32)__builtin_amdgcn_ds_bpermute(src, (int)bt.sblk);
                const u32 mw = (u32)__builtin_amdgcn_ds_bpermute(src, (int)bt.mblk);
                const u32 sh = (off & 1) << 4;
                sb = (sw >> sh) & 0xFFFFu;
                mb = (mw >> sh) & 0xFFFFu;
            }
            const float t = unit_qx<B, UNIT>(bt.w[r][c], xu);
            if constexpr (has_affine<B>())
                yacc[r] = __builtin_fmaf(scale_value<B>(sb), t,
                                         __builtin_fmaf(half_bits_to_float((uint16_t)mb), xu.xsum, yacc[r]));
            else
                yacc[r] += t;
        }
        // One unit's pairs at a time: left alone, the scheduler hoists all
        // three units' reads and the registers they were meant to save.
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Reduce the U row sums over the LPR lanes of each slot and store them.  The
// store is unconditional: lanes with nothing to write aim past the end of y.
template <int LPR, int U>
__device__ __forceinline__ void store_batch(float (&yacc)[U], rsrc_t yr, int rb, int n, int slot,
                                            int j, const float (&res)[U]) {
    constexpr int SLOTS = 64 / LPR;
#pragma unroll
    for (int r = 0; r < U; ++r) {
        const float v = group_sum<LPR>(yacc[r]) + res[r];
        const int row = rb + r * SLOTS + slot;
        buffer_store_f32(v, yr, (j == 0 && row < n) ? (uint32_t)row * 4u : (uint32_t)n * 4u);
    }
}

// Decode GEMV.  Single pass (k <= LPR*XC*UNIT): each wave takes row batches
// wave, wave + waves, ... (all waves read neighbouring rows at a time); the
// activation units stay in registers for the whole kernel, and the loop is
// software-pipelined -- the next row batch's loads are issued before the
// current batch's arithmetic, and the first batch's loads before the
// activation set-up, so memory latency overlaps both.  STG: the same sweep
// through gemv_run, with the row sums staged in LDS and stored outside the
// loop (for 64-lane rows and several batches per wave; a launch with one
// batch per wave pays the staging round trip for nothing).  Multi-pass (MP,
// larger k): each row batch walks k in passes and rebuilds the activation
// units per pass (no pipelining).
//
// The output pointer is restrict-qualified unless the residual may alias it.
template <bool RES>
using out_ptr = std::conditional_t<RES, float*, float* __restrict__>;

// RES: R holds an fp32 residual [n] added to every output (y = r + W x).  It
// may be y itself: each row's residual is read, by the lanes of that row's
// slot, before the row is written.  Without RES, R is ignored and the
// kernel issues no residual loads.
template <int B, int UNIT, int LPR, int XC, int U, bool MP, bool RES = false, bool STG = false, bool LATE = false>
__global__ __launch_bounds__(256) void gemv_kernel(const u32* __restrict__ W,
                                                   const uint16_t* __restrict__ S,
                                                   const uint16_t* __restrict__ Mn,
                                                   const uint16_t* __restrict__ X,
                                                   out_ptr<RES> Y, int n, int k, int group, const float* R) {
    __shared__ float ystage_all[GEMV_WAVES_PER_BLOCK][STG ? YSTAGE : 1];
    // Two or three units per lane: the activation units live in LDS, built
    // once per work-group, instead of each unit's pairs in every lane's
    // registers.
    constexpr bool XL = xunits_in_lds<B, LPR, XC>() && !MP;
    static_assert(!LATE || (XL && !STG), "the late unit build is for the single-pass store-per-batch loop");
    __shared__ __attribute__((aligned(16))) u32 xl_all[XL ? LPR * XC * XUNIT_LDS_WORDS : 4];
    constexpr int SLOTS = 64 / LPR;
    const int lane = threadIdx.x & 63;
    const int slot = lane / LPR, j = lane % LPR;
    constexpr int waves_per_block = GEMV_WAVES_PER_BLOCK;  // every launch: 256 threads
    const int wave = blockIdx.x * waves_per_block + (threadIdx.x >> 6);
    const int nwaves = gridDim.x * waves_per_block;
    const int nu = k / UNIT;
    const int wpr = k / 32 * B;
    const int gpr = div_group(k, group);
    const int stride = nwaves * SLOTS * U;
    const MatRsrc mr = mat_rsrc<B>(W, S, Mn, n, wpr, gpr);
    const rsrc_t xr = make_rsrc(X, (uint32_t)k * 2u);
    const rsrc_t yr = make_rsrc(Y, (uint32_t)n * 4u);
    const rsrc_t rr = make_rsrc(R, RES ? (uint32_t)n * 4u : 0u);
    // The residuals of a batch's rows (zero past n, or without RES).
    auto load_res = [&](int rb, bool live, float (&res)[U]) {
#pragma unroll
        for (int r = 0; r < U; ++r) {
            if constexpr (!RES) {
                res[r] = -0.f;  // x + (-0) is x for every x: the add folds away
                continue;
            }
            const int row = rb + r * SLOTS + slot;
            res[r] = __builtin_bit_cast(float, buffer_u32(rr, (live && row < n) ? (uint32_t)row * 4u : (uint32_t)n * 4u));
        }
    };

    if constexpr (XL && !LATE) {
        // Unit u (< LPR * XC) built by thread u; units past the row are
        // zero.  Every wave reaches the barrier before any exits.  (Issuing
        // the first weight loads before this, as the fused gate/up kernel
        // does, measured slower here but for small Q4 launches, see LATE:
        // 8192 x 3072 5.62 -> 6.24 us, 8192 x 2048 Q2 4.66 -> 4.96, 65536 x
        // 1024 Q8 14.75 -> 15.38.)
        const int u = threadIdx.x;
        if (u < LPR * XC) {
            XUnit<B, UNIT> t;
            prep_xunit<B, UNIT>(xr, u < nu ? (uint32_t)(u * UNIT * 2) : (uint32_t)k * 2u, t);
            store_xunit_lds<B, UNIT>(t, xl_all + u * XUNIT_LDS_WORDS);
        }
        __syncthreads();
    }
    XUnit<B, UNIT> xu[XC];
    int unit[XC], gidx[XC];
    auto units_of_pass = [&](int pass) {
#pragma unroll
        for (int c = 0; c < XC; ++c) {
            unit[c] = (pass * XC + c) * LPR + j;
            gidx[c] = unit[c] < nu ? div_group(unit[c] * UNIT, group) : 0;
        }
    };
    // Units past the row read zeros (offset at the end of x), which gives the
    // all-zero unit state without a branch around the loads.
    auto prep = [&]() {
#pragma unroll
        for (int c = 0; c < XC; ++c)
            prep_xunit<B, UNIT>(xr, unit[c] < nu ? (uint32_t)(unit[c] * UNIT * 2) : (uint32_t)k * 2u, xu[c]);
    };

    // The scale layout is fixed for the whole launch; both variants are
    // compiled and one is chosen here, outside every loop.
    auto body = [&](auto wide_c) {
        constexpr bool WIDE = decltype(wide_c)::value;
        if constexpr (MP) {
            const int passes = (nu + LPR * XC - 1) / (LPR * XC);
            for (int rb = wave * SLOTS * U; rb < n; rb += stride) {
                float yacc[U];
#pragma unroll
                for (int r = 0; r < U; ++r) yacc[r] = 0.f;
                float res[U];
                load_res(rb, true, res);
                for (int pass = 0; pass < passes; ++pass) {
                    units_of_pass(pass);
                    RowBatch<B, UNIT, XC, U> bt;
                    load_batch<B, UNIT, LPR, XC, U, WIDE>(bt, mr, rb, true, wpr, gpr, slot, unit, gidx, nu, lane);
                    prep();
                    accumulate_batch<B, UNIT, LPR, XC, U, WIDE>(bt, xu, yacc, slot, gpr, gidx);
                }
                store_batch<LPR, U>(yacc, yr, rb, n, slot, j, res);
            }
        } else if constexpr (!STG) {
            units_of_pass(0);
            int rb = wave * SLOTS * U;
            if (!LATE && rb >= n) return;
            // LATE (small Q4 launches, one unit per lane): the activation
            // words first, then the first batch's weights; the units are
            // built and shared behind an LDS-only barrier while the weights
            // are in flight, as in the fused gate/up kernel.  Every wave
            // reaches that barrier before any exits.  Measured (Q4): 3072 x
            // 1024 3.47 -> 3.21 us, 1024 x 1024 3.33 -> 3.06, 4096 x 1024
            // 3.53 -> 3.34, 1024 x 2048 3.41 -> 3.16, 151936 x 1024 17.8 ->
            // 17.1.
            const int xb = (int)threadIdx.x < LPR * XC ? (int)threadIdx.x : LPR * XC;
            u32 xw[LATE ? UNIT / 2 : 1];
            if constexpr (LATE) {
                buffer_words<UNIT / 2, 16>(xr, xb < nu ? (uint32_t)(xb * UNIT * 2) : (uint32_t)k * 2u, xw);
                __builtin_amdgcn_sched_barrier(0);
            }
            RowBatch<B, UNIT, XC, U> ba, bb;
            float ra[U], rb_res[U];
            load_batch<B, UNIT, LPR, XC, U, WIDE>(ba, mr, rb, LATE ? rb < n : true, wpr, gpr, slot, unit, gidx, nu,
                                                  lane);
            load_res(rb, LATE ? rb < n : true, ra);
            // The first batch's weight loads go out before the activation
            // set-up arithmetic.
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (LATE) {
                if (xb < LPR * XC) {
                    XUnit<B, UNIT> t;
                    xunit_from_words<B, UNIT>(xw, t);
                    store_xunit_lds<B, UNIT>(t, xl_all + xb * XUNIT_LDS_WORDS);
                }
                lds_barrier();
                if (rb >= n) return;
            } else if constexpr (!XL) {
                prep();
            }
            while (true) {
                float yacc[U];
                int nxt = rb + stride;
                load_batch<B, UNIT, LPR, XC, U, WIDE>(bb, mr, nxt, nxt < n, wpr, gpr, slot, unit, gidx, nu, lane);
                load_res(nxt, nxt < n, rb_res);
#pragma unroll
                for (int r = 0; r < U; ++r) yacc[r] = 0.f;
                if constexpr (XL)
                    accumulate_batch_lds<B, UNIT, LPR, XC, U, WIDE>(ba, xl_all, unit, yacc, slot, gpr, gidx);
                else
                    accumulate_batch<B, UNIT, LPR, XC, U, WIDE>(ba, xu, yacc, slot, gpr, gidx);
                store_batch<LPR, U>(yacc, yr, rb, n, slot, j, ra);
                rb = nxt;
                if (rb >= n) break;
                nxt = rb + stride;
                load_batch<B, UNIT, LPR, XC, U, WIDE>(ba, mr, nxt, nxt < n, wpr, gpr, slot, unit, gidx, nu, lane);
                load_res(nxt, nxt < n, ra);
#pragma unroll
                for (int r = 0; r < U; ++r) yacc[r] = 0.f;
                if constexpr (XL)
                    accumulate_batch_lds<B, UNIT, LPR, XC, U, WIDE>(bb, xl_all, unit, yacc, slot, gpr, gidx);
                else
                    accumulate_batch<B, UNIT, LPR, XC, U, WIDE>(bb, xu, yacc, slot, gpr, gidx);
                store_batch<LPR, U>(yacc, yr, rb, n, slot, j, rb_res);
                rb = nxt;
                if (rb >= n) break;
            }
        }
    };
    if constexpr (STG) {
        // This wave's grid-strided row batches through the pipelined run
        // with its row sums staged in LDS (stores leave the loop).
        constexpr int ROWS = SLOTS * U;
        const int batches = (n + ROWS - 1) / ROWS;
        if (wave >= batches) return;
        const int nb = (batches - wave + nwaves - 1) / nwaves;
        gemv_run<B, UNIT, LPR, XC, U, RES, XL>(W, S, Mn, X, Y, n, k, group, 0, nb, lane,
                                               ystage_all[threadIdx.x >> 6], wave, nwaves, R, xl_all);
    } else if (wide_scales_ok<LPR, U>(S, Mn, gpr)) {
        body(std::true_type{});
    } else {
        body(std::false_type{});
    }
}

// Fused gate/up projection of a feed-forward block: h[n] = silu(g[n]) * u[n]
// with g = Wg x, u = Wu x and silu(v) = v / (1 + e^-v), both matrices N x K in
// one format.  Kernel fusion removes a launch and a global-memory round trip
// ("BaseRT claims fastest Apple Silicon inference", section "What BaseRT does
// differently"; gist.science summary, section "Metodologia", item "Fusão e
// Especialização de Kernel": operator sequences of feed-forward blocks run as
// one kernel).  Each row batch is loaded from both matrices (same row index),
// so g and u meet in registers and only h is written.  The loop is the
// single-pass pipelined loop of the decode GEMV (k <= LPR * XC * UNIT).
template <int LPR>
__device__ __forceinline__ void store_glu(float g, float u, rsrc_t hr, int rb, int n, int slot, int j) {
    const float gs = group_sum<LPR>(g), us = group_sum<LPR>(u);
    const float h = gs / (1.0f + expf(-gs)) * us;
    const int row = rb + slot;
    buffer_store_f32(h, hr, (j == 0 && row < n) ? (uint32_t)row * 4u : (uint32_t)n * 4u);
}

template <int B, int UNIT, int LPR, int XC>
__global__ __launch_bounds__(256) void gemv_glu_kernel(
    const u32* __restrict__ Wg, const uint16_t* __restrict__ Sg, const uint16_t* __restrict__ Mg,
    const u32* __restrict__ Wu, const uint16_t* __restrict__ Su, const uint16_t* __restrict__ Mu,
    const uint16_t* __restrict__ X, float* __restrict__ H, int n, int k, int group) {
    constexpr int SLOTS = 64 / LPR;
    const int lane = threadIdx.x & 63;
    const int slot = lane / LPR, j = lane % LPR;
    constexpr int waves_per_block = GEMV_WAVES_PER_BLOCK;  // every launch: 256 threads
    const int wave = blockIdx.x * waves_per_block + (threadIdx.x >> 6);
    const int nwaves = gridDim.x * waves_per_block;
    const int nu = k / UNIT;
    const int wpr = k / 32 * B;
    const int gpr = div_group(k, group);
    const int stride = nwaves * SLOTS;
    const MatRsrc mg = mat_rsrc<B>(Wg, Sg, Mg, n, wpr, gpr);
    const MatRsrc mu = mat_rsrc<B>(Wu, Su, Mu, n, wpr, gpr);
    const rsrc_t xr = make_rsrc(X, (uint32_t)k * 2u);
    const rsrc_t hr = make_rsrc(H, (uint32_t)n * 4u);
    int unit[XC], gidx[XC];
#pragma unroll
    for (int c = 0; c < XC; ++c) {
        unit[c] = c * LPR + j;
        gidx[c] = unit[c] < nu ? div_group(unit[c] * UNIT, group) : 0;
    }
    XUnit<B, UNIT> xu[XC];
    // Activation units in LDS, built once per work-group, where the single
    // GEMV keeps them there (the same layouts; one spare unit, see below).
    // Every wave reaches the barrier before any exits.  Measured (Q4 unless named, two matrices,
    // cache-busted): 3072 x 1024 4.60 -> 4.00 us, 8192 x 2048 7.22 -> 6.67,
    // 3072 x 8192 10.71 -> 8.73, 14336 x 4096 15.00 -> 14.64; 8192 x 3072 on
    // 16 x 3 rows instead of 64 x 1, Q4 9.27 -> 8.75, Q2 8.81 -> 6.94.
    constexpr bool XL = xunits_in_lds<B, LPR, XC>();
    __shared__ __attribute__((aligned(16))) u32 xl_all[XL ? (LPR * XC + 1) * XUNIT_LDS_WORDS : 4];

    auto body = [&](auto wide_c) {
        constexpr bool WIDE = decltype(wide_c)::value;
        using RB = RowBatch<B, UNIT, XC, 1>;
        int rb = wave * SLOTS;
        if (!XL && rb >= n) return;
        // Activation words first, then the weights; the units are built and
        // shared behind an LDS-only barrier while the weights are in flight
        // (loads complete in order, so waiting on the activation words does
        // not wait on the weights).  Every thread builds one unit, those
        // past LPR * XC (zeros, no memory traffic) into a spare slot, so no
        // branch holds a load.  Measured against building the units before
        // any weight load (Q4): 3072 x 1024 3.99 -> 3.77 us, 8192 x 2048 6.72
        // -> 6.44, 8192 x 3072 8.82 -> 8.48, 3072 x 8192 8.80 -> 8.45.
        const int xb = (int)threadIdx.x < LPR * XC ? (int)threadIdx.x : LPR * XC;
        u32 xw[XL ? UNIT / 2 : 1];
        if constexpr (XL) {
            buffer_words<UNIT / 2, 16>(xr, xb < nu ? (uint32_t)(xb * UNIT * 2) : (uint32_t)k * 2u, xw);
            __builtin_amdgcn_sched_barrier(0);
        }
        RB ga, ua, gb, ub;
        load_batch<B, UNIT, LPR, XC, 1, WIDE>(ga, mg, rb, rb < n, wpr, gpr, slot, unit, gidx, nu, lane);
        load_batch<B, UNIT, LPR, XC, 1, WIDE>(ua, mu, rb, rb < n, wpr, gpr, slot, unit, gidx, nu, lane);
        // The first batch's weight loads go out before the activation set-up.
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (XL) {
            XUnit<B, UNIT> t;
            xunit_from_words<B, UNIT>(xw, t);
            store_xunit_lds<B, UNIT>(t, xl_all + xb * XUNIT_LDS_WORDS);
            lds_barrier();
            if (rb >= n) return;
        }
        if constexpr (!XL) {
#pragma unroll
            for (int c = 0; c < XC; ++c)
                prep_xunit<B, UNIT>(xr, unit[c] < nu ? (uint32_t)(unit[c] * UNIT * 2) : (uint32_t)k * 2u, xu[c]);
        }
        auto finish = [&](const RB& g_b, const RB& u_b, int at) {
            float g[1] = {0.f}, u[1] = {0.f};
            if constexpr (XL) {
                accumulate_batch_lds<B, UNIT, LPR, XC, 1, WIDE>(g_b, xl_all, unit, g, slot, gpr, gidx);
                accumulate_batch_lds<B, UNIT, LPR, XC, 1, WIDE>(u_b, xl_all, unit, u, slot, gpr, gidx);
            } else {
                accumulate_batch<B, UNIT, LPR, XC, 1, WIDE>(g_b, xu, g, slot, gpr, gidx);
                accumulate_batch<B, UNIT, LPR, XC, 1, WIDE>(u_b, xu, u, slot, gpr, gidx);
            }
            store_glu<LPR>(g[0], u[0], hr, at, n, slot, j);
        };
        while (true) {
            int nxt = rb + stride;
            load_batch<B, UNIT, LPR, XC, 1, WIDE>(gb, mg, nxt, nxt < n, wpr, gpr, slot, unit, gidx, nu, lane);
            load_batch<B, UNIT, LPR, XC, 1, WIDE>(ub, mu, nxt, nxt < n, wpr, gpr, slot, unit, gidx, nu, lane);
            __builtin_amdgcn_sched_barrier(0);
            finish(ga, ua, rb);
            rb = nxt;
            if (rb >= n) break;
            nxt = rb + stride;
            load_batch<B, UNIT, LPR, XC, 1, WIDE>(ga, mg, nxt, nxt < n, wpr, gpr, slot, unit, gidx, nu, lane);
            load_batch<B, UNIT, LPR, XC, 1, WIDE>(ua, mu, nxt, nxt < n, wpr, gpr, slot, unit, gidx, nu, lane);
            __builtin_amdgcn_sched_barrier(0);
            finish(gb, ub, rb);
            rb = nxt;
            if (rb >= n) break;
        }
    };
    if (wide_scales_ok<LPR, 1>(Sg, Mg, gpr) && wide_scales_ok<LPR, 1>(Su, Mu, gpr))
        body(std::true_type{});
    else
        body(std::false_type{});
}

// Multi-row product over row segments.  Segment e covers activation rows
// [offsets[e], offsets[e+1]) (clamped to [0, m_total]; [0, m_total) when
// offsets is NULL) and multiplies them by weight matrix e of a stack
// (W + e*n*wpr, S/Mn + e*n*gpr).  Only non-empty segments get work, one
// work-group row (blockIdx.y) per batch of MR activation rows, so the host
// can bound the grid by the row count without reading the offsets.  The waves
// of blockIdx.x stride over the weight rows.  Activations are taken MR rows at a time and
// their unit state is built once per MR-batch; each weight unit loaded is then
// used for all MR rows.  Rows whose activation index is out of range produce
// NaN.  Single pass (k <= LPR*XC*UNIT): the weight-row loop is pipelined like
// the decode GEMV, and the first batch's weight loads go out as soon as the
// segment is known, ahead of the activation lookups.
template <int B, int UNIT, int LPR, int XC, int MR, bool WIDE>
__device__ __forceinline__ void accumulate_rows(const RowBatch<B, UNIT, XC, 1>& bt,
                                                const XUnit<B, UNIT> (&xu)[MR][XC],
                                                float (&yacc)[MR], int slot, int gpr,
                                                const int (&gidx)[XC]) {
#pragma unroll
    for (int c = 0; c < XC; ++c) {
        if constexpr (!has_affine<B>()) {
            // No scale or min (none was loaded): the dot product itself.
#pragma unroll
            for (int r = 0; r < MR; ++r) yacc[r] += unit_qx<B, UNIT>(bt.w[0][c], xu[r][c]);
            continue;
        }
        u32 sb, mb;
        if constexpr (!WIDE) {
            sb = bt.s[0][c];
            mb = bt.m[0][c];
        } else {
            const int off = slot * gpr + gidx[c];
            const int src = (off >> 1) << 2;
            const u32 sw = (u32)__builtin_amdgcn_ds_bpermute(src, (int)bt.sblk);
            const u32 mw = (u32)__builtin_amdgcn_ds_bpermute(src, (int)bt.mblk);
            const u32 sh = (off & 1) << 4;
            sb = (sw >> sh) & 0xFFFFu;
            mb = (mw >> sh) & 0xFFFFu;
        }
        const float sf = scale_value<B>(sb), mf = half_bits_to_float((uint16_t)mb);
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            const float t = unit_qx<B, UNIT>(bt.w[0][c], xu[r][c]);
            yacc[r] = __builtin_fmaf(sf, t, __builtin_fmaf(mf, xu[r][c].xsum, yacc[r]));
        }
    }
}

// The same with the activation units in the work-group's LDS copy: unit u of
// activation row r at xl + (r * LPR * XC + u) * XUNIT_LDS_WORDS, read one at a
// time.
template <int B, int UNIT, int LPR, int XC, int MR, bool WIDE>
__device__ __forceinline__ void accumulate_rows_lds(const RowBatch<B, UNIT, XC, 1>& bt, const u32* xl,
                                                    const int (&unit)[XC], float (&yacc)[MR], int slot,
                                                    int gpr, const int (&gidx)[XC]) {
#pragma unroll
    for (int c = 0; c < XC; ++c) {
        u32 sb = 0, mb = 0;
        if constexpr (!has_affine<B>()) {
        } else if constexpr (!WIDE) {
            sb = bt.s[0][c];
            mb = bt.m[0][c];
        } else {
            const int off = slot * gpr + gidx[c];
            const int src = (off >> 1) << 2;
            const u32 sw = (u32)__builtin_amdgcn_ds_bpermute(src, (int)bt.sblk);
            const u32 mw = (u32)__builtin_amdgcn_ds_bpermute(src, (int)bt.mblk);
            const u32 sh = (off & 1) << 4;
            sb = (sw >> sh) & 0xFFFFu;
            mb = (mw >> sh) & 0xFFFFu;
        }
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            XUnit<B, UNIT> xu;
            load_xunit_lds<B, UNIT>(xl + (r * LPR * XC + unit[c]) * XUNIT_LDS_WORDS, xu);
            const float t = unit_qx<B, UNIT>(bt.w[0][c], xu);
            if constexpr (has_affine<B>())
                yacc[r] = __builtin_fmaf(scale_value<B>(sb), t,
                                         __builtin_fmaf(half_bits_to_float((uint16_t)mb), xu.xsum, yacc[r]));
            else
                yacc[r] += t;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

//
// GLU: a second stack (W2, S2, M2, same shapes) is multiplied alongside and
// each output is silu(first) * second -- the gate and up projections of the
// selected experts and their SiLU-gated product in one launch (the fusion of
// qmm_gemv_swiglu applied to expert rows).  Single pass only.
//
// CMB: weighted combine.  Output row p is not stored; instead
// pair_weight[p] * (row p) is added to row pair_token[p] of Y [n_tokens][n]
// with a float atomic add, so the top-k expert outputs of a token land in
// one row (on top of whatever Y held, e.g. the residual stream).  The order
// of the adds into one element is not fixed.  Pairs whose token is outside
// [0, n_tokens) add nothing.
template <int B, int UNIT, int LPR, int XC, int MR, bool MP, bool GLU = false, bool CMB = false>
__global__ __launch_bounds__(256) void gemv_rows_kernel(
    const u32* __restrict__ W, const uint16_t* __restrict__ S, const uint16_t* __restrict__ Mn,
    const u32* __restrict__ W2, const uint16_t* __restrict__ S2, const uint16_t* __restrict__ M2,
    const uint16_t* __restrict__ X, const int32_t* __restrict__ x_rows, int x_count,
    const int32_t* __restrict__ offsets, int n_seg, int m_total, float* __restrict__ Y, int n,
    int k, int group, int pair_bound, const int32_t* __restrict__ pair_token,
    const float* __restrict__ pair_weight, int n_tokens) {
    constexpr int SLOTS = 64 / LPR;
    constexpr int WPU = UNIT * B / 32;
    constexpr int ALIGN = unit_align(B, UNIT);
    const int lane = threadIdx.x & 63;
    const int slot = lane / LPR, j = lane % LPR;
    constexpr int waves_per_block = GEMV_WAVES_PER_BLOCK;  // every launch: 256 threads
    const int wave = blockIdx.x * waves_per_block + (threadIdx.x >> 6);
    const int nwaves = gridDim.x * waves_per_block;
    const int nu = k / UNIT;
    const int wpr = k / 32 * B;
    const int gpr = div_group(k, group);
    const int passes = MP ? (nu + LPR * XC - 1) / (LPR * XC) : 1;
    // The fused gate/up rows keep their activation units in LDS where the
    // single GEMV does: the MR rows' units of the current batch, built once
    // per work-group (all waves of a work-group take the same pairs) and
    // read for both stacks.  Measured on the Qwen3-30B-A3B expert shapes,
    // Q4: 16 tokens 38.5 -> 34.2 us, one token 7.4 -> 7.5 us.  The
    // single-stack rows keep their registers: with units in LDS they ran
    // 2-8 % slower at 16 tokens (the two barriers of every pair
    // synchronise the waves of a work-group, whose pairs are short).
    constexpr bool XL = GLU && !MP && xunits_in_lds<B, LPR, XC>();
    __shared__ __attribute__((aligned(16))) u32 xl_all[XL ? MR * LPR * XC * XUNIT_LDS_WORDS : 4];

    // A work-group row handles one (segment, MR-row batch) pair at a time:
    // target is a rank among the pairs of the non-empty segments, in segment
    // order, so segments with more rows get more work-groups instead of
    // longer ones.  pair_bound is the host's upper bound on the number of
    // pairs; when the grid's y extent is capped below it, each work-group row
    // takes every gridDim.y-th pair.
    auto find = [&](int target, int& e, int& p0, int& p1) {
        e = -1;
        p0 = p1 = 0;
        if (!offsets) {
            if (target * MR < m_total) {
                e = 0;
                p0 = target * MR;
                p1 = min(m_total, p0 + MR);
            }
            return;
        }
        int base = 0;
        for (int e0 = 0; e0 < n_seg && e < 0; e0 += 64) {
            const int ee = e0 + lane;
            int a = 0, b = 0;
            if (ee < n_seg) {
                a = offsets[ee];
                b = offsets[ee + 1];
                a = a < 0 ? 0 : (a > m_total ? m_total : a);
                b = b < a ? a : (b > m_total ? m_total : b);
            }
            const int cnt = (b - a + MR - 1) / MR;
            int incl = cnt;  // inclusive prefix sum over the lanes
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int t = __shfl_up(incl, d, 64);
                if (lane >= d) incl += t;
            }
            const int total = __shfl(incl, 63, 64);
            if (target < base + total) {
                const unsigned long long past = __ballot(base + incl > target);
                const int src = __ffsll((long long)past) - 1;
                const int before = __shfl(incl - cnt, src, 64);
                const int bi = target - base - before;
                e = __shfl(ee, src, 64);
                p0 = __shfl(a, src, 64) + bi * MR;
                p1 = min(__shfl(b, src, 64), p0 + MR);
            }
            base += total;
        }
    };
    for (int target = blockIdx.y; target < pair_bound; target += gridDim.y) {
        int e, p0, p1;
        find(target, e, p0, p1);
        e = uniform(e);
        p0 = uniform(p0);
        p1 = uniform(p1);
        if (e < 0 || p0 >= p1) break;
        const u32* We = W + (size_t)e * n * wpr;
        const uint16_t* Se = S + (size_t)e * n * gpr;
        const uint16_t* Me = Mn + (size_t)e * n * gpr;
        const MatRsrc mr = mat_rsrc<B>(We, Se, Me, n, wpr, gpr);
        // The second stack (GLU only; otherwise an unused copy of the first).
        const u32* We2 = GLU ? W2 + (size_t)e * n * wpr : We;
        const uint16_t* Se2 = GLU ? S2 + (size_t)e * n * gpr : Se;
        const uint16_t* Me2 = GLU ? M2 + (size_t)e * n * gpr : Me;
        const MatRsrc mr2 = mat_rsrc<B>(We2, Se2, Me2, n, wpr, gpr);
        const uint32_t x_bytes = (uint32_t)x_count * (uint32_t)k * 2u;
        const rsrc_t xbuf = make_rsrc(X, x_bytes);
        const uint32_t y_bytes = (uint32_t)(CMB ? n_tokens : m_total) * (uint32_t)n * 4u;
        const rsrc_t yr = make_rsrc(Y, y_bytes);

        // Activation row indices of one MR-batch; out-of-range indices give
        // NaN.  With CMB also each row's token (-1: adds nothing) and weight.
        int xr[MR], tok[MR];
        bool bad[MR];
        float wgt[MR];
        auto rows_of = [&](int pb) {
#pragma unroll
            for (int r = 0; r < MR; ++r) {
                const int p = pb + r;
                const int idx = (p < p1) ? (x_rows ? x_rows[p] : p) : -1;
                bad[r] = (p < p1) && (idx < 0 || idx >= x_count);
                xr[r] = (p < p1 && !bad[r]) ? idx : -1;
                if constexpr (CMB) {
                    const int t = (p < p1) ? pair_token[p] : -1;
                    tok[r] = (t >= 0 && t < n_tokens) ? t : -1;
                    wgt[r] = (p < p1) ? pair_weight[p] : 0.f;
                }
            }
        };
        XUnit<B, UNIT> xu[MR][XC];
        // Missing rows and units read zeros: the all-zero unit state, branch-free.
        auto prep = [&](int pass) {
#pragma unroll
            for (int r = 0; r < MR; ++r)
#pragma unroll
                for (int c = 0; c < XC; ++c) {
                    const int u = (pass * XC + c) * LPR + j;
                    const uint32_t off = (xr[r] >= 0 && u < nu)
                                             ? ((uint32_t)xr[r] * (uint32_t)k + (uint32_t)(u * UNIT)) * 2u
                                             : x_bytes;
                    prep_xunit<B, UNIT>(xbuf, off, xu[r][c]);
                }
        };
        auto store_rows = [&](float (&yacc)[MR], int pb, int row) {
#pragma unroll
            for (int r = 0; r < MR; ++r) {
                const float sum = group_sum<LPR>(yacc[r]);
                const float v = bad[r] ? __builtin_nanf("") : sum;
                const int p = pb + r;
                if constexpr (CMB) {
                    const bool ok = j == 0 && row < n && tok[r] >= 0;
                    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
                        wgt[r] * v, yr, ok ? ((uint32_t)tok[r] * (uint32_t)n + (uint32_t)row) * 4u : y_bytes, 0, 0);
                } else {
                    const bool ok = j == 0 && row < n && p < p1;
                    buffer_store_f32(v, yr, ok ? ((uint32_t)p * (uint32_t)n + (uint32_t)row) * 4u : y_bytes);
                }
            }
        };
        auto store_rows_glu = [&](float (&gacc)[MR], float (&uacc)[MR], int pb, int row) {
#pragma unroll
            for (int r = 0; r < MR; ++r) {
                const float g = group_sum<LPR>(gacc[r]), u = group_sum<LPR>(uacc[r]);
                const float v = g / (1.0f + expf(-g)) * u;
                const int p = pb + r;
                const bool ok = j == 0 && row < n && p < p1;
                buffer_store_f32(bad[r] ? __builtin_nanf("") : v, yr,
                                 ok ? ((uint32_t)p * (uint32_t)n + (uint32_t)row) * 4u : y_bytes);
            }
        };
        static_assert(!(MP && GLU), "the fused gate/up rows are single-pass only");
        static_assert(!(GLU && CMB), "the combine follows the down projection, not gate/up");

        if constexpr (MP) {
            for (int pb = p0; pb < p1; pb += MR) {
                rows_of(pb);
                for (int rb = wave * SLOTS; rb < n; rb += nwaves * SLOTS) {
                    const int row = rb + slot;
                    float yacc[MR];
#pragma unroll
                    for (int r = 0; r < MR; ++r) yacc[r] = 0.f;
                    for (int pass = 0; pass < passes; ++pass) {
                        prep(pass);
                        u32 wv[XC][WPU];
                        u32 sv[XC], mv[XC];
#pragma unroll
                        for (int c = 0; c < XC; ++c) {
                            const int u = (pass * XC + c) * LPR + j;
                            const bool live = row < n && u < nu;
                            buffer_words<WPU, ALIGN>(mr.w,
                                                     live ? ((uint32_t)row * (uint32_t)wpr + (uint32_t)(u * WPU)) * 4u
                                                          : mr.wbytes,
                                                     wv[c]);
                            const uint32_t so = live ? ((uint32_t)row * (uint32_t)gpr + (uint32_t)div_group(u * UNIT, group)) * 2u
                                                     : mr.sbytes;
                            sv[c] = buffer_u16(mr.s, so);
                            mv[c] = buffer_u16(mr.m, so);
                        }
#pragma unroll
                        for (int r = 0; r < MR; ++r)
#pragma unroll
                            for (int c = 0; c < XC; ++c) {
                                const float t = unit_qx<B, UNIT>(wv[c], xu[r][c]);
                                yacc[r] = __builtin_fmaf(scale_value<B>(sv[c]), t,
                                                         __builtin_fmaf(half_bits_to_float((uint16_t)mv[c]),
                                                                        xu[r][c].xsum, yacc[r]));
                            }
                    }
                    store_rows(yacc, pb, row);
                }
            }
        } else {
            int unit[XC], gidx[XC];
#pragma unroll
            for (int c = 0; c < XC; ++c) {
                unit[c] = c * LPR + j;
                gidx[c] = unit[c] < nu ? div_group(unit[c] * UNIT, group) : 0;
            }
            const int stride = nwaves * SLOTS;
            auto body = [&](auto wide_c) {
                constexpr bool WIDE = decltype(wide_c)::value;
                using RB = RowBatch<B, UNIT, XC, 1>;
                auto load = [&](RB& bt, RB& bt2, int at, bool live) {
                    load_batch<B, UNIT, LPR, XC, 1, WIDE>(bt, mr, at, live, wpr, gpr, slot, unit, gidx, nu, lane);
                    if constexpr (GLU)
                        load_batch<B, UNIT, LPR, XC, 1, WIDE>(bt2, mr2, at, live, wpr, gpr, slot, unit, gidx, nu, lane);
                };
                auto finish = [&](const RB& bt, const RB& bt2, int pb, int row) {
                    float yacc[MR];
#pragma unroll
                    for (int r = 0; r < MR; ++r) yacc[r] = 0.f;
                    if constexpr (XL)
                        accumulate_rows_lds<B, UNIT, LPR, XC, MR, WIDE>(bt, xl_all, unit, yacc, slot, gpr, gidx);
                    else
                        accumulate_rows<B, UNIT, LPR, XC, MR, WIDE>(bt, xu, yacc, slot, gpr, gidx);
                    if constexpr (GLU) {
                        float uacc[MR];
#pragma unroll
                        for (int r = 0; r < MR; ++r) uacc[r] = 0.f;
                        if constexpr (XL)
                            accumulate_rows_lds<B, UNIT, LPR, XC, MR, WIDE>(bt2, xl_all, unit, uacc, slot, gpr, gidx);
                        else
                            accumulate_rows<B, UNIT, LPR, XC, MR, WIDE>(bt2, xu, uacc, slot, gpr, gidx);
                        store_rows_glu(yacc, uacc, pb, row);
                    } else {
                        store_rows(yacc, pb, row);
                    }
                };
                for (int pb = p0; pb < p1; pb += MR) {
                    int rb = wave * SLOTS;
                    // With units in LDS every wave of the work-group takes
                    // part in building them, rows or not.
                    if (!XL && rb >= n) return;
                    RB ba, bb, ba2, bb2;
                    load(ba, ba2, rb, rb < n);
                    __builtin_amdgcn_sched_barrier(0);
                    rows_of(pb);
                    if constexpr (XL) {
                        __syncthreads();  // the previous batch's units are no longer read
                        const int t = threadIdx.x;
                        if (t < MR * LPR * XC) {
                            const int r = t / (LPR * XC), u = t % (LPR * XC);
                            int xrow = xr[0];
#pragma unroll
                            for (int q = 1; q < MR; ++q)
                                if (r == q) xrow = xr[q];
                            const uint32_t off = (xrow >= 0 && u < nu)
                                                     ? ((uint32_t)xrow * (uint32_t)k + (uint32_t)(u * UNIT)) * 2u
                                                     : x_bytes;
                            XUnit<B, UNIT> tu;
                            prep_xunit<B, UNIT>(xbuf, off, tu);
                            store_xunit_lds<B, UNIT>(tu, xl_all + t * XUNIT_LDS_WORDS);
                        }
                        __syncthreads();
                        if (rb >= n) continue;
                    } else {
                        prep(0);
                    }
                    while (true) {
                        int nxt = rb + stride;
                        load(bb, bb2, nxt, nxt < n);
                        finish(ba, ba2, pb, rb + slot);
                        rb = nxt;
                        if (rb >= n) break;
                        nxt = rb + stride;
                        load(ba, ba2, nxt, nxt < n);
                        finish(bb, bb2, pb, rb + slot);
                        rb = nxt;
                        if (rb >= n) break;
                    }
                }
            };
            if (wide_scales_ok<LPR, 1>(Se, Me, gpr) && (!GLU || wide_scales_ok<LPR, 1>(Se2, Me2, gpr)))
                body(std::true_type{});
            else
                body(std::false_type{});
        }
    }
}

// Many independent GEMVs in one launch (same bit width and group size).
// Each descriptor gets its own lane layout, chosen from its K exactly as
// batched_lanes_per_row_host() does on the host: LPR lanes per row (16, 32 or
// 64) with XC units each, so matrices of different K share one launch.  The
// work list is the concatenation, descriptor by descriptor, of each GEMV's
// row batches (64/LPR * U rows each); descriptor d's batches start at item
// D[d].first.  Wave w takes the contiguous item range
// [w*total/nwaves, (w+1)*total/nwaves) -- sizes differ by at most one -- and
// walks it as runs, one per descriptor it touches.  A run is the same
// pipelined loop as the single GEMV with the lane layout fixed at compile
// time; between runs the wave rebuilds its activation units.
template <int XC>
__device__ __forceinline__ int batched_lanes_per_row(int nu) {
    int lpr = 16;
    while (lpr < 64 && lpr * XC < nu) lpr *= 2;
    return lpr;
}


// Row batches [b0, b1) of one matrix (all arguments wave-uniform), with the
// scale layout fixed at compile time; batch b holds rows (base + b * bstride)
// * ROWS onwards (contiguous batches: base 0, bstride 1; a grid-strided
// sweep: base = the wave, bstride = the grid's waves).  ystage: this wave's
// LDS area.  RES: R holds an fp32 residual [n] added to every output at the
// flush (R may be Y: a row's residual is read by the lane that then writes
// the row).
template <int B, int UNIT, int LPR, int XC, int U, bool WIDE, bool RES, bool XL>
__device__ __forceinline__ void gemv_run_w(const u32* W, const uint16_t* S, const uint16_t* Mn,
                                           const uint16_t* X, float* Y, int n, int k, int group,
                                           int b0, int b1, int lane, float* ystage, int base, int bstride,
                                           const float* R, const u32* xl) {
    constexpr int SLOTS = 64 / LPR;
    constexpr int ROWS = SLOTS * U;
    auto row_of = [&](int b) { return (base + b * bstride) * ROWS; };
    const int slot = lane / LPR, j = lane % LPR;
    const int nu = k / UNIT;
    const int wpr = k / 32 * B;
    const int gpr = div_group(k, group);
    const MatRsrc mr = mat_rsrc<B>(W, S, Mn, n, wpr, gpr);
    const rsrc_t xr = make_rsrc(X, (uint32_t)k * 2u);
    const rsrc_t yr = make_rsrc(Y, (uint32_t)n * 4u);
    const rsrc_t rr = make_rsrc(R, RES ? (uint32_t)n * 4u : 0u);
    int unit[XC], gidx[XC];
#pragma unroll
    for (int c = 0; c < XC; ++c) {
        unit[c] = c * LPR + j;
        gidx[c] = unit[c] < nu ? div_group(unit[c] * UNIT, group) : 0;
    }
    RowBatch<B, UNIT, XC, U> ba, bb;
    load_batch<B, UNIT, LPR, XC, U, WIDE>(ba, mr, row_of(b0), true, wpr, gpr, slot, unit, gidx, nu, lane);
    // The first batch's weight loads go out before the activation loads and
    // their set-up arithmetic, which the scheduler would otherwise hoist.
    __builtin_amdgcn_sched_barrier(0);
    // Units past the row read zeros: the all-zero unit state, branch-free.
    XUnit<B, UNIT> xu[XC];
    if constexpr (!XL) {
#pragma unroll
        for (int c = 0; c < XC; ++c)
            prep_xunit<B, UNIT>(xr, unit[c] < nu ? (uint32_t)(unit[c] * UNIT * 2) : (uint32_t)k * 2u, xu[c]);
    }
    // The batch range is wave-uniform; saying so keeps the loop a scalar loop
    // (no per-lane exit masks).
    b0 = uniform(b0);
    b1 = uniform(b1);
    // Batches the staging area takes per flush: even, so that batches go
    // through the loop in pairs with no early exit (an exit in mid-iteration
    // joins the loop's back edge with the next batch's loads still pending,
    // and the compiler then drains the memory queue at the top of every
    // iteration).  For an odd count the pair's second batch lies past the run:
    // it reads zeros, and its staging slot (still inside the area) is never
    // flushed.
    constexpr int CAP = (YSTAGE / ROWS) & ~1;
    static_assert(CAP >= 2, "staging area too small");
    int bf = b0;                        // first batch held in the staging area (uniform)
    // Write batches [bf, be) out: lane l stores staged value l (+64 ...);
    // rows past n get an offset past the end of y and are dropped.
    auto flush = [&](int be) {
        const int cnt = (be - bf) * ROWS;
        for (int i0 = 0; i0 < cnt; i0 += 64) {
            const int i = i0 + lane;
            const int row = row_of(bf + i / ROWS) + i % ROWS;
            float v = ystage[i < YSTAGE ? i : 0];
            const uint32_t off = (i < cnt && row < n) ? (uint32_t)row * 4u : (uint32_t)n * 4u;
            if constexpr (RES) v += __builtin_bit_cast(float, buffer_u32(rr, off));
            buffer_store_f32(v, yr, off);
        }
        bf = be;
    };
    // Every lane of a slot holds its row's sum, so all of them write it (the
    // same value to the same word): no branch.
    auto finish = [&](const RowBatch<B, UNIT, XC, U>& bt, int b) {
        float yacc[U];
#pragma unroll
        for (int r = 0; r < U; ++r) yacc[r] = 0.f;
        if constexpr (XL)
            accumulate_batch_lds<B, UNIT, LPR, XC, U, WIDE>(bt, xl, unit, yacc, slot, gpr, gidx);
        else
            accumulate_batch<B, UNIT, LPR, XC, U, WIDE>(bt, xu, yacc, slot, gpr, gidx);
#pragma unroll
        for (int r = 0; r < U; ++r) ystage[(b - bf) * ROWS + r * SLOTS + slot] = group_sum<LPR>(yacc[r]);
    };
    // The run goes in chunks of CAP batches: a pipelined loop without any
    // store, then one flush.  (A store inside the loop, even a conditional
    // one, makes the compiler drain the memory queue at the top of every
    // iteration.)  The scheduling barriers keep each batch's loads ahead of
    // the previous batch's arithmetic; left alone, the scheduler moves them
    // below it and only one batch is ever in flight.  A loop's last load
    // fetches the next chunk's first batch, so the flush overlaps it.
    for (int c0 = b0; c0 < b1; c0 += CAP) {
        const int c1 = c0 + CAP < b1 ? c0 + CAP : b1;
        for (int b = c0; b < c1; b += 2) {
            load_batch<B, UNIT, LPR, XC, U, WIDE>(bb, mr, row_of(b + 1), b + 1 < b1, wpr, gpr, slot, unit, gidx, nu, lane);
            __builtin_amdgcn_sched_barrier(0);
            finish(ba, b);
            load_batch<B, UNIT, LPR, XC, U, WIDE>(ba, mr, row_of(b + 2), b + 2 < b1, wpr, gpr, slot, unit, gidx, nu, lane);
            __builtin_amdgcn_sched_barrier(0);
            finish(bb, b + 1);
        }
        flush(c1);
    }
}

template <int B, int UNIT, int LPR, int XC, int U, bool RES, bool XLDS>
__device__ __forceinline__ void gemv_run(const u32* W, const uint16_t* S, const uint16_t* Mn,
                                         const uint16_t* X, float* Y, int n, int k, int group, int b0,
                                         int b1, int lane, float* ystage, int base, int bstride,
                                         const float* R, const u32* xl) {
    if (wide_scales_ok<LPR, U>(S, Mn, div_group(k, group)))
        gemv_run_w<B, UNIT, LPR, XC, U, true, RES, XLDS>(W, S, Mn, X, Y, n, k, group, b0, b1, lane, ystage,
                                                         base, bstride, R, xl);
    else
        gemv_run_w<B, UNIT, LPR, XC, U, false, RES, XLDS>(W, S, Mn, X, Y, n, k, group, b0, b1, lane, ystage,
                                                          base, bstride, R, xl);
}

template <int B, int UNIT, int XC, int U>
__global__ __launch_bounds__(256) void gemv_batched_kernel(BatchCoarse coarse, const BatchDesc* __restrict__ D,
                                                           int count, int per_wave, int extra, int group,
                                                           int stride) {
    (void)coarse;  // read through the kernel-argument segment pointer below
    __shared__ float ystage_all[GEMV_WAVES_PER_BLOCK][YSTAGE];
    const int lane = threadIdx.x & 63;
    // The coarse index loads depend on nothing, so they go out first.
    typedef const __attribute__((address_space(4))) int kernarg_int;
    kernarg_int* kc = (kernarg_int*)__builtin_amdgcn_kernarg_segment_ptr();
    int ci[BATCH_COARSE / 64];
#pragma unroll
    for (int r = 0; r < BATCH_COARSE / 64; ++r) ci[r] = kc[64 * r + lane];
    constexpr int waves_per_block = GEMV_WAVES_PER_BLOCK;  // every launch: 256 threads
    const int wave = blockIdx.x * waves_per_block + (threadIdx.x >> 6);
    float* ystage = ystage_all[threadIdx.x >> 6];
    // Items [i0, i1): per_wave = total / waves, and the first extra = total
    // mod waves waves take one more (32-bit arithmetic, no division).
    const int i0 = per_wave * wave + (wave < extra ? wave : extra);
    const int i1 = i0 + per_wave + (wave < extra ? 1 : 0);

    // Last descriptor whose first item is <= i0.  The coarse index (every
    // stride-th descriptor's first item) is the kernel's first argument:
    // lanes read it straight from the argument segment, with loads that
    // depend on nothing, so they overlap the waves' own argument loads.
    // Counting the entries <= i0 (non-decreasing, entry 0 is 0) gives the
    // coarse block; one round of 64 lanes then reads the stride candidate
    // descriptors of that block whole, so the chosen one needs no further
    // load.  (One dependent descriptor load before the first weight load,
    // where a search over the descriptors in memory took two.)  A block
    // wider than 64 descriptors is finished by the forward walk below.
    int below = 0;
#pragma unroll
    for (int r = 0; r < BATCH_COARSE / 64; ++r) below += __popcll(__ballot(ci[r] <= i0));
    // (The exit of waves without items comes after the compare, so that the
    // compiler keeps the coarse loads at the top instead of sinking them.)
    if (i0 >= i1) return;
    const int S = stride;
    const int base = (below - 1) * S;
    const bool in2 = lane < S && base + lane < count;
    const BatchDesc cand = D[in2 ? base + lane : base];
    const uint64_t m2 = __ballot(in2 && cand.first <= i0);
    const int win = uniform(63 - __clzll((long long)m2));
    int d = base + win;
    // Descriptor fields are made explicitly wave-uniform: the table is read
    // through the vector path (the kernel writes memory), and the values feed
    // buffer resources that must live in scalar registers.
    auto lane_u64 = [&](uint64_t v) -> uint64_t {
        const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, win);
        const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), win);
        return ((uint64_t)hi << 32) | lo;
    };
    BatchDesc bd;
    bd.w = reinterpret_cast<const u32*>(lane_u64(reinterpret_cast<uint64_t>(cand.w)));
    bd.s = reinterpret_cast<const uint16_t*>(lane_u64(reinterpret_cast<uint64_t>(cand.s)));
    bd.m = reinterpret_cast<const uint16_t*>(lane_u64(reinterpret_cast<uint64_t>(cand.m)));
    bd.x = reinterpret_cast<const uint16_t*>(lane_u64(reinterpret_cast<uint64_t>(cand.x)));
    bd.y = reinterpret_cast<float*>(lane_u64(reinterpret_cast<uint64_t>(cand.y)));
    bd.n = (int64_t)lane_u64((uint64_t)cand.n);
    bd.k = (int64_t)lane_u64((uint64_t)cand.k);
    bd.first = (int64_t)lane_u64((uint64_t)cand.first);
    int64_t i = i0;
    while (true) {
        const int n = (int)bd.n, k = (int)bd.k;
        const int64_t first = bd.first;
        const int lpr = batched_lanes_per_row<XC>(k / UNIT);
        const int rows = (64 / lpr) * U;
        const int64_t end = first + (n + rows - 1) / rows;
        if (i < end) {
            const int b0 = (int)(i - first);
            const int b1 = (int)((i1 < end ? i1 : end) - first);
            if (lpr == 16)
                gemv_run<B, UNIT, 16, XC, U, false>(bd.w, bd.s, bd.m, bd.x, bd.y, n, k, group, b0, b1, lane, ystage,
                                                    0, 1, nullptr);
            else if (lpr == 32)
                gemv_run<B, UNIT, 32, XC, U, false>(bd.w, bd.s, bd.m, bd.x, bd.y, n, k, group, b0, b1, lane, ystage,
                                                    0, 1, nullptr);
            else
                gemv_run<B, UNIT, 64, XC, U, false>(bd.w, bd.s, bd.m, bd.x, bd.y, n, k, group, b0, b1, lane, ystage,
                                                    0, 1, nullptr);
            i = first + b1;
        }
        if (++d >= count || i >= i1) break;
        const BatchDesc& nx = D[d];
        bd.w = uniform(nx.w);
        bd.s = uniform(nx.s);
        bd.m = uniform(nx.m);
        bd.x = uniform(nx.x);
        bd.y = uniform(nx.y);
        bd.n = uniform((int)nx.n);
        bd.k = uniform((int)nx.k);
        bd.first = uniform(nx.first);
    }
}

// ---- launch templates (instantiated per bit width in gemv_bits.hip) -----------

template <auto Kernel>
hipError_t launch_gemv_k(const GemvArgs& a, const GemvShape& sh, hipStream_t st) {
    const int grid = persistent_grid(sh.work, sh.cus, blocks_per_cu<Kernel>(), sh.waves_per_cu);
    hipLaunchKernelGGL(Kernel, dim3(grid), dim3(64 * GEMV_WAVES_PER_BLOCK), 0, st, a.w, a.s, a.m, a.x, a.y, a.n, a.k, a.group, a.r);
    return hipGetLastError();
}

template <int B, int UNIT, int LPR, int XC, int U>
hipError_t launch_gemv_t(const GemvArgs& a, const GemvShape& sh, hipStream_t st) {
    if (sh.multipass) {
        if (a.r) return launch_gemv_k<gemv_kernel<B, UNIT, LPR, XC, U, true, true>>(a, sh, st);
        return launch_gemv_k<gemv_kernel<B, UNIT, LPR, XC, U, true, false>>(a, sh, st);
    }
    if constexpr (LPR == 64 || (LPR == 16 && XC == 3)) {
        if (sh.staged) {
            if (a.r) return launch_gemv_k<gemv_kernel<B, UNIT, LPR, XC, U, false, true, true>>(a, sh, st);
            return launch_gemv_k<gemv_kernel<B, UNIT, LPR, XC, U, false, false, true>>(a, sh, st);
        }
    }
    if constexpr (B == 4 && LPR <= 32 && XC == 1 && xunits_in_lds<B, LPR, XC>()) {
        if (sh.late) {
            if (a.r) return launch_gemv_k<gemv_kernel<B, UNIT, LPR, XC, U, false, true, false, true>>(a, sh, st);
            return launch_gemv_k<gemv_kernel<B, UNIT, LPR, XC, U, false, false, false, true>>(a, sh, st);
        }
    }
    if (a.r) return launch_gemv_k<gemv_kernel<B, UNIT, LPR, XC, U, false, true>>(a, sh, st);
    return launch_gemv_k<gemv_kernel<B, UNIT, LPR, XC, U, false, false>>(a, sh, st);
}

template <int B, int UNIT, int XC, int U>
hipError_t launch_batched_t(const BatchArgs& a, const GemvShape& sh, hipStream_t st) {
    constexpr auto kern = gemv_batched_kernel<B, UNIT, XC, U>;
    const int grid = persistent_grid(sh.work, sh.cus, blocks_per_cu<kern>(), sh.waves_per_cu);
    const int64_t waves = (int64_t)grid * GEMV_WAVES_PER_BLOCK;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * GEMV_WAVES_PER_BLOCK), 0, st, a.coarse, a.descs, a.count, (int)(a.total_items / waves),
                       (int)(a.total_items % waves), a.group, a.stride);
    return hipGetLastError();
}

// The grid is (row chunks, active segments); the row chunks of all segments
// together are capped at what the GPU holds resident, so every wave starts at
// once and loops over its rows instead of queueing behind other work-groups.
template <auto Kernel>
inline dim3 rows_grid(const RowsShape& sh) {
    const int64_t resident = (int64_t)sh.cus * (sh.waves_per_cu > 0 ? sh.waves_per_cu / 4 : blocks_per_cu<Kernel>());
    int64_t gx = resident / (sh.grid_y > 0 ? sh.grid_y : 1);
    if (gx > sh.grid_x) gx = sh.grid_x;
    if (gx < 1) gx = 1;
    return dim3((unsigned)gx, (unsigned)sh.grid_y);
}

template <auto Kernel>
hipError_t launch_rows_k(const RowsArgs& a, const RowsShape& sh, hipStream_t st, bool second_stack) {
    hipLaunchKernelGGL(Kernel, rows_grid<Kernel>(sh), dim3(64 * GEMV_WAVES_PER_BLOCK), 0, st, a.w, a.s, a.m,
                       second_stack ? a.w2 : a.w, second_stack ? a.s2 : a.s, second_stack ? a.m2 : a.m, a.x,
                       a.x_rows, a.x_count, a.offsets, a.n_seg, a.m_total, a.y, a.n, a.k, a.group, sh.pairs,
                       a.pair_token, a.pair_weight, a.n_tokens);
    return hipGetLastError();
}

template <int B, int UNIT, int LPR, int XC, int MR>
hipError_t launch_rows_t(const RowsArgs& a, const RowsShape& sh, hipStream_t st) {
    if (a.w2) {
        if (sh.multipass) return hipErrorInvalidValue;  // the host rejects this before
        return launch_rows_k<gemv_rows_kernel<B, UNIT, LPR, XC, MR, false, true>>(a, sh, st, true);
    }
    if (a.pair_token) {
        if (sh.multipass) return launch_rows_k<gemv_rows_kernel<B, UNIT, LPR, XC, MR, true, false, true>>(a, sh, st, false);
        return launch_rows_k<gemv_rows_kernel<B, UNIT, LPR, XC, MR, false, false, true>>(a, sh, st, false);
    }
    if (sh.multipass) return launch_rows_k<gemv_rows_kernel<B, UNIT, LPR, XC, MR, true>>(a, sh, st, false);
    return launch_rows_k<gemv_rows_kernel<B, UNIT, LPR, XC, MR, false>>(a, sh, st, false);
}

template <int B, int UNIT, int LPR, int XC>
hipError_t launch_glu_t(const GluArgs& a, const GemvShape& sh, hipStream_t st) {
    constexpr auto kern = gemv_glu_kernel<B, UNIT, LPR, XC>;
    const int grid = persistent_grid(sh.work, sh.cus, blocks_per_cu<kern>(), sh.waves_per_cu);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * GEMV_WAVES_PER_BLOCK), 0, st, a.wg, a.sg, a.mg, a.wu, a.su, a.mu, a.x, a.h,
                       a.n, a.k, a.group);
    return hipGetLastError();
}

template <int B, int UNIT>
hipError_t launch_glu_unit(const GluArgs& a, const GemvShape& sh, hipStream_t st) {
#define X(L, C) \
    if (sh.lpr == L && sh.xc == C) return launch_glu_t<B, UNIT, L, C>(a, sh, st);
    QMM_GLU_SHAPES(X)
#undef X
    return hipErrorInvalidValue;
}

template <int B, int UNIT>
hipError_t launch_gemv_unit(const GemvArgs& a, const GemvShape& sh, hipStream_t st) {
#define X(L, C, UU) \
    if (sh.lpr == L && sh.xc == C && sh.u == UU) return launch_gemv_t<B, UNIT, L, C, UU>(a, sh, st);
    QMM_GEMV_SHAPES(X)
#undef X
    return hipErrorInvalidValue;
}

template <int B, int UNIT>
hipError_t launch_batched_unit(const BatchArgs& a, const GemvShape& sh, hipStream_t st) {
#define X(C, UU) \
    if (sh.xc == C && sh.u == UU) return launch_batched_t<B, UNIT, C, UU>(a, sh, st);
    QMM_BATCHED_SHAPES(X)
#undef X
    return hipErrorInvalidValue;
}

template <int B, int UNIT>
hipError_t launch_rows_unit(const RowsArgs& a, const RowsShape& sh, hipStream_t st) {
#define X(L, C, R) \
    if (sh.lpr == L && sh.xc == C && sh.mr == R) return launch_rows_t<B, UNIT, L, C, R>(a, sh, st);
    QMM_ROWS_SHAPES(X)
#undef X
    return hipErrorInvalidValue;
}

}  // namespace qmm
