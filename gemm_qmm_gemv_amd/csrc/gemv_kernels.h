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
//   with cross-lane shuffles; no atomics, so results are deterministic.
#pragma once

#include "qmm_device.h"
#include "qmm_kernels.h"

namespace qmm {

// K fits in one pass (k <= LPR*XC*UNIT): activations stay in registers for the
// whole kernel.  Otherwise (MP) each row batch walks K in passes and rebuilds
// the activation units per pass.
template <int B, int UNIT, int LPR, int XC, int U, bool MP>
__global__ __launch_bounds__(256) void gemv_kernel(const u32* __restrict__ W,
                                                   const uint16_t* __restrict__ S,
                                                   const uint16_t* __restrict__ Mn,
                                                   const uint16_t* __restrict__ X,
                                                   float* __restrict__ Y, int n, int k, int group) {
    constexpr int SLOTS = 64 / LPR;
    constexpr int WPU = UNIT * B / 32;
    constexpr int ALIGN = unit_align(B, UNIT);
    const int lane = threadIdx.x & 63;
    const int slot = lane / LPR, j = lane % LPR;
    const int waves_per_block = blockDim.x >> 6;
    const int wave = blockIdx.x * waves_per_block + (threadIdx.x >> 6);
    const int nwaves = gridDim.x * waves_per_block;
    const int nu = k / UNIT;
    const int wpr = k / 32 * B;
    const int gpr = k / group;
    const int passes = MP ? (nu + LPR * XC - 1) / (LPR * XC) : 1;

    XUnit<B, UNIT> xu[XC];
    int gidx[XC];
    bool uok[XC];

    auto prep = [&](int pass) {
#pragma unroll
        for (int c = 0; c < XC; ++c) {
            const int u = (pass * XC + c) * LPR + j;
            uok[c] = u < nu;
            gidx[c] = uok[c] ? (u * UNIT) / group : 0;
            if (uok[c])
                prep_xunit<B, UNIT>(X + (size_t)u * UNIT, xu[c]);
            else
                zero_xunit<B, UNIT>(xu[c]);
        }
    };
    if constexpr (!MP) prep(0);

    for (int rb = wave * SLOTS * U; rb < n; rb += nwaves * SLOTS * U) {
        float yacc[U];
#pragma unroll
        for (int r = 0; r < U; ++r) yacc[r] = 0.f;
        for (int pass = 0; pass < passes; ++pass) {
            if constexpr (MP) prep(pass);
            u32 wv[U][XC][WPU];
            uint16_t sv[U][XC], mv[U][XC];
#pragma unroll
            for (int r = 0; r < U; ++r) {
                const int row = rb + r * SLOTS + slot;
#pragma unroll
                for (int c = 0; c < XC; ++c) {
                    const int u = (pass * XC + c) * LPR + j;
                    if (row < n && uok[c]) {
                        load_words<WPU, ALIGN>(W + (size_t)row * wpr + (size_t)u * WPU, wv[r][c]);
                        sv[r][c] = S[(size_t)row * gpr + gidx[c]];
                        mv[r][c] = Mn[(size_t)row * gpr + gidx[c]];
                    } else {
#pragma unroll
                        for (int i = 0; i < WPU; ++i) wv[r][c][i] = 0u;
                        sv[r][c] = 0;
                        mv[r][c] = 0;
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < U; ++r) {
#pragma unroll
                for (int c = 0; c < XC; ++c) {
                    const float t = unit_qx<B, UNIT>(wv[r][c], xu[c]);
                    const float s = half_bits_to_float(sv[r][c]);
                    const float m = half_bits_to_float(mv[r][c]);
                    yacc[r] = __builtin_fmaf(s, t, __builtin_fmaf(m, xu[c].xsum, yacc[r]));
                }
            }
        }
#pragma unroll
        for (int r = 0; r < U; ++r) {
            const float v = group_sum<LPR>(yacc[r]);
            const int row = rb + r * SLOTS + slot;
            if (j == 0 && row < n) Y[row] = v;
        }
    }
}

// Multi-row product over row segments.  Segment e covers activation rows
// [offsets[e], offsets[e+1]) (clamped to [0, m_total]; [0, m_total) when
// offsets is NULL) and multiplies them by weight matrix e of a stack
// (W + e*n*wpr, S/Mn + e*n*gpr).  Only non-empty segments get work: blockIdx.y
// is a rank among the non-empty segments, so the host can size the grid by
// min(segments, rows) without reading the offsets.  blockIdx.x strides over
// the weight rows.  Activations are taken MR rows at a time and their unit
// state is built once per MR-batch; each weight unit loaded is then used for
// all MR rows.  Rows whose activation index is out of range produce NaN.
template <int B, int UNIT, int LPR, int XC, int MR, bool MP>
__global__ __launch_bounds__(256) void gemv_rows_kernel(
    const u32* __restrict__ W, const uint16_t* __restrict__ S, const uint16_t* __restrict__ Mn,
    const uint16_t* __restrict__ X, const int32_t* __restrict__ x_rows, int x_count,
    const int32_t* __restrict__ offsets, int n_seg, int m_total, float* __restrict__ Y, int n,
    int k, int group) {
    constexpr int SLOTS = 64 / LPR;
    constexpr int WPU = UNIT * B / 32;
    constexpr int ALIGN = unit_align(B, UNIT);
    const int lane = threadIdx.x & 63;
    const int slot = lane / LPR, j = lane % LPR;
    const int waves_per_block = blockDim.x >> 6;
    const int wave = blockIdx.x * waves_per_block + (threadIdx.x >> 6);
    const int nwaves = gridDim.x * waves_per_block;
    const int nu = k / UNIT;
    const int wpr = k / 32 * B;
    const int gpr = k / group;
    const int passes = MP ? (nu + LPR * XC - 1) / (LPR * XC) : 1;

    // Find the segment of rank blockIdx.y among the non-empty ones.
    int e = -1, p0 = 0, p1 = 0;
    if (!offsets) {
        if (blockIdx.y == 0) { e = 0; p1 = m_total; }
    } else {
        const int target = blockIdx.y;
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
            const bool ne = b > a;
            const unsigned long long mask = __ballot(ne);
            const int cnt = __popcll(mask);
            if (target < base + cnt) {
                const int before = __popcll(mask & ((1ull << lane) - 1ull));
                const bool mine = ne && (before == target - base);
                const unsigned long long who = __ballot(mine);
                const int src = __ffsll((long long)who) - 1;
                e = __shfl(ee, src, 64);
                p0 = __shfl(a, src, 64);
                p1 = __shfl(b, src, 64);
            }
            base += cnt;
        }
    }
    if (e < 0 || p0 >= p1) return;
    const u32* We = W + (size_t)e * n * wpr;
    const uint16_t* Se = S + (size_t)e * n * gpr;
    const uint16_t* Me = Mn + (size_t)e * n * gpr;

    for (int pb = p0; pb < p1; pb += MR) {
        int xr[MR];
        bool bad[MR];
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            const int p = pb + r;
            const int idx = (p < p1) ? (x_rows ? x_rows[p] : p) : -1;
            bad[r] = (p < p1) && (idx < 0 || idx >= x_count);
            xr[r] = (p < p1 && !bad[r]) ? idx : -1;
        }
        XUnit<B, UNIT> xu[MR][XC];
        auto prep = [&](int pass) {
#pragma unroll
            for (int r = 0; r < MR; ++r)
#pragma unroll
                for (int c = 0; c < XC; ++c) {
                    const int u = (pass * XC + c) * LPR + j;
                    if (xr[r] >= 0 && u < nu)
                        prep_xunit<B, UNIT>(X + (size_t)xr[r] * k + (size_t)u * UNIT, xu[r][c]);
                    else
                        zero_xunit<B, UNIT>(xu[r][c]);
                }
        };
        if constexpr (!MP) prep(0);
        for (int rb = wave * SLOTS; rb < n; rb += nwaves * SLOTS) {
            const int row = rb + slot;
            float yacc[MR];
#pragma unroll
            for (int r = 0; r < MR; ++r) yacc[r] = 0.f;
            for (int pass = 0; pass < passes; ++pass) {
                if constexpr (MP) prep(pass);
                u32 wv[XC][WPU];
                uint16_t sv[XC], mv[XC];
#pragma unroll
                for (int c = 0; c < XC; ++c) {
                    const int u = (pass * XC + c) * LPR + j;
                    if (row < n && u < nu) {
                        load_words<WPU, ALIGN>(We + (size_t)row * wpr + (size_t)u * WPU, wv[c]);
                        const int g = (u * UNIT) / group;
                        sv[c] = Se[(size_t)row * gpr + g];
                        mv[c] = Me[(size_t)row * gpr + g];
                    } else {
#pragma unroll
                        for (int i = 0; i < WPU; ++i) wv[c][i] = 0u;
                        sv[c] = 0;
                        mv[c] = 0;
                    }
                }
#pragma unroll
                for (int r = 0; r < MR; ++r)
#pragma unroll
                    for (int c = 0; c < XC; ++c) {
                        const float t = unit_qx<B, UNIT>(wv[c], xu[r][c]);
                        yacc[r] = __builtin_fmaf(half_bits_to_float(sv[c]), t,
                                                 __builtin_fmaf(half_bits_to_float(mv[c]), xu[r][c].xsum, yacc[r]));
                    }
            }
#pragma unroll
            for (int r = 0; r < MR; ++r) {
                const float v = group_sum<LPR>(yacc[r]);
                const int p = pb + r;
                if (j == 0 && row < n && p < p1)
                    Y[(size_t)p * n + row] = bad[r] ? __builtin_nanf("") : v;
            }
        }
    }
}

// Many independent GEMVs in one launch (same bit width and group size; every
// K fits one pass).  The work list is the concatenation, descriptor by
// descriptor, of each GEMV's row batches (SLOTS*U rows each); descriptor d's
// batches start at item D[d].first.  Wave w takes the contiguous item range
// [w*per, (w+1)*per), so it changes descriptor rarely; on every change it
// rebuilds its activation units from the new x.
template <int B, int UNIT, int LPR, int XC, int U>
__global__ __launch_bounds__(256) void gemv_batched_kernel(const BatchDesc* __restrict__ D, int count,
                                                           int64_t total, int group) {
    constexpr int SLOTS = 64 / LPR;
    constexpr int WPU = UNIT * B / 32;
    constexpr int ALIGN = unit_align(B, UNIT);
    constexpr int ROWS = SLOTS * U;
    const int lane = threadIdx.x & 63;
    const int slot = lane / LPR, j = lane % LPR;
    const int waves_per_block = blockDim.x >> 6;
    const int wave = blockIdx.x * waves_per_block + (threadIdx.x >> 6);
    const int nwaves = gridDim.x * waves_per_block;
    const int64_t per = (total + nwaves - 1) / nwaves;
    const int64_t i0 = (int64_t)wave * per;
    const int64_t i1 = i0 + per < total ? i0 + per : total;
    if (i0 >= i1) return;

    // Last descriptor whose first item is <= i0 (binary search, wave-uniform).
    int lo = 0, hi = count - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (D[mid].first <= i0) lo = mid; else hi = mid - 1;
    }
    int d = __builtin_amdgcn_readfirstlane(lo);

    BatchDesc cur;
    XUnit<B, UNIT> xu[XC];
    int gidx[XC];
    bool uok[XC];
    int64_t d_end = 0;
    int nu = 0, wpr = 0, gpr = 0, n = 0;
    auto enter = [&](int dd) {
        cur = D[dd];
        n = (int)cur.n;
        const int k = (int)cur.k;
        nu = k / UNIT;
        wpr = k / 32 * B;
        gpr = k / group;
        d_end = cur.first + (cur.n + ROWS - 1) / ROWS;
#pragma unroll
        for (int c = 0; c < XC; ++c) {
            const int u = c * LPR + j;
            uok[c] = u < nu && n > 0;
            gidx[c] = uok[c] ? (u * UNIT) / group : 0;
            if (uok[c])
                prep_xunit<B, UNIT>(cur.x + (size_t)u * UNIT, xu[c]);
            else
                zero_xunit<B, UNIT>(xu[c]);
        }
    };
    enter(d);

    for (int64_t i = i0; i < i1; ++i) {
        while (i >= d_end) enter(++d);
        const int rb = (int)(i - cur.first) * ROWS;
        u32 wv[U][XC][WPU];
        uint16_t sv[U][XC], mv[U][XC];
#pragma unroll
        for (int r = 0; r < U; ++r) {
            const int row = rb + r * SLOTS + slot;
#pragma unroll
            for (int c = 0; c < XC; ++c) {
                const int u = c * LPR + j;
                if (row < n && uok[c]) {
                    load_words<WPU, ALIGN>(cur.w + (size_t)row * wpr + (size_t)u * WPU, wv[r][c]);
                    sv[r][c] = cur.s[(size_t)row * gpr + gidx[c]];
                    mv[r][c] = cur.m[(size_t)row * gpr + gidx[c]];
                } else {
#pragma unroll
                    for (int t = 0; t < WPU; ++t) wv[r][c][t] = 0u;
                    sv[r][c] = 0;
                    mv[r][c] = 0;
                }
            }
        }
        float yacc[U];
#pragma unroll
        for (int r = 0; r < U; ++r) {
            yacc[r] = 0.f;
#pragma unroll
            for (int c = 0; c < XC; ++c) {
                const float t = unit_qx<B, UNIT>(wv[r][c], xu[c]);
                yacc[r] = __builtin_fmaf(half_bits_to_float(sv[r][c]), t,
                                         __builtin_fmaf(half_bits_to_float(mv[r][c]), xu[c].xsum, yacc[r]));
            }
        }
#pragma unroll
        for (int r = 0; r < U; ++r) {
            const float v = group_sum<LPR>(yacc[r]);
            const int row = rb + r * SLOTS + slot;
            if (j == 0 && row < n) cur.y[row] = v;
        }
    }
}

// ---- launch templates (instantiated per bit width in gemv_bits.hip) -----------

template <int B, int UNIT, int LPR, int XC, int U>
hipError_t launch_gemv_t(const GemvArgs& a, const GemvShape& sh, hipStream_t st) {
    if (sh.multipass)
        hipLaunchKernelGGL((gemv_kernel<B, UNIT, LPR, XC, U, true>), dim3(sh.grid), dim3(256), 0, st,
                           a.w, a.s, a.m, a.x, a.y, a.n, a.k, a.group);
    else
        hipLaunchKernelGGL((gemv_kernel<B, UNIT, LPR, XC, U, false>), dim3(sh.grid), dim3(256), 0, st,
                           a.w, a.s, a.m, a.x, a.y, a.n, a.k, a.group);
    return hipGetLastError();
}

template <int B, int UNIT, int LPR, int XC, int U>
hipError_t launch_batched_t(const BatchArgs& a, const GemvShape& sh, hipStream_t st) {
    hipLaunchKernelGGL((gemv_batched_kernel<B, UNIT, LPR, XC, U>), dim3(sh.grid), dim3(256), 0, st,
                       a.descs, a.count, a.total_items, a.group);
    return hipGetLastError();
}

template <int B, int UNIT, int LPR, int XC, int MR>
hipError_t launch_rows_t(const RowsArgs& a, const RowsShape& sh, hipStream_t st) {
    const dim3 grid(sh.grid_x, sh.grid_y);
    if (sh.multipass)
        hipLaunchKernelGGL((gemv_rows_kernel<B, UNIT, LPR, XC, MR, true>), grid, dim3(256), 0, st,
                           a.w, a.s, a.m, a.x, a.x_rows, a.x_count, a.offsets, a.n_seg, a.m_total,
                           a.y, a.n, a.k, a.group);
    else
        hipLaunchKernelGGL((gemv_rows_kernel<B, UNIT, LPR, XC, MR, false>), grid, dim3(256), 0, st,
                           a.w, a.s, a.m, a.x, a.x_rows, a.x_count, a.offsets, a.n_seg, a.m_total,
                           a.y, a.n, a.k, a.group);
    return hipGetLastError();
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
#define X(L, C, UU) \
    if (sh.lpr == L && sh.xc == C && sh.u == UU) return launch_batched_t<B, UNIT, L, C, UU>(a, sh, st);
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
