// qmm_kernels.h -- host-side interface between the C ABI layer (qmm_api.hip)
// and the kernel files.  Internal to the library; not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

struct GemvArgs {
    const uint32_t* w;
    const uint16_t* s;
    const uint16_t* m;
    const uint16_t* x;
    float* y;
    int n, k, group, bits;
    const float* r = nullptr;  // residual added to y (may be y), or null
};

struct GemvShape {
    int unit;           // codes per unit: 64 or 32
    int lpr;            // lanes per row
    int xc;             // units per lane per pass
    int u;              // rows per slot per iteration
    bool multipass;     // k > lpr * xc * unit
    bool staged;        // single pass, row sums staged in LDS (64-lane rows only)
    bool late;          // single pass, activation units built after the first weight loads
    int64_t work;       // row batches (waves that have work)
    int cus;            // compute units of the device
    int waves_per_cu;   // > 0: cap resident waves per CU; 0: the kernel's occupancy
    int grid;           // work-groups of 256 threads (set at launch)
};

// Work-groups for a persistent launch: enough for the work, at most what the
// device holds resident at once (blocks_per_cu from the kernel's occupancy),
// so no wave waits for another to finish before it can start.
inline int persistent_grid(int64_t work_waves, int cus, int blocks_per_cu, int waves_per_cu_override) {
    const int64_t cap = waves_per_cu_override > 0 ? (int64_t)cus * waves_per_cu_override / 4
                                                  : (int64_t)cus * blocks_per_cu;
    int64_t g = (work_waves + 3) / 4;
    if (g > cap) g = cap;
    return g < 1 ? 1 : (int)g;
}

// Resident 256-thread work-groups per CU for a kernel (queried once per
// kernel: the template parameter is the kernel itself).
template <auto Kernel>
inline int blocks_per_cu() {
    static int cached = 0;
    if (cached == 0) {
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(Kernel), 256, 0) !=
                hipSuccess || nb <= 0) {
            (void)hipGetLastError();
            nb = 2;
        }
        cached = nb;
    }
    return cached;
}

// Fused gate/up projection: h = silu(Wg x) * (Wu x).
struct GluArgs {
    const uint32_t* wg;
    const uint16_t* sg;
    const uint16_t* mg;
    const uint32_t* wu;
    const uint16_t* su;
    const uint16_t* mu;
    const uint16_t* x;
    float* h;
    int n, k, group, bits;
};

struct RowsArgs {
    const uint32_t* w;
    const uint16_t* s;
    const uint16_t* m;
    const uint16_t* x;
    const int32_t* x_rows;  // may be null
    int x_count;            // rows of x
    const int32_t* offsets; // may be null (one segment of m_total rows)
    int n_seg;              // segments (experts)
    int m_total;            // output rows
    float* y;
    int n, k, group, bits;
    // Second stack for the fused gate/up rows (y = silu(W x) * (W2 x)); null
    // for a plain product.
    const uint32_t* w2 = nullptr;
    const uint16_t* s2 = nullptr;
    const uint16_t* m2 = nullptr;
    // Weighted combine into y [n_tokens][n] (y[token[p]] += weight[p] * row
    // p); null pair_token for a plain product.
    const int32_t* pair_token = nullptr;
    const float* pair_weight = nullptr;
    int n_tokens = 0;
};

struct RowsShape {
    int unit, lpr, xc, mr;
    bool multipass;
    int grid_x, grid_y;  // grid_x: row chunks wanted per segment (capped at launch)
    int pairs;           // upper bound on (segment, row batch) pairs; grid_y = min(pairs, 65535)
    int cus;
    int waves_per_cu;    // > 0: resident waves per CU the grid assumes; 0: the kernel's occupancy
};

// A grouped GEMM: up to GEMM_GROUP_MAX weight matrices sharing X, M and K
// in one launch.  Their N-tiles are concatenated: member d owns global tiles
// [tile0[d], tile0[d + 1]) and, with a K split, the partial sums from
// column col0[d] of a [split][M][sum of N] area.
constexpr int GEMM_GROUP_MAX = 4;
struct GemmGroupArgs {
    const uint32_t* w[GEMM_GROUP_MAX];
    const uint16_t* s[GEMM_GROUP_MAX];
    const uint16_t* m[GEMM_GROUP_MAX];
    float* y[GEMM_GROUP_MAX];
    int n[GEMM_GROUP_MAX];
    int col0[GEMM_GROUP_MAX];
    int tile0[GEMM_GROUP_MAX + 1];
    int count;
};

struct GemmArgs {
    const uint32_t* w;
    const uint16_t* s;
    const uint16_t* m;
    const uint16_t* x;
    float* y;
    float* partial;  // split-K partial sums [split][m][n], or null when split == 1
    int* counters;   // split-K arrival counter per tile (zero between calls), or null
    int m_rows, n, k, group, bits;
    int out16;       // y holds fp16 [m][n] (else fp32)
    const GemmGroupArgs* grp = nullptr;  // grouped launch (members replace w, s, m, y, n)
};

struct GemmShape {
    int kernel;        // 0: weights dequantized into registers (gemm.hip), 1: into LDS (gemm_wl.hip)
    int tile_m, tile_n;
    int split;        // K split
    int k_tiles_per_split;
    int grid_m, grid_n;
    bool wide_scales;  // 16-byte scale/min loads per four steps (group 64, K % 512 == 0)
    bool n_fast;       // tile order: column tile fastest within an XCD's range
};

// One GEMV of a batched launch.  Same layout as qmm_gemv_desc in qmm.h.
struct BatchDesc {
    const uint32_t* w;
    const uint16_t* s;
    const uint16_t* m;
    const uint16_t* x;
    float* y;
    int64_t n, k;
    int64_t first;  // index of this GEMV's first row batch in the launch's work list
};
static_assert(sizeof(BatchDesc) == 64, "descriptor layout");

// Coarse index of a batched launch's work list, passed by value as the
// kernel's first argument (so it sits at offset 0 of the kernel-argument
// segment, which the waves read at start-up anyway): entry j is the first
// item of descriptor j * stride, INT_MAX past the last descriptor.
constexpr int BATCH_COARSE = 256;
struct BatchCoarse {
    int first[BATCH_COARSE];
};

struct BatchArgs {
    const BatchDesc* descs;  // device memory
    int count;
    int64_t total_items;     // below 2^31
    int group, bits;
    int stride;              // descriptors per coarse entry
    BatchCoarse coarse;
};

// Kernel shapes compiled for each bit width and unit: (lanes per row, units
// per lane, rows per slot) for the GEMV kernels, (lanes, units, activation
// rows) for the multi-row kernel.
#define QMM_GEMV_SHAPES(X) \
    X(16, 1, 1) X(16, 1, 2) X(16, 3, 1) X(16, 3, 2) \
    X(32, 1, 1) X(32, 1, 2) \
    X(64, 1, 1) X(64, 1, 2) \
    X(64, 2, 1)

// Batched launches choose the lanes per row per descriptor at run time;
// compiled shapes are (units per lane, rows per slot).
// (lanes per row, units per lane) of the fused gate/up kernel: single pass,
// one row per slot and iteration (two with both matrices).
#define QMM_GLU_SHAPES(X) X(16, 1) X(16, 3) X(32, 1) X(64, 1) X(64, 2)
constexpr bool glu_shape_supported(int lpr, int xc) {
#define X(L, C) if (lpr == L && xc == C) return true;
    QMM_GLU_SHAPES(X)
#undef X
    return false;
}
#define QMM_BATCHED_SHAPES(X) X(1, 1) X(1, 2) X(2, 1)

// Multi-row kernel: at most two activation units per lane in flight (MR*XC
// <= 2); beyond that the unit state no longer stays in registers.
#define QMM_ROWS_SHAPES(X) \
    X(16, 1, 2) X(32, 1, 2) X(64, 1, 2) \
    X(16, 1, 1) X(32, 1, 1) X(64, 1, 1) X(64, 2, 1) X(32, 2, 1) X(16, 2, 1)

constexpr bool gemv_shape_supported(int lpr, int xc, int u) {
#define X(L, C, UU) if (lpr == L && xc == C && u == UU) return true;
    QMM_GEMV_SHAPES(X)
#undef X
    return false;
}
constexpr bool batched_shape_supported(int xc, int u) {
#define X(C, UU) if (xc == C && u == UU) return true;
    QMM_BATCHED_SHAPES(X)
#undef X
    return false;
}

// Lanes per row a batched launch gives a descriptor with nu units per row
// (the kernel computes the same from K): the smallest of 16, 32, 64 whose
// lanes cover the row with xc units each.
constexpr int batched_lanes_per_row_host(int nu, int xc) {
    int lpr = 16;
    while (lpr < 64 && lpr * xc < nu) lpr *= 2;
    return lpr;
}
constexpr bool rows_shape_supported(int lpr, int xc, int mr) {
#define X(L, C, R) if (lpr == L && xc == C && mr == R) return true;
    QMM_ROWS_SHAPES(X)
#undef X
    return false;
}

// Per-bit-width launchers, each defined in its own translation unit
// (gemv_bits.hip built with -DQMM_BITS=b).
template <int B> hipError_t launch_gemv_bits(const GemvArgs& a, const GemvShape& sh, hipStream_t st);
template <int B> hipError_t launch_batched_bits(const BatchArgs& a, const GemvShape& sh, hipStream_t st);
template <int B> hipError_t launch_rows_bits(const RowsArgs& a, const RowsShape& sh, hipStream_t st);
template <int B> hipError_t launch_glu_bits(const GluArgs& a, const GemvShape& sh, hipStream_t st);
#define QMM_DECLARE_BITS(B)                                                                      \
    template <> hipError_t launch_gemv_bits<B>(const GemvArgs&, const GemvShape&, hipStream_t);  \
    template <> hipError_t launch_batched_bits<B>(const BatchArgs&, const GemvShape&, hipStream_t); \
    template <> hipError_t launch_rows_bits<B>(const RowsArgs&, const RowsShape&, hipStream_t);   \
    template <> hipError_t launch_glu_bits<B>(const GluArgs&, const GemvShape&, hipStream_t);
QMM_DECLARE_BITS(2)
QMM_DECLARE_BITS(3)
QMM_DECLARE_BITS(4)
QMM_DECLARE_BITS(5)
QMM_DECLARE_BITS(6)
QMM_DECLARE_BITS(8)
QMM_DECLARE_BITS(16)
#undef QMM_DECLARE_BITS

hipError_t launch_gemm(const GemmArgs& a, const GemmShape& sh, hipStream_t st);
hipError_t launch_gemm_wl(const GemmArgs& a, const GemmShape& sh, hipStream_t st);
// y = the sum over `split` partial-sum blocks of `count` floats each, in split
// order (fp32, or rounded once to fp16 when out16).
hipError_t launch_splitk_reduce(const float* partial, void* y, int64_t count, int split, int out16,
                                hipStream_t st);
// K per step of the LDS-dequantizing GEMM.
constexpr int gemm_wl_step_codes(int) { return 64; }
// Threads of its work-groups: 64 per consumer wave (4 or 8) plus 4 producer waves.
constexpr int gemm_wl_threads(int tile_m) { return 64 * (tile_m / 64 * 2 + 4); }
#ifndef GEMM_BK_STEP
#define GEMM_BK_STEP 128
#endif
constexpr int GEMM_BK = GEMM_BK_STEP;  // K per main-loop step
// Threads per GEMM work-group: 128 per wave column along N (two waves along
// K); tiles of 64 and 128 rows use GEMM_WN columns, 32-row tiles two.
#ifndef GEMM_WN
#define GEMM_WN 4
#endif
constexpr int gemm_threads(int tile_m) { return 128 * (tile_m == 32 ? 2 : GEMM_WN); }

hipError_t launch_unpack(const uint32_t* w, uint8_t* codes, int64_t n, int64_t k, int bits,
                         hipStream_t st);

}  // namespace qmm
