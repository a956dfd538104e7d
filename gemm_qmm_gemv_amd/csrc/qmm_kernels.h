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
};

struct GemvShape {
    int unit;       // codes per unit: 64 or 32
    int lpr;        // lanes per row
    int xc;         // units per lane per pass
    int u;          // rows per slot per iteration
    bool multipass; // k > lpr * xc * unit
    int grid;       // work-groups of 256 threads
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
};

struct RowsShape {
    int unit, lpr, xc, mr;
    bool multipass;
    int grid_x, grid_y;
};

struct GemmArgs {
    const uint32_t* w;
    const uint16_t* s;
    const uint16_t* m;
    const uint16_t* x;
    float* y;
    float* partial;  // split-K partial sums [split][m][n], or null when split == 1
    int m_rows, n, k, group, bits;
};

struct GemmShape {
    int tile_m, tile_n;
    int split;        // K split
    int k_tiles_per_split;
    int grid_m, grid_n;
};

hipError_t launch_gemv(const GemvArgs& a, const GemvShape& sh, hipStream_t st);
bool gemv_shape_supported(int lpr, int xc, int u);

hipError_t launch_rows(const RowsArgs& a, const RowsShape& sh, hipStream_t st);
bool rows_shape_supported(int lpr, int xc, int mr);

hipError_t launch_gemm(const GemmArgs& a, const GemmShape& sh, hipStream_t st);
constexpr int GEMM_BK = 64;  // K per main-loop step

hipError_t launch_unpack(const uint32_t* w, uint8_t* codes, int64_t n, int64_t k, int bits,
                         hipStream_t st);

}  // namespace qmm
