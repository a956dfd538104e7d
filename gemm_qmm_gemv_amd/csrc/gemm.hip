// gemm.hip -- prefill GEMM with inline dequantization on fp16 matrix cores.
//
// Pages: "BaseRT claims fastest Apple Silicon inference" (thetesserapress.com),
// section "What BaseRT does differently" (GEMM kernels for prefill where
// M > 1, dequantization inside the compute loop); "BaseRT: Best-in-Class LLM
// Inference on Apple Silicon via Native Metal" (gist.science summary),
// section "Metodologia" (tiled prefill GEMM on the GPU's matrix hardware).
//
// Y[M][N] = X[M][K] * W^T with W = s*q + m.  One work-group (4 waves) owns a
// TILE_M x 128 tile of Y and walks its share of K in steps of 64:
//   * the X tile (fp16) is copied to LDS;
//   * the W tile is read packed (b/8 bytes per weight plus one scale and min
//     per 64), dequantized in registers -- exact code, then one fused
//     multiply-add s*q + m rounded once to fp16 -- and written to LDS;
//   * each wave multiplies a (TILE_M/2) x 64 sub-tile with
//     v_mfma_f32_32x32x16_f16, fp32 accumulation.
// The next step's global loads are issued before the current step's matrix
// work, so memory and MFMA overlap.  When the tile grid alone would leave
// compute units idle, K is split across work-groups; partial sums go to a
// caller-provided workspace and a second kernel adds them in split order
// (deterministic, no atomics).  Work-group ids are remapped so that the tiles
// sharing a W column block land on the same XCD (and its L2).
#include "qmm_device.h"
#include "qmm_kernels.h"

namespace qmm {

constexpr int BK = GEMM_BK;   // K per step
constexpr int BN = 128;       // N per work-group
constexpr int PAD = 8;        // halves of padding per LDS row (conflict-free 16-byte reads)
constexpr int LDS_ROW = BK + PAD;

// Dequantize one 32-code chunk (B words) to 32 fp16 values in k order.
template <int B>
__device__ __forceinline__ void dequant_chunk(const u32* w, uint16_t s_bits, uint16_t m_bits,
                                              f16x2 (&out)[16]) {
    using F = PairFmt<B>;
    u32 p[16];
    F::extract(w, p);
    const f16 s = __builtin_bit_cast(f16, s_bits), m = __builtin_bit_cast(f16, m_bits);
    const f16x2 s2 = {s, s}, m2 = {m, m};
    f16x2 wv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const f16 inv = (f16)F::inv_factor(F::acc(i));
        const f16x2 inv2 = {inv, inv};
        const f16 off = (f16)(-1024.0f * F::inv_factor(F::acc(i)));
        const f16x2 off2 = {off, off};
        // (1024 + f q) * (1/f) - 1024/f == q exactly (f a power of two).
        const f16x2 q2 = __builtin_elementwise_fma(as_h2(p[i]), inv2, off2);
        // s*q + m with a single rounding to fp16.
        wv[i] = __builtin_elementwise_fma(q2, s2, m2);
    }
    // Pairs 2t and 2t+1 hold codes (a, b) and (a+1, b+1): regroup to k order.
    f16 h[32];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int a = F::ka(2 * t), b = F::kb(2 * t);
        h[a] = wv[2 * t][0];
        h[a + 1] = wv[2 * t + 1][0];
        h[b] = wv[2 * t][1];
        h[b + 1] = wv[2 * t + 1][1];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) out[i] = f16x2{h[2 * i], h[2 * i + 1]};
}

// TM: 32x32 fragments per wave along M (TILE_M = 64 * TM).
template <int B, int TM>
__global__ __launch_bounds__(256) void gemm_kernel(const u32* __restrict__ W,
                                                   const uint16_t* __restrict__ S,
                                                   const uint16_t* __restrict__ Mn,
                                                   const uint16_t* __restrict__ X,
                                                   float* __restrict__ Y, float* __restrict__ P,
                                                   int M, int N, int K, int group, int grid_m,
                                                   int grid_n, int split, int kt_per_split) {
    constexpr int TILE_M = 64 * TM;
    constexpr int XH = TILE_M * BK / 256;  // halves of X per thread per step
    __shared__ __attribute__((aligned(16))) f16 As[TILE_M * LDS_ROW];
    __shared__ __attribute__((aligned(16))) f16 Bs[BN * LDS_ROW];

    // XCD-aware tile order: the 8 XCDs take contiguous tile ranges.
    const int tiles = grid_m * grid_n * split;
    const int per_xcd = (tiles + 7) / 8;
    const int t = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (t >= tiles) return;
    const int mt = t % grid_m;
    const int ns = t / grid_m;
    const int sk = ns % split;
    const int nt = ns / split;
    const int m0 = mt * TILE_M, n0 = nt * BN;
    const int k_tiles = (K + BK - 1) / BK;
    const int kt0 = sk * kt_per_split;
    const int kt1 = min(k_tiles, kt0 + kt_per_split);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int wpr = K / 32 * B;
    const int gpr = K / group;

    // X loader: thread -> (row, XH consecutive halves).
    const int xrow = tid / (BK / XH);
    const int xcol = (tid % (BK / XH)) * XH;
    // W loader: thread -> (row, 32-code chunk).
    const int wrow = tid >> 1;
    const int wch = tid & 1;

    u32 xr[XH / 2];
    u32 wr[B];
    uint16_t sr = 0, mr = 0;

    auto load_step = [&](int kt) {
        const int kx = kt * BK + xcol;
        const bool xok = (m0 + xrow) < M && kx < K;
        if (xok) {
            load_words<XH / 2, 16>(reinterpret_cast<const u32*>(X + (size_t)(m0 + xrow) * K + kx), xr);
        } else {
#pragma unroll
            for (int i = 0; i < XH / 2; ++i) xr[i] = 0u;
        }
        const int kw = kt * BK + wch * 32;
        const bool wok = (n0 + wrow) < N && kw < K;
        if (wok) {
            load_words<B, unit_align(B, 32)>(W + (size_t)(n0 + wrow) * wpr + (size_t)(kw / 32) * B, wr);
            sr = S[(size_t)(n0 + wrow) * gpr + kw / group];
            mr = Mn[(size_t)(n0 + wrow) * gpr + kw / group];
        } else {
#pragma unroll
            for (int i = 0; i < B; ++i) wr[i] = 0u;
            sr = 0;
            mr = 0;
        }
    };

    f32x16 acc[TM][2];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    if (kt0 < kt1) load_step(kt0);
    for (int kt = kt0; kt < kt1; ++kt) {
        __syncthreads();  // previous step's fragment reads are done
        {
            u32x4* dst = reinterpret_cast<u32x4*>(&As[xrow * LDS_ROW + xcol]);
#pragma unroll
            for (int i = 0; i < XH / 8; ++i)
                dst[i] = u32x4{xr[4 * i], xr[4 * i + 1], xr[4 * i + 2], xr[4 * i + 3]};
            f16x2 wh[16];
            dequant_chunk<B>(wr, sr, mr, wh);
            u32x4* wdst = reinterpret_cast<u32x4*>(&Bs[wrow * LDS_ROW + wch * 32]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                wdst[i] = u32x4{as_u32(wh[4 * i]), as_u32(wh[4 * i + 1]), as_u32(wh[4 * i + 2]),
                                as_u32(wh[4 * i + 3])};
        }
        __syncthreads();
        if (kt + 1 < kt1) load_step(kt + 1);
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int kofs = kk * 16 + 8 * (lane >> 5);
            f16x8 a[TM], b[2];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                a[i] = *reinterpret_cast<const f16x8*>(
                    &As[(wm * TM * 32 + i * 32 + (lane & 31)) * LDS_ROW + kofs]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                b[j] = *reinterpret_cast<const f16x8*>(
                    &Bs[(wn * 64 + j * 32 + (lane & 31)) * LDS_ROW + kofs]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }

    // Store: lane holds column (lane % 32) of each 32x32 fragment, rows
    // 8*(v/4) + 4*(lane/32) + v%4.
    float* out = (split == 1) ? Y : P + (size_t)sk * M * N;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = m0 + wm * TM * 32 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (row < M && col < N) out[(size_t)row * N + col] = acc[i][j][v];
            }
        }
}

// y = sum over splits of the partial sums, in split order.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ P,
                                                            float* __restrict__ Y, int64_t count,
                                                            int split) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= count) return;
    float v = P[i];
    for (int s = 1; s < split; ++s) v += P[(size_t)s * count + i];
    Y[i] = v;
}

template <int B, int TM>
static hipError_t launch_gemm_t(const GemmArgs& a, const GemmShape& sh, hipStream_t st) {
    const int tiles = sh.grid_m * sh.grid_n * sh.split;
    const int grid = 8 * ((tiles + 7) / 8);
    hipLaunchKernelGGL((gemm_kernel<B, TM>), dim3(grid), dim3(256), 0, st, a.w, a.s, a.m, a.x, a.y,
                       a.partial, a.m_rows, a.n, a.k, a.group, sh.grid_m, sh.grid_n, sh.split,
                       sh.k_tiles_per_split);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || sh.split == 1) return err;
    const int64_t count = (int64_t)a.m_rows * a.n;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st,
                       a.partial, a.y, count, sh.split);
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, const GemmShape& sh, hipStream_t st) {
    const bool t2 = sh.tile_m == 128;
    switch (a.bits) {
        case 2: return t2 ? launch_gemm_t<2, 2>(a, sh, st) : launch_gemm_t<2, 1>(a, sh, st);
        case 3: return t2 ? launch_gemm_t<3, 2>(a, sh, st) : launch_gemm_t<3, 1>(a, sh, st);
        case 4: return t2 ? launch_gemm_t<4, 2>(a, sh, st) : launch_gemm_t<4, 1>(a, sh, st);
        case 6: return t2 ? launch_gemm_t<6, 2>(a, sh, st) : launch_gemm_t<6, 1>(a, sh, st);
        case 8: return t2 ? launch_gemm_t<8, 2>(a, sh, st) : launch_gemm_t<8, 1>(a, sh, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
