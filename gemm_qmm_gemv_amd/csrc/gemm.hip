// gemm.hip -- prefill GEMM with inline dequantization on fp16 matrix cores.
//
// Pages: "BaseRT claims fastest Apple Silicon inference" (thetesserapress.com),
// section "What BaseRT does differently" (GEMM kernels for prefill where
// M > 1, dequantization inside the compute loop); "BaseRT: Best-in-Class LLM
// Inference on Apple Silicon via Native Metal" (gist.science summary),
// section "Metodologia" (tiled prefill GEMM on the GPU's matrix hardware).
//
// Y[M][N] = X[M][K] * W^T with W = s*q + m, on v_mfma_f32_32x32x16_f16.
//
// Work-group: tile TILE_M (= 32*MS) x TN of Y, K in steps of 128.  With
// 128-column tiles, eight waves: four along N (32 columns each) times two
// along K (each takes one 64-wide half of every step; the halves are added
// through LDS at the end).  With 256-column tiles, eight waves along N, each
// taking whole steps.
//
//   * W never goes through LDS.  The matrix core's B operand for lane l is
//     eight K values of column l%32, and lanes l and l+32 cover the two
//     K-halves of a 16-deep step.  Each lane therefore loads one 32-code
//     chunk of its own column straight into registers (b words), turns it
//     into sixteen fp16 pairs -- exact code, then s*q + m with one rounding --
//     and feeds four consecutive pairs to each of four MFMA steps.
//   * The pairs come out of the bit tricks in a fixed, format-dependent order
//     (for Q4: codes 0,4 / 1,5 / 2,6 / 3,7 of every eight).  A dot product
//     does not care about the order of its terms, only that both operands use
//     the same one, so X is written to LDS in that same order ("slot order")
//     while it is staged; the W side needs no shuffles at all.
//   * X (fp16) is the shared operand: the work-group copies its TILE_M x 128
//     block to LDS once per step (double-buffered, one barrier per step) and
//     every wave reads 32x16 A fragments from there.
//   * Software pipeline: a step's loads are issued PD steps ahead; each step
//     first stages X for step s + 1, then the matrix core works on step s
//     while the same wave dequantizes W for step s + 1 (no dependence
//     between the two, so VALU and MFMA instructions interleave within the
//     wave instead of alternating between barrier-separated phases).
//
// When the tile grid alone would leave compute units idle, K is split across
// work-groups; partial sums go to a caller-provided workspace and are added
// in split order (deterministic) -- two splits by the last work-group of each
// tile inside this kernel, more by a second kernel.  Work-group ids are
// remapped so that each XCD (and its L2) takes a contiguous range of tiles.
// A grouped launch runs several weight matrices that share X as one grid.
#include "gemm_common.h"

#include <type_traits>

namespace qmm {

constexpr int BK = GEMM_BK;     // K per step
static_assert(BK % 128 == 0, "each of two waves along K takes whole 64-code chunks");
constexpr int BN = 128;         // columns per work-group (default tile width)
constexpr int XPAD = 8;         // halves of padding per LDS row (conflict-free 16-byte reads)
constexpr int XROW = BK + XPAD; // halves per LDS row

// Halves of X reordered as one unit: every format keeps each aligned block
// of XH slots inside the same XH codes, with the same pattern in every block
// of a chunk (XH = 8 except for Q2, whose pairs span 16 codes).
template <int B>
constexpr int x_unit_halves() { return B == 2 ? 16 : 8; }

template <int B>
constexpr bool slot_blocks_ok() {
    constexpr int XH = x_unit_halves<B>();
    for (int p = 0; p < 32; ++p)
        if (slot_k<B>(p) / XH != p / XH || slot_k<B>(p) % XH != slot_k<B>(p % XH)) return false;
    return true;
}
static_assert(slot_blocks_ok<2>() && slot_blocks_ok<3>() && slot_blocks_ok<4>() &&
                  slot_blocks_ok<5>() && slot_blocks_ok<6>() && slot_blocks_ok<8>() &&
                  slot_blocks_ok<16>(),
              "slot order must stay within aligned blocks of x_unit_halves codes");

// XH halves of X in natural k order -> slot order, one byte permute per
// output dword.  v_perm_b32 selector bytes 0-3 pick bytes of its second
// operand and 4-7 bytes of its first.
template <int B>
__device__ __forceinline__ void to_slot_order(const u32 (&in)[x_unit_halves<B>() / 2],
                                              u32 (&out)[x_unit_halves<B>() / 2]) {
#pragma unroll
    for (int d = 0; d < x_unit_halves<B>() / 2; ++d) {
        const int a = slot_k<B>(2 * d), b = slot_k<B>(2 * d + 1);
        const u32 sel = (u32)(2 * (a & 1)) | (u32)(2 * (a & 1) + 1) << 8 |
                        (u32)(4 + 2 * (b & 1)) << 16 | (u32)(4 + 2 * (b & 1) + 1) << 24;
        out[d] = __builtin_amdgcn_perm(in[b >> 1], in[a >> 1], sel);
    }
}

// Prefetch distance (steps between a step's loads and its matrix work) and
// the occupancy target (work-groups per CU the register allocation must
// allow).
#ifndef GEMM_PD
#define GEMM_PD 2
#endif
#ifndef GEMM_MINB
#define GEMM_MINB 2
#endif
constexpr int PD = GEMM_PD;
static_assert(PD >= 2 && PD <= 4, "prefetch distance");
// The main loop is unrolled so that every ring index is a compile-time
// constant: the raw rings have PD slots, the dequantized W and the LDS
// buffers two.
constexpr int UNROLL = PD % 2 ? 2 * PD : PD;
// Wide scale loads (SW): with groups of 64 codes and steps of 128, a lane's
// scales for four consecutive steps are eight consecutive fp16 values of its
// own row (its K-half takes every other group), fetched as one 16-byte load
// for the scales and one for the mins instead of eight 2-byte loads.
constexpr int SW_STEPS = 4;
// With wide scales the loop is unrolled by a multiple of four as well, so a
// block's word index is a compile-time constant.
constexpr int UNROLL_SW = UNROLL % SW_STEPS ? UNROLL * SW_STEPS / (UNROLL % SW_STEPS == 2 ? 2 : 1) : UNROLL;
static_assert(UNROLL_SW % SW_STEPS == 0 && UNROLL_SW % UNROLL == 0, "wide-scale unroll");

// MS: 32-row fragments per wave along M (TILE_M = 32 * MS); WN: waves along
// N (each with TN / WN columns, NS = TN / (32 WN) fragments); KW: waves
// along K (two: each takes one half of every step and the halves are added
// at the end; one: a wave takes whole steps).  The work-group has
// 64 * WN * KW threads and covers TILE_M x TN of Y.
//
// SW: wide scale loads (see SW_STEPS); the host enables it only for groups of
// 64, rows of scales 16-byte aligned (K a multiple of 512) and splits that
// start at multiples of four steps.
// One tile of y = the sum over splits of the partial sums P [split][M][N],
// in split order (fp32, or rounded once to fp16 when out16).  Each thread
// takes up to four 4-column groups at a time and issues the loads of four
// splits for all of them before adding, so the latencies overlap; loads past
// the last split or outside the matrix read zeros, and stores outside it are
// dropped (buffer range checks).  N % 4 != 0 takes single columns.
constexpr int gemm_min_blocks(int wn) { return GEMM_MINB * 2 / wn > 0 ? GEMM_MINB * 2 / wn : 1; }

//
// GRP (grouped launch): W, S, Mn, Y, N and the partial-sum area come from
// the member of `grp` that owns the work-group's N-tile; the plain
// arguments are unused.  Grouped launches reduce K splits in the kernel.
template <int B, int MS, int WN, int KW = 2, int TN = BN, bool SW = false, bool RED = false, bool GRP = false>
__global__ __launch_bounds__(64 * WN * KW, gemm_min_blocks(WN)) void gemm_kernel(const u32* __restrict__ W_arg,
                                                   const uint16_t* __restrict__ S_arg,
                                                   const uint16_t* __restrict__ Mn_arg,
                                                   const uint16_t* __restrict__ X,
                                                   float* __restrict__ Y_arg, float* __restrict__ P_arg,
                                                   int* __restrict__ counters,
                                                   int M, int N_arg, int K, uint64_t gmul, int gsh,
                                                   int grid_m, int grid_n, int split,
                                                   int steps_per_split, int out16, GemmGroupArgs grp,
                                                   int n_fast) {
    constexpr int TILE_M = 32 * MS;
    constexpr int THREADS = 64 * WN * KW;
    constexpr int NS = TN / (32 * WN);                   // 32-column fragments per wave
    constexpr int HK = BK / KW;                          // K per wave and step
    constexpr int CH = HK / 64;                          // 64-code chunks per wave and step
    static_assert(KW == 1 || KW == 2, "one or two waves along K");
    static_assert(NS * 32 * WN == TN && CH * 64 == HK, "tile shape");
    constexpr int NF = MS * NS;                          // fragments per wave
    constexpr int XH = x_unit_halves<B>();               // halves per X unit
    constexpr int XW = XH / 2;                           // dwords per X unit
    constexpr int UPR = BK / XH;                         // X units per row and step
    constexpr int XU = TILE_M * UPR / THREADS;           // X units per thread
    static_assert(NS >= 1 && XU >= 1 && XU * THREADS == TILE_M * UPR, "tile shape");
    constexpr int XBUF = TILE_M * XROW;                  // halves per X buffer
    constexpr int X_BYTES = 2 * XBUF * 2;                // two buffers
    // K-half exchange: every wave hands over half of its fragments (all of
    // them when it has only one).
    constexpr int GIVE = NF > 1 ? NF / 2 : 1;
    constexpr int R_BYTES = KW == 2 ? 2 * WN * GIVE * 16 * 64 * 4 : 0;
    constexpr int LDS_BYTES = X_BYTES > R_BYTES ? X_BYTES : R_BYTES;
    __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_BYTES];
    f16* xs = reinterpret_cast<f16*>(smem);

    // XCD-aware tile order: the 8 XCDs take contiguous tile ranges.
    const int tiles = grid_m * grid_n * split;
    const int per_xcd = (tiles + 7) / 8;
    const int t = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (t >= tiles) return;
    // Each XCD takes a contiguous range of tiles.  With few row tiles the
    // row tile varies fastest (an XCD's tiles share W column blocks in its
    // L2); with many (n_fast) the column tile does, so an XCD's tiles share
    // X rows, which then stay in its L2 while W streams (measured at 2048
    // tokens: -2 to -9 % on the 2048- and 512-column shapes; +3 to +12 % at
    // 512 and 128 tokens, hence the host's choice per grid).
    int mt, ntg, sk;  // ntg: N-tile over the whole launch
    if (n_fast) {
        ntg = t % grid_n;
        const int rest = t / grid_n;
        sk = rest % split;
        mt = rest / split;
    } else {
        mt = t % grid_m;
        const int rest = t / grid_m;
        sk = rest % split;
        ntg = rest / split;
    }
    // The member owning N-tile ntg (wave-uniform; at most three compares).
    int d = 0;
    if constexpr (GRP) {
#pragma unroll
        for (int i = 1; i < GEMM_GROUP_MAX; ++i) d += (i < grp.count && ntg >= grp.tile0[i]) ? 1 : 0;
    }
    const u32* __restrict__ W = GRP ? grp.w[d] : W_arg;
    const uint16_t* __restrict__ S = GRP ? grp.s[d] : S_arg;
    const uint16_t* __restrict__ Mn = GRP ? grp.m[d] : Mn_arg;
    float* __restrict__ Y = GRP ? grp.y[d] : Y_arg;
    const int N = GRP ? grp.n[d] : N_arg;
    float* __restrict__ P = GRP ? P_arg + (size_t)split * M * grp.col0[d] : P_arg;
    const int nt = GRP ? ntg - grp.tile0[d] : ntg;
    const int m0 = mt * TILE_M, n0 = nt * TN;
    const int steps = (K + BK - 1) / BK;
    const int st0 = sk * steps_per_split;
    const int st1 = min(steps, st0 + steps_per_split);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wn = wave % WN, wk = wave / WN;
    const int col = lane & 31, kh = lane >> 5;
    const uint32_t wpr = (uint32_t)K / 32 * B;  // words per W row
    // K / group through the multiply-shift pair computed on the host (exact
    // for every 31-bit dividend).
    auto group_of = [&](uint32_t kk) { return (uint32_t)(((uint64_t)kk * gmul) >> gsh); };
    const uint32_t gpr = group_of((uint32_t)K);

    const uint32_t w_bytes = (uint32_t)N * wpr * 4;
    // Formats without scales and mins read none (empty resources, null
    // pointers allowed).
    const uint32_t sm_bytes = has_affine<B>() ? (uint32_t)N * gpr * 2 : 0u;
    const uint32_t x_bytes = (uint32_t)M * (uint32_t)K * 2;
    const rsrc_t wr = make_rsrc(W, w_bytes);
    const rsrc_t sr = make_rsrc(S, sm_bytes);
    const rsrc_t mr = make_rsrc(Mn, sm_bytes);
    const rsrc_t xr = make_rsrc(X, x_bytes);

    // W side: this lane's NS columns; OOB columns read as zero.
    uint32_t w_row[NS], s_row[NS];
    bool n_ok[NS];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
        const int n = n0 + 32 * NS * wn + 32 * ns + col;
        n_ok[ns] = n < N;
        w_row[ns] = (uint32_t)n * wpr * 4;
        s_row[ns] = (uint32_t)n * gpr * 2;
    }
    // X side: this thread stages XU units of XH halves per step; the
    // threads of a row read it contiguously.
    const int xcu = tid % UPR;
    uint32_t x_row[XU];
    bool m_ok[XU];
#pragma unroll
    for (int r = 0; r < XU; ++r) {
        const int row = tid / UPR + (THREADS / UPR) * r;
        m_ok[r] = m0 + row < M;
        x_row[r] = (uint32_t)(m0 + row) * (uint32_t)K * 2;
    }

    // Raw rings: slot r holds the codes, scales and mins of W and the X
    // block of every step st with (st - st0) % PD == r.  Dequantized W pairs
    // live in a ring of two (this step's and the next one's).
    u32 xq[PD][XU][XW];
    u32 wq[PD][CH][NS][B];
    u32 sq[PD][CH][NS], mq[PD][CH][NS];
    f16x2 wv[2][CH][NS][16];
    // SW: scale and min blocks of the current and the next four steps.
    static_assert(!SW || (BK == 128 && has_affine<B>()), "wide scales: 64-code groups, 128-deep steps");
    u32x4 s_cur[NS], m_cur[NS], s_nxt[NS], m_nxt[NS];
    auto load_sm_block = [&](int st, u32x4 (&sb)[NS], u32x4 (&mb)[NS]) {
        // Groups 2*st .. 2*st + 7 of each of this lane's columns.
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
            const uint32_t so = n_ok[ns] ? s_row[ns] + (uint32_t)st * 4u : sm_bytes;
            sb[ns] = __builtin_amdgcn_raw_buffer_load_b128(sr, so, 0, 0);
            mb[ns] = __builtin_amdgcn_raw_buffer_load_b128(mr, so, 0, 0);
        }
    };
    // Step st's scales and mins from the current block: word st % 4, half
    // (HK / 64) * wk + c (group 2 * st + that).
    auto sm_of_block = [&](auto w_c, u32 (&sv)[CH][NS], u32 (&mv)[CH][NS]) {
        constexpr int WI = decltype(w_c)::value;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const uint32_t sh = 16u * (uint32_t)((HK / 64) * wk + c);
#pragma unroll
            for (int ns = 0; ns < NS; ++ns) {
                sv[c][ns] = (s_cur[ns][WI] >> sh) & 0xFFFFu;
                mv[c][ns] = (m_cur[ns][WI] >> sh) & 0xFFFFu;
            }
        }
    };

    // Loads are unconditional: a step past this split's range, like a row
    // or column past the matrix, reads zeros through the buffer range check.
    // Branch-free step bodies let the compiler count outstanding loads
    // exactly instead of draining the memory queue at every join.
    auto load_x = [&](int st, u32 (&dst)[XU][XW]) {
        const int kx = st * BK + XH * xcu;
        const bool live = st < st1 && kx < K;
#pragma unroll
        for (int r = 0; r < XU; ++r) {
            const uint32_t off = (m_ok[r] && live) ? x_row[r] + (uint32_t)kx * 2 : x_bytes;
#pragma unroll
            for (int h = 0; h < XW / 4; ++h) {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(xr, off + 16 * h, 0, 0);
                dst[r][4 * h] = v[0]; dst[r][4 * h + 1] = v[1]; dst[r][4 * h + 2] = v[2]; dst[r][4 * h + 3] = v[3];
            }
        }
    };
    auto load_w = [&](int st, u32 (&w)[CH][NS][B], u32 (&sv)[CH][NS], u32 (&mv)[CH][NS]) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int kc = st * BK + HK * wk + 64 * c + 32 * kh;
            const bool live = st < st1 && kc < K;
#pragma unroll
            for (int ns = 0; ns < NS; ++ns) {
                const bool ok = n_ok[ns] && live;
                const uint32_t wo = ok ? w_row[ns] + (uint32_t)(kc / 32) * B * 4 : w_bytes;
                buffer_words<B, unit_align(B, 32)>(wr, wo, w[c][ns]);
                if constexpr (SW) {
                    // Scales come from the block registers.
                } else if constexpr (has_affine<B>()) {
                    const uint32_t so = ok ? s_row[ns] + group_of((uint32_t)kc) * 2 : sm_bytes;
                    sv[c][ns] = buffer_u16(sr, so);
                    mv[c][ns] = buffer_u16(mr, so);
                } else {
                    sv[c][ns] = 0u;
                    mv[c][ns] = 0u;
                }
            }
        }
    };
    auto stage_x = [&](const u32 (&src)[XU][XW], int buf) {
#pragma unroll
        for (int r = 0; r < XU; ++r) {
            u32 o[XW];
            to_slot_order<B>(src[r], o);
            const int row = tid / UPR + (THREADS / UPR) * r;
            u32x4* dst = reinterpret_cast<u32x4*>(&xs[buf * XBUF + row * XROW + XH * xcu]);
#pragma unroll
            for (int h = 0; h < XW / 4; ++h) dst[h] = u32x4{o[4 * h], o[4 * h + 1], o[4 * h + 2], o[4 * h + 3]};
        }
    };
    auto dequant = [&](const u32 (&w)[CH][NS][B], const u32 (&sv)[CH][NS], const u32 (&mv)[CH][NS],
                       f16x2 (&out)[CH][NS][16]) {
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
            for (int ns = 0; ns < NS; ++ns) dequant_pairs<B>(w[c][ns], sv[c][ns], mv[c][ns], out[c][ns]);
    };

    f32x16 acc[MS][NS];
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int ns = 0; ns < NS; ++ns)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][ns][v] = 0.f;

    // Prologue: raw data for the first PD steps; the first step's X staged
    // and its W dequantized.
#pragma unroll
    for (int d = 0; d < PD; ++d) {
        load_x(st0 + d, xq[d]);
        load_w(st0 + d, wq[d], sq[d], mq[d]);
    }
    if constexpr (SW) {
        load_sm_block(st0, s_cur, m_cur);
        sm_of_block(std::integral_constant<int, 0>{}, sq[0], mq[0]);
    }
    stage_x(xq[0], 0);
    dequant(wq[0], sq[0], mq[0], wv[0]);
    __syncthreads();

    // One step at position U = (st - st0) mod UNR.  On entry X(st) sits
    // in LDS buffer U % 2 and W(st) is dequantized in wv[U % 2]; raw slot
    // U % PD is free (its data went into this step's operands during the
    // previous step).  The step
    //   * issues the loads of step st + PD into that slot,
    //   * stages X(st + 1) into the other LDS buffer (the previous step's
    //     barrier freed it), then runs its matrix work and -- independent of
    //     it, so the two overlap within the wave -- dequantizes W(st + 1),
    //   * ends with the barrier that publishes X(st + 1) and frees buffer
    //     U % 2 for step st + 2.
    constexpr int UNR = SW ? UNROLL_SW : UNROLL;
    static_assert(UNR % 2 == 0 && UNR % PD == 0, "ring positions must be compile-time");
    auto step = [&](auto u_c, int st) {
        constexpr int U = decltype(u_c)::value;
        constexpr int BUF = U % 2;
        constexpr int SLOT = U % PD, NEXT = (U + 1) % PD;
        load_w(st + PD, wq[SLOT], sq[SLOT], mq[SLOT]);
        load_x(st + PD, xq[SLOT]);
        // SW: the next block (steps st + 2 .. st + 5) goes out two steps
        // before its first use, the dequantization of step st + 2 in step
        // st + 1.  (st0 is a multiple of four, so U == st % 4.)
        if constexpr (SW && U % SW_STEPS == 2) load_sm_block(st + 2, s_nxt, m_nxt);
        // Keep the loads at the top of the step: left alone, the scheduler
        // sinks them towards their first use.
        __builtin_amdgcn_sched_barrier(0);
        // X(st + 1) (loaded a step ago) goes into the other buffer before the
        // matrix work, so the LDS writes overlap it instead of queueing just
        // before the barrier (measured -4 % on 2048 x 8192 x 2048).
        stage_x(xq[NEXT], BUF ^ 1);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const f16* xa = xs + BUF * XBUF + col * XROW + HK * wk + 64 * c + 32 * kh;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f16x8 a[MS];
#pragma unroll
                for (int i = 0; i < MS; ++i) a[i] = *reinterpret_cast<const f16x8*>(xa + 32 * i * XROW + 8 * j);
#pragma unroll
                for (int ns = 0; ns < NS; ++ns) {
                    const u32x4 bw = {as_u32(wv[BUF][c][ns][4 * j]), as_u32(wv[BUF][c][ns][4 * j + 1]),
                                      as_u32(wv[BUF][c][ns][4 * j + 2]), as_u32(wv[BUF][c][ns][4 * j + 3])};
                    const f16x8 b = __builtin_bit_cast(f16x8, bw);
#pragma unroll
                    for (int i = 0; i < MS; ++i)
                        acc[i][ns] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b, acc[i][ns], 0, 0, 0);
                }
            }
        }
        if constexpr (SW) {
            // Step st + 1 opens a new block at U % 4 == 3.
            if constexpr (U % SW_STEPS == SW_STEPS - 1) {
#pragma unroll
                for (int ns = 0; ns < NS; ++ns) {
                    s_cur[ns] = s_nxt[ns];
                    m_cur[ns] = m_nxt[ns];
                }
            }
            sm_of_block(std::integral_constant<int, (U + 1) % SW_STEPS>{}, sq[NEXT], mq[NEXT]);
        }
        dequant(wq[NEXT], sq[NEXT], mq[NEXT], wv[BUF ^ 1]);
        __syncthreads();
    };
    // Whole passes in the loop, the remainder after it: an exit from the
    // middle of a pass would reach the loop's back edge with that step's
    // loads in flight, and the compiler would then drain the memory queue
    // at the top of every pass.
    int st = st0;
    for (; st + UNR <= st1; st += UNR) all_steps<0, UNR>(step, st);
    unrolled_steps<0, UNR>(step, st, st1);

    // Add the two K-halves (KW = 2).  Fragment f = i * NS + ns; wave (wn, wk)
    // keeps the fragments with f % 2 == wk (all of them for wk == 0 when it
    // has only one) and hands the others to its partner through LDS (the X
    // buffers are free after the loop's last barrier).  With one wave along
    // K every wave stores all of its fragments.
    float* red = reinterpret_cast<float*>(smem);
    auto keeps = [&](int f) { return KW == 1 ? true : NF > 1 ? (f % 2) == wk : wk == 0; };
    if constexpr (KW == 2) {
        float* dst = red + ((wn * 2 + wk) * GIVE) * 16 * 64 + lane;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            if (keeps(f)) continue;
            const int slot = NF > 1 ? f / 2 : 0;
#pragma unroll
            for (int v = 0; v < 16; ++v) dst[(slot * 16 + v) * 64] = acc[f / NS][f % NS][v];
        }
        __syncthreads();
    }
    {
        // Store: lane holds column (lane % 32) of each 32x32 fragment, rows
        // 8*(v/4) + 4*(lane/32) + v%4.  Buffer stores, unconditional: an
        // element outside the matrix gets an offset past its end and is
        // dropped, so the epilogue has no branches (a branch per element
        // would wait for each LDS read in turn).
        // fp16 output (out16, unsplit only: split partials stay fp32 and the
        // reduction rounds): each sum rounded to nearest even, 2-byte stores.
        const float* src = red + ((wn * 2 + (1 - wk)) * GIVE) * 16 * 64 + lane;
        float* out = (split == 1) ? Y : P + (size_t)sk * M * N;
        auto store_all = [&](auto half_c) {
            constexpr bool HALF = decltype(half_c)::value;
            constexpr uint32_t ESZ = HALF ? 2u : 4u;
            const uint32_t out_bytes = (uint32_t)M * (uint32_t)N * ESZ;
            const rsrc_t orr = make_rsrc(out, out_bytes);
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                if (!keeps(f)) continue;
                const int slot = NF > 1 ? f / 2 : 0;
                const int i = f / NS, ns = f % NS;
                const int c = n0 + 32 * NS * wn + 32 * ns + col;
                float part[16];
#pragma unroll
                for (int v = 0; v < 16; ++v) part[v] = KW == 2 ? src[(slot * 16 + v) * 64] : 0.f;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = m0 + 32 * i + 8 * (v >> 2) + 4 * kh + (v & 3);
                    const uint32_t off =
                        (row < M && c < N) ? ((uint32_t)row * (uint32_t)N + (uint32_t)c) * ESZ : out_bytes;
                    const float sum = acc[i][ns][v] + part[v];
                    if constexpr (HALF)
                        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (f16)sum), orr, off, 0, 0);
                    else if constexpr (RED)
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(u32, sum), orr, off, 0,
                                                              CPOL_COHERENT);
                    else
                        buffer_store_f32(sum, orr, off);
                }
            }
        };
        if (out16 && split == 1)
            store_all(std::true_type{});
        else
            store_all(std::false_type{});
    }
    if constexpr (!RED) return;  // no split, or a separate reduction kernel

    // RED (split K, in-kernel reduction; launched only with split > 1): the
    // work-group that finishes a tile last adds the partial sums of all
    // splits and writes y.  The partial sums are written through to
    // memory (coherent stores, above) and every wave waits until its stores
    // are acknowledged before the work-group counts itself in, so whoever
    // counts in last finds all of them in memory and reads them with
    // cache-bypassing loads.  (A device-scope fence would do the same by
    // writing back and invalidating whole L2 caches, once per wave.)  The
    // last arrival also resets the tile's counter to zero for the next call.
    // Nothing waits on another work-group.
    int* flag = reinterpret_cast<int*>(smem);  // the exchange area is no longer read
    __builtin_amdgcn_s_waitcnt(WAITCNT_VM0);
    __syncthreads();
    if (tid == 0) {
        int* cnt = counters + (ntg * grid_m + mt);
        const int prev = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = prev == split - 1;
        if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = last;
    }
    __syncthreads();
    if (!*flag) return;
    reduce_tile<TILE_M, TN, THREADS>(P, Y, M, N, split, m0, n0, tid, out16);
}

// Split K, separate reduction: y = sum over splits of the partial sums, in
// split order (fp32, or rounded to fp16 when out16), spread over the whole
// GPU.  Used for more than two splits, where one work-group per tile would
// have to read too many partial sums by itself.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ P,
                                                            float* __restrict__ Y, int64_t count,
                                                            int split, int out16) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= count) return;
    float v = P[i];
    for (int s = 1; s < split; ++s) v += P[(size_t)s * count + i];
    if (out16)
        reinterpret_cast<f16*>(Y)[i] = (f16)v;
    else
        Y[i] = v;
}

hipError_t launch_splitk_reduce(const float* partial, void* y, int64_t count, int split, int out16,
                                hipStream_t st) {
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st, partial,
                       static_cast<float*>(y), count, split, out16);
    return hipGetLastError();
}

template <int B, int MS, int WN, int KW = 2, int TN = BN>
static hipError_t launch_gemm_t(const GemmArgs& a, const GemmShape& sh, hipStream_t st) {
    const DivMagic gm = div_magic(a.group);
    const int tiles = sh.grid_m * sh.grid_n * sh.split;
    const int grid = 8 * ((tiles + 7) / 8);
    constexpr bool SW_OK = has_affine<B>() && BK == 128;
    constexpr int THREADS = 64 * WN * KW;
    // The in-kernel split reduction exists for the tiles that split (32 and
    // 64 rows, 128 columns); the host passes counters only for those.
    constexpr bool RED_OK = MS <= 2 && TN == BN && KW == 2;
    const bool red = RED_OK && sh.split > 1 && a.counters;
    const GemmGroupArgs g = a.grp ? *a.grp : GemmGroupArgs{};
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(grid), dim3(THREADS), 0, st, a.w, a.s, a.m, a.x, a.y, a.partial, a.counters,
                           a.m_rows, a.n, a.k, gm.mul, gm.shift, sh.grid_m, sh.grid_n, sh.split,
                           sh.k_tiles_per_split, a.out16, g, sh.n_fast ? 1 : 0);
    };
    if (a.grp) {
        // Grouped launches: 128-column tiles, K splits reduced in the kernel
        // (the host plans no split for the tiles without that reduction).
        if constexpr (TN == BN) {
            if (sh.split > 1 && !red) return hipErrorInvalidValue;
            if (SW_OK && sh.wide_scales) {
                if (red)
                    go(gemm_kernel<B, MS, WN, KW, TN, SW_OK, RED_OK, true>);
                else
                    go(gemm_kernel<B, MS, WN, KW, TN, SW_OK, false, true>);
            } else {
                if (red)
                    go(gemm_kernel<B, MS, WN, KW, TN, false, RED_OK, true>);
                else
                    go(gemm_kernel<B, MS, WN, KW, TN, false, false, true>);
            }
            return hipGetLastError();
        } else {
            return hipErrorInvalidValue;
        }
    }
    if (SW_OK && sh.wide_scales) {
        if (red)
            go(gemm_kernel<B, MS, WN, KW, TN, SW_OK, RED_OK>);
        else
            go(gemm_kernel<B, MS, WN, KW, TN, SW_OK>);
    } else {
        if (red)
            go(gemm_kernel<B, MS, WN, KW, TN, false, RED_OK>);
        else
            go(gemm_kernel<B, MS, WN, KW, TN>);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || sh.split == 1 || red) return err;
    return launch_splitk_reduce(a.partial, a.y, (int64_t)a.m_rows * a.n, sh.split, a.out16, st);
}

template <int B>
static hipError_t launch_gemm_b(const GemmArgs& a, const GemmShape& sh, hipStream_t st) {
    if (sh.tile_n == 256) {
        // Eight waves along N, each taking whole steps.
        switch (sh.tile_m) {
            case 64: return launch_gemm_t<B, 2, 8, 1, 256>(a, sh, st);
            case 128: return launch_gemm_t<B, 4, 8, 1, 256>(a, sh, st);
            default: return hipErrorInvalidValue;
        }
    }
    switch (sh.tile_m) {
        case 32: return launch_gemm_t<B, 1, gemm_threads(32) / 128>(a, sh, st);
        case 64: return launch_gemm_t<B, 2, gemm_threads(64) / 128>(a, sh, st);
        case 128: return launch_gemm_t<B, 4, gemm_threads(128) / 128>(a, sh, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm(const GemmArgs& a, const GemmShape& sh, hipStream_t st) {
    if (sh.kernel == 1) return launch_gemm_wl(a, sh, st);
    switch (a.bits) {
        case 2: return launch_gemm_b<2>(a, sh, st);
        case 3: return launch_gemm_b<3>(a, sh, st);
        case 4: return launch_gemm_b<4>(a, sh, st);
        case 5: return launch_gemm_b<5>(a, sh, st);
        case 6: return launch_gemm_b<6>(a, sh, st);
        case 8: return launch_gemm_b<8>(a, sh, st);
        case 16: return launch_gemm_b<16>(a, sh, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
