// gemm_wl.hip -- prefill GEMM with the weights dequantized into LDS tiles
// that feed the fp16 matrix cores.
//
// Pages: "BaseRT claims fastest Apple Silicon inference" (thetesserapress.com),
// section "What BaseRT does differently" (GEMM kernels for prefill where
// M > 1, dequantization inside the compute loop, full-precision weights never
// written back to memory); "BaseRT: Best-in-Class LLM Inference on Apple
// Silicon via Native Metal" (gist.science summary), section "Metodologia"
// (tiled prefill GEMM on the GPU's matrix hardware).
//
// Y[M][N] = X[M][K] * W^T with W = s*q + m, on v_mfma_f32_32x32x16_f16.
//
// Warp-specialized work-group: WM x 2 consumer waves and four producer
// waves share a ring of LDS stages (three for 128-column tiles, two for
// 256-column tiles); K advances 64 codes per step and every step ends at
// one work-group barrier.
//
//   * Producers, X: the step's X tile goes from memory straight into LDS
//     with the direct global-to-LDS buffer loads (one kilobyte per wave and
//     instruction, no registers, no reordering).
//   * Producers, W: each thread owns one or two 32-code chunks of the step's
//     W tile: it loads the chunk's b words and the group's scale and min two
//     steps ahead, then dequantizes the chunk into 32 fp16 values s*q + m
//     (exact code through the fp16 mantissa, one rounding), puts them in
//     natural k order with one byte permute per pair and writes them to the
//     stage.  Every weight is dequantized once per work-group, and only the
//     compressed bytes come from memory.
//   * Consumers: read A (X rows) and B (dequantized W columns) fragments
//     from the stage and issue the matrix instructions; no global loads and
//     no dequantization, so the matrix pipe is fed by LDS alone.  Each
//     consumer wave owns a 64 x 32 NS block of Y (NS = 2 or 4).
//   * LDS rows are 128 bytes of eight 16-byte pieces, XOR-swizzled so that
//     the producers' stores and the consumers' 16-byte fragment reads are
//     free of bank conflicts.
//   * The barrier closing a step waits for the stage it hands over and for
//     nothing newer: the producers' direct loads are not tracked by the
//     compiler, so the wait counts them explicitly (scheduling barriers fix
//     the order of the loads it counts).
//
// K splits (partial sums summed in the kernel by the last work-group of a
// tile), the XCD-aware tile order and grouped launches (several matrices
// sharing X, their column tiles concatenated) work as in gemm.hip.
#include "gemm_common.h"

namespace qmm {

namespace {

// Slot (position in dequant_pairs' output, 2 * pair + half) of code k of a chunk.
template <int B>
struct SlotOfCode {
    int v[32];
};
template <int B>
constexpr SlotOfCode<B> slot_of_code() {
    SlotOfCode<B> t{};
    for (int k = 0; k < 32; ++k)
        for (int p = 0; p < 32; ++p)
            if (slot_k<B>(p) == k) t.v[k] = p;
    return t;
}

// One chunk (b words) -> 32 fp16 weights s*q + m in natural k order, as
// four 16-byte pieces.
template <int B>
__device__ __forceinline__ void chunk_natural(const u32 (&w)[B], u32 s_bits, u32 m_bits, u32x4 (&out)[4]) {
    if constexpr (!has_affine<B>()) {
        // fp16 weights: the words are the natural pairs already.
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
    } else {
        constexpr SlotOfCode<B> SL = slot_of_code<B>();
        f16x2 pr[16];
        dequant_pairs<B>(w, s_bits, m_bits, pr);
        u32 o[16];
#pragma unroll
        for (int d = 0; d < 16; ++d) {
            const int p0 = SL.v[2 * d], p1 = SL.v[2 * d + 1];
            const int i0 = p0 >> 1, h0 = p0 & 1, i1 = p1 >> 1, h1 = p1 & 1;
            if (i0 == i1 && h0 == 0 && h1 == 1) {
                o[d] = as_u32(pr[i0]);
            } else {
                // v_perm_b32: selector bytes 0-3 index the second operand,
                // 4-7 the first.
                const u32 sel = (u32)(2 * h0) | (u32)(2 * h0 + 1) << 8 | (u32)(4 + 2 * h1) << 16 |
                                (u32)(5 + 2 * h1) << 24;
                o[d] = __builtin_amdgcn_perm(as_u32(pr[i1]), as_u32(pr[i0]), sel);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = u32x4{o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
    }
}

// Fewest load instructions one chunk's b words can take: the compiler may
// merge neighbouring word loads into wider ones (three 4-byte loads into one
// 12-byte load for Q3), up to 16 bytes each.  A barrier that leaves "the
// newest n loads" in flight must count with this lower bound, never with
// the instructions written in the source.
template <int B>
constexpr int chunk_load_instructions_min() {
    return (B + 3) / 4;
}

constexpr int WL_WN = 2;          // consumer waves along N
constexpr int WL_PRODUCERS = 4;   // producer waves
constexpr int WL_BK = 64;         // codes per step
// Cache policy of the split-K partial sums and s_waitcnt vmcnt(0), as in gemm.hip.
constexpr int WL_CPOL_COHERENT = 1 | 16;
constexpr int WL_WAITCNT_VM0 = 0x0F70;

template <int WM>
constexpr int wl_threads() { return 64 * (WM * WL_WN + WL_PRODUCERS); }

// Work-group barrier after waiting for all LDS traffic and for all but the
// VM newest vector-memory loads.  The wait is the builtin, so the compiler's
// own wait bookkeeping knows about it; the barrier is an asm statement with
// a memory clobber, so no load or store moves across it.
template <int VM>
__device__ __forceinline__ void wl_barrier() {
    static_assert(VM >= 0 && VM <= 63, "vmcnt range");
    // s_waitcnt fields: vmcnt bits 3:0 and 15:14, expcnt 6:4 (7: no wait),
    // lgkmcnt 11:8.
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));
    asm volatile("s_barrier" ::: "memory");
}
typedef __attribute__((address_space(3))) unsigned char lds_u8;

// LDS tiles hold 128-byte rows of eight 16-byte pieces; piece q of row r
// sits in slot q ^ f(r), f(r) = (r & 7) ^ ((r >> 3) & 1).  Sixteen
// consecutive rows (from a multiple of 16) reading the same piece then
// cover all 64 banks -- the rows of one parity take eight distinct slots --
// and so do eight consecutive rows.  f depends on r mod 16 only.
__host__ __device__ constexpr int wl_slot(int r, int q) { return q ^ ((r & 7) ^ ((r >> 3) & 1)); }

// WM consumer waves along M (2 or 4, 64 rows each), two along N with NS
// 32-column fragments each (NS = 2: 128-column tiles, three LDS stages;
// NS = 4: 256-column tiles, two stages).
template <int NS>
constexpr int wl_stages() { return NS == 2 ? 3 : 2; }

template <int B, int WM, int NS, bool RED = false, bool GRP = false>
__global__ __launch_bounds__(wl_threads<WM>(), 1) void gemm_wl_kernel(
    const u32* __restrict__ W_arg, const uint16_t* __restrict__ S_arg, const uint16_t* __restrict__ Mn_arg,
    const uint16_t* __restrict__ X, float* __restrict__ Y_arg, float* __restrict__ P_arg,
    int* __restrict__ counters, int M, int N_arg, int K, uint64_t gmul, int gsh, int grid_m, int grid_n,
    int split, int steps_per_split, int out16, GemmGroupArgs grp, int n_fast) {
    constexpr int WN = WL_WN, MS = 2;
    constexpr int CONSUMERS = 64 * WM * WN;
    constexpr int TM = 32 * MS * WM, TN = 32 * NS * WN;
    constexpr int BK = WL_BK;
    constexpr int NSTG = wl_stages<NS>();
    constexpr int ROWB = BK * 2;                          // bytes per tile row and step
    constexpr int XST = TM * ROWB, WST = TN * ROWB;       // bytes per stage
    constexpr int STAGE = XST + WST;
    constexpr int XLOADS = TM / 8 / WL_PRODUCERS;         // 1 KB direct loads per producer wave and step
    constexpr int CPT = TN * (BK / 32) / (64 * WL_PRODUCERS);  // W chunks per producer thread and step
    constexpr int CLOADS = CPT * (chunk_load_instructions_min<B>() + (has_affine<B>() ? 2 : 0));
    static_assert(CPT * 64 * WL_PRODUCERS == TN * (BK / 32), "whole W chunks per producer thread");
    // Loads issued after X(st + 1) when the barrier closing step st waits
    // for it: with three stages X(st + 1) went out a step earlier, followed
    // by two steps' codes and X(st + 2); with two, only this step's codes.
    constexpr int VM_AT_BARRIER = NSTG == 3 ? 2 * CLOADS + XLOADS : CLOADS;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NSTG * STAGE];

    const int tiles = grid_m * grid_n * split;
    const int t = xcd_tile(tiles);
    if (t >= tiles) return;
    int mt, ntg, sk;
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
    const int m0 = mt * TM, n0 = nt * TN;
    const int steps = (K + BK - 1) / BK;
    const int st0 = sk * steps_per_split;
    const int st1 = min(steps, st0 + steps_per_split);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    lds_u8* const lds = (lds_u8*)smem;
    auto stage_of = [&](int st) { return (uint32_t)((st - st0) % NSTG) * STAGE; };

    f32x16 acc[MS][NS];
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int j = 0; j < NS; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    if (wave >= WM * WN) {
        // ---- producer: X tiles by direct loads, W tiles dequantized ----
        // pw is made explicitly wave-uniform: the direct loads take their LDS
        // address from M0, and a per-lane value there costs a loop.
        const int p = tid - CONSUMERS, pw = __builtin_amdgcn_readfirstlane(p >> 6);
        const uint32_t wpr = (uint32_t)K / 32 * B;  // words per W row
        auto group_of = [&](uint32_t kk) { return (uint32_t)(((uint64_t)kk * gmul) >> gsh); };
        const uint32_t gpr = group_of((uint32_t)K);
        const uint32_t w_bytes = (uint32_t)N * wpr * 4;
        const uint32_t sm_bytes = has_affine<B>() ? (uint32_t)N * gpr * 2 : 0u;
        const uint32_t x_bytes = (uint32_t)M * (uint32_t)K * 2;
        const rsrc_t wr = make_rsrc(W, w_bytes);
        const rsrc_t sr = make_rsrc(S, sm_bytes);
        const rsrc_t mr = make_rsrc(Mn, sm_bytes);
        const rsrc_t xr = make_rsrc(X, x_bytes);
        const int nblk = K / 32;
        // W: chunk c of this thread is (column cn + 128 c, block cb of the
        // step): lanes 0-15 of a wave take block 0 of sixteen rows, lanes
        // 16-31 block 1 of the same rows, and so on.
        const int cb = (p >> 4) & 1;
        uint32_t w_row[CPT], s_row[CPT], w_lds[CPT][4];
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int cn = ((p & 15) | ((p >> 5) << 4)) + 128 * c;
            const bool ok = n0 + cn < N;
            w_row[c] = ok ? (uint32_t)(n0 + cn) * wpr * 4 : w_bytes;
            s_row[c] = ok ? (uint32_t)(n0 + cn) * gpr * 2 : sm_bytes;
            // The chunk's four 16-byte pieces in swizzled slots (sixteen
            // lanes store the same piece of sixteen consecutive rows).
#pragma unroll
            for (int i = 0; i < 4; ++i) w_lds[c][i] = XST + cn * ROWB + 16 * wl_slot(cn, 4 * cb + i);
        }
        // X: load i of this wave covers tile rows 8 * (XLOADS * pw + i) ..+7
        // (one KB: lane l writes slot l % 8 of row l / 8 of them, so it
        // brings the piece that the swizzle puts there).
        uint32_t x_off[XLOADS];
        int x_k[XLOADS];  // halves into the step of that piece
#pragma unroll
        for (int i = 0; i < XLOADS; ++i) {
            const int r = 8 * (XLOADS * pw + i) + (lane >> 3);
            x_k[i] = 8 * wl_slot(r, lane & 7);  // the swizzle is an involution
            x_off[i] = m0 + r < M ? (uint32_t)(m0 + r) * (uint32_t)K * 2 + 2u * x_k[i] : x_bytes;
        }
        auto load_x = [&](int st) {
            const uint32_t stage = stage_of(st);
#pragma unroll
            for (int i = 0; i < XLOADS; ++i) {
                // Past K (a step may hold one block beyond it) the load reads
                // zeros.  Steps past the split's end load real rows that are
                // never multiplied (no uniform test here: the compiler would
                // turn it into branches around the loads).
                const bool live = st * BK + x_k[i] < K && x_off[i] < x_bytes;
                const uint32_t off = live ? x_off[i] + (uint32_t)st * ROWB : x_bytes;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, lds + stage + 1024u * (XLOADS * pw + i), 16, off,
                                                         0, 0, 0);
            }
        };
        // W codes need no liveness test: a step past the split is never
        // multiplied and a block past K meets zero activations (its index
        // is clamped into the row); columns past N read zeros.
        typedef u32 Codes[CPT][B];
        auto load_w = [&](int st, Codes& w, u32 (&sv)[CPT], u32 (&mv)[CPT]) {
            const uint32_t pb = (uint32_t)min(st * (BK / 32) + cb, nblk - 1);
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                buffer_words<B, unit_align(B, 32)>(wr, w_row[c] + pb * B * 4, w[c]);
                if constexpr (has_affine<B>()) {
                    const uint32_t so = s_row[c] + group_of(pb * 32u) * 2;
                    sv[c] = buffer_u16(sr, so);
                    mv[c] = buffer_u16(mr, so);
                } else {
                    sv[c] = 0u;
                    mv[c] = 0u;
                }
            }
        };
        auto store_w = [&](int st, const Codes& w, const u32 (&sv)[CPT], const u32 (&mv)[CPT]) {
            const uint32_t stage = stage_of(st);
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                u32x4 o[4];
                chunk_natural<B>(w[c], sv[c], mv[c], o);
#pragma unroll
                for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(smem + stage + w_lds[c][i]) = o[i];
            }
        };
        // Codes ring by step parity: the codes of step s sit in slot
        // (s - st0) % 2 from two steps before their dequantization.
        Codes wq[2];
        u32 sq[2][CPT], mq[2][CPT];
        // Prologue: stages 0 .. NSTG - 2 filled (steps st0 ..), the codes of
        // the next two steps in flight.
#pragma unroll
        for (int j = 0; j < NSTG - 1; ++j) {
            load_w(st0 + j, wq[j % 2], sq[j % 2], mq[j % 2]);
            load_x(st0 + j);
            store_w(st0 + j, wq[j % 2], sq[j % 2], mq[j % 2]);
        }
        load_w(st0 + NSTG - 1, wq[(NSTG - 1) % 2], sq[(NSTG - 1) % 2], mq[(NSTG - 1) % 2]);
        load_w(st0 + NSTG, wq[NSTG % 2], sq[NSTG % 2], mq[NSTG % 2]);
        wl_barrier<0>();
        // Step st fills the stage of step st + NSTG - 1: the W tile from the
        // codes loaded two steps ago (they came before the previous step's
        // loads, so using them waits for nothing newer), then the X loads,
        // then the codes of two steps later into the freed slot; and waits
        // for X(st + 1).
        auto step = [&](auto u_c, int st) {
            constexpr int U = decltype(u_c)::value;  // (st - st0) % 2
            constexpr int SL = (U + NSTG - 1) % 2;   // slot of step st + NSTG - 1
            store_w(st + NSTG - 1, wq[SL], sq[SL], mq[SL]);
            // The scheduling barriers keep every X load ahead of every code
            // load: the barrier's count of loads left in flight relies on
            // that order.
            __builtin_amdgcn_sched_barrier(0);
            load_x(st + NSTG - 1);
            __builtin_amdgcn_sched_barrier(0);
            load_w(st + NSTG + 1, wq[SL], sq[SL], mq[SL]);
            __builtin_amdgcn_sched_barrier(0);
            wl_barrier<VM_AT_BARRIER>();
        };
        int st = st0;
        for (; st + 2 <= st1; st += 2) {
            step(std::integral_constant<int, 0>{}, st);
            step(std::integral_constant<int, 1>{}, st + 1);
        }
        if (st < st1) step(std::integral_constant<int, 0>{}, st);
    } else {
        // ---- consumer: A and B fragments from LDS into the matrix cores ----
        const int wm = wave % WM, wn = wave / WM;
        const int l32 = lane & 31, h = lane >> 5;
        // Row r (column n) of the tile: piece 2t + h of substep t sits in
        // slot wl_slot(r, 2t + h); every fragment starts at a multiple of 32
        // rows, so the swizzle depends on l32 alone.
        uint32_t a_row[MS], b_row[NS];
#pragma unroll
        for (int i = 0; i < MS; ++i) a_row[i] = (uint32_t)(64 * wm + 32 * i + l32) * ROWB;
#pragma unroll
        for (int j = 0; j < NS; ++j) b_row[j] = XST + (uint32_t)(32 * NS * wn + 32 * j + l32) * ROWB;
        const int sw = wl_slot(l32, 0);
        constexpr int SUB = BK / 16;
        // Fragments of two substeps (one for 128-column wave tiles, whose
        // accumulators leave no room for a second set).
        constexpr int FB = NS == 4 ? 1 : 2;
        f16x8 fa[FB][MS], fb[FB][NS];
        auto read = [&](uint32_t stage, int s4, f16x8 (&a)[MS], f16x8 (&b)[NS]) {
            const uint32_t slot = 16u * (uint32_t)((2 * s4 + h) ^ sw);
#pragma unroll
            for (int i = 0; i < MS; ++i) a[i] = *reinterpret_cast<const f16x8*>(smem + stage + a_row[i] + slot);
#pragma unroll
            for (int j = 0; j < NS; ++j) b[j] = *reinterpret_cast<const f16x8*>(smem + stage + b_row[j] + slot);
        };
        auto mfma = [&](const f16x8 (&a)[MS], const f16x8 (&b)[NS]) {
#pragma unroll
            for (int i = 0; i < MS; ++i)
#pragma unroll
                for (int j = 0; j < NS; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        };
        wl_barrier<0>();  // the producers' prologue
        if constexpr (FB == 2) {
            read(stage_of(st0), 0, fa[0], fb[0]);
            // Fragments are read one substep ahead; the last substep's
            // matrix work goes after the barrier, beside the first reads of
            // the next step.
            for (int st = st0; st < st1; ++st) {
                const uint32_t stage = stage_of(st);
#pragma unroll
                for (int s4 = 0; s4 + 1 < SUB; ++s4) {
                    read(stage, s4 + 1, fa[(s4 + 1) % 2], fb[(s4 + 1) % 2]);
                    mfma(fa[s4 % 2], fb[s4 % 2]);
                }
                wl_barrier<0>();
                if (st + 1 < st1) read(stage_of(st + 1), 0, fa[0], fb[0]);
                mfma(fa[(SUB - 1) % 2], fb[(SUB - 1) % 2]);
            }
        } else {
            for (int st = st0; st < st1; ++st) {
                const uint32_t stage = stage_of(st);
#pragma unroll
                for (int s4 = 0; s4 < SUB; ++s4) {
                    read(stage, s4, fa[0], fb[0]);
                    mfma(fa[0], fb[0]);
                }
                wl_barrier<0>();
            }
        }
    }

    // Store (consumers): lane holds column l32 of each 32x32 fragment, rows
    // 8*(v/4) + 4*h + v%4.  Unconditional buffer stores: elements outside
    // the matrix get an offset past its end and are dropped.
    if (wave < WM * WN) {
        const int wm = wave % WM, wn = wave / WM;
        const int l32 = lane & 31, h = lane >> 5;
        float* out = (split == 1) ? Y : P + (size_t)sk * M * N;
        auto store_all = [&](auto half_c) {
            constexpr bool HALF = decltype(half_c)::value;
            constexpr uint32_t ESZ = HALF ? 2u : 4u;
            const uint32_t out_bytes = (uint32_t)M * (uint32_t)N * ESZ;
            const rsrc_t orr = make_rsrc(out, out_bytes);
#pragma unroll
            for (int i = 0; i < MS; ++i)
#pragma unroll
                for (int j = 0; j < NS; ++j) {
                    const int c = n0 + 32 * NS * wn + 32 * j + l32;
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int row = m0 + 64 * wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
                        const uint32_t off =
                            (row < M && c < N) ? ((uint32_t)row * (uint32_t)N + (uint32_t)c) * ESZ : out_bytes;
                        const float sum = acc[i][j][v];
                        if constexpr (HALF)
                            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (f16)sum), orr, off,
                                                                  0, 0);
                        else if constexpr (RED)
                            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(u32, sum), orr, off, 0,
                                                                  WL_CPOL_COHERENT);
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
    if constexpr (!RED) return;

    // Two splits summed here by whichever work-group of the tile finishes
    // last (as in gemm.hip: write-through partial sums, acknowledged before
    // the arrival count, read back past the caches; the counter is reset).
    int* flag = reinterpret_cast<int*>(smem);  // the last step's barrier ended every LDS access
    __builtin_amdgcn_s_waitcnt(WL_WAITCNT_VM0);
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
    if (tid < CONSUMERS) reduce_tile<TM, TN, CONSUMERS>(P, Y, M, N, split, m0, n0, tid, out16);
}

template <int B, int WM, int NS>
hipError_t launch_wl_t(const GemmArgs& a, const GemmShape& sh, hipStream_t st) {
    const DivMagic gm = div_magic(a.group);
    const int tiles = sh.grid_m * sh.grid_n * sh.split;
    const int grid = 8 * ((tiles + 7) / 8);
    const bool red = sh.split > 1 && a.counters;
    const GemmGroupArgs g = a.grp ? *a.grp : GemmGroupArgs{};
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(grid), dim3(wl_threads<WM>()), 0, st, a.w, a.s, a.m, a.x, a.y, a.partial,
                           a.counters, a.m_rows, a.n, a.k, gm.mul, gm.shift, sh.grid_m, sh.grid_n, sh.split,
                           sh.k_tiles_per_split, a.out16, g, sh.n_fast ? 1 : 0);
    };
    if (a.grp) {
        if (sh.split > 1 && !red) return hipErrorInvalidValue;
        if (red)
            go(gemm_wl_kernel<B, WM, NS, true, true>);
        else
            go(gemm_wl_kernel<B, WM, NS, false, true>);
        return hipGetLastError();
    }
    if (red)
        go(gemm_wl_kernel<B, WM, NS, true>);
    else
        go(gemm_wl_kernel<B, WM, NS>);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || sh.split == 1 || red) return err;
    return launch_splitk_reduce(a.partial, a.y, (int64_t)a.m_rows * a.n, sh.split, a.out16, st);
}

template <int B>
hipError_t launch_wl_b(const GemmArgs& a, const GemmShape& sh, hipStream_t st) {
    if (sh.tile_m == 256 && sh.tile_n == 128) return launch_wl_t<B, 4, 2>(a, sh, st);
    if (sh.tile_m == 128 && sh.tile_n == 128) return launch_wl_t<B, 2, 2>(a, sh, st);
    if (sh.tile_m == 128 && sh.tile_n == 256) return launch_wl_t<B, 2, 4>(a, sh, st);
    if (sh.tile_m == 256 && sh.tile_n == 256) return launch_wl_t<B, 4, 4>(a, sh, st);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_wl(const GemmArgs& a, const GemmShape& sh, hipStream_t st) {
#ifdef QMM_WL_BITS_ONLY
    if (a.bits != QMM_WL_BITS_ONLY) return hipErrorInvalidValue;
    return launch_wl_b<QMM_WL_BITS_ONLY>(a, sh, st);
#else
    switch (a.bits) {
        case 2: return launch_wl_b<2>(a, sh, st);
        case 3: return launch_wl_b<3>(a, sh, st);
        case 4: return launch_wl_b<4>(a, sh, st);
        case 5: return launch_wl_b<5>(a, sh, st);
        case 6: return launch_wl_b<6>(a, sh, st);
        case 8: return launch_wl_b<8>(a, sh, st);
        case 16: return launch_wl_b<16>(a, sh, st);
        default: return hipErrorInvalidValue;
    }
#endif
}

}  // namespace qmm
