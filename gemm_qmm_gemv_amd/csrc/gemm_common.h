// gemm_common.h -- pieces shared by the two prefill GEMM kernels (weights
// dequantized into registers, gemm.hip; weights dequantized into LDS,
// gemm_wl.hip): chunk dequantization, the split-K tile reduction and host
// helpers.
#pragma once

#include "qmm_device.h"
#include "qmm_kernels.h"

#include <type_traits>

namespace qmm {

// Slot order of a 32-code chunk: slot 2i holds code ka(i) and slot 2i+1 code
// kb(i) of the pair format, i.e. exactly the order in which the dequantized
// pairs sit in registers.
template <int B>
constexpr int slot_k(int p) {
    return (p & 1) ? PairFmt<B>::kb(p >> 1) : PairFmt<B>::ka(p >> 1);
}

// One 32-code chunk (b words) -> 16 fp16 pairs s*q + m in slot order.
template <int B>
__device__ __forceinline__ void dequant_pairs(const u32 (&w)[B], u32 s_bits, u32 m_bits,
                                              f16x2 (&out)[16]) {
    using F = PairFmt<B>;
    if constexpr (!has_affine<B>()) {
        // fp16 weights: the words are the operand pairs already.
#pragma unroll
        for (int i = 0; i < 16; ++i) out[i] = as_h2(w[i]);
        return;
    }
    u32 p[16];
    F::extract(w, p);
    const f16 s = __builtin_bit_cast(f16, (uint16_t)s_bits);
    const f16 m = __builtin_bit_cast(f16, (uint16_t)m_bits);
    const f16x2 s2 = {s, s}, m2 = {m, m};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const f16 inv = (f16)F::inv_factor(F::acc(i));
        const f16 off = (f16)(-1024.0f * F::inv_factor(F::acc(i)));
        const f16x2 inv2 = {inv, inv}, off2 = {off, off};
        // (1024 + f q) * (1/f) - 1024/f is exactly q (f a power of two).
        const f16x2 q2 = __builtin_elementwise_fma(as_h2(p[i]), inv2, off2);
        // s*q + m, fused: one rounding of the exact value to fp16.
        out[i] = __builtin_elementwise_fma(q2, s2, m2);
    }
}

// Steps U..N-1 of one pass of the unrolled main loop: all of them, or (for
// the remainder after the loop) only those before st1.
template <int U, int N, class F>
__device__ __forceinline__ void all_steps(F& f, int st) {
    if constexpr (U < N) {
        f(std::integral_constant<int, U>{}, st + U);
        all_steps<U + 1, N>(f, st);
    }
}
template <int U, int N, class F>
__device__ __forceinline__ void unrolled_steps(F& f, int st, int st1) {
    if constexpr (U < N) {
        if (st + U < st1) {
            f(std::integral_constant<int, U>{}, st + U);
            unrolled_steps<U + 1, N>(f, st, st1);
        }
    }
}

// Cache policy of the split-K partial sums: sc0 | sc1 (system coherence), so
// stores write through to memory and loads fetch from it, past every cache.
constexpr int CPOL_COHERENT = 1 | 16;
// s_waitcnt with vmcnt = 0 (expcnt and lgkmcnt at their maxima, not waited on).
constexpr int WAITCNT_VM0 = 0x0F70;
template <int TILE_M, int TN, int THREADS>
__device__ __forceinline__ void reduce_tile(const float* P, float* Y, int M, int N, int split, int m0, int n0,
                                            int tid, int out16) {
    const uint32_t mn = (uint32_t)M * (uint32_t)N;  // floats per split
    const uint32_t p_bytes = mn * 4u * (uint32_t)split;  // < 2^32: checked on the host
    const uint32_t y_bytes = mn * (out16 ? 2u : 4u);
    const rsrc_t pr = make_rsrc(P, p_bytes);
    const rsrc_t yr = make_rsrc(Y, y_bytes);
    auto sum_groups = [&](auto vec_c) {
        constexpr int V = decltype(vec_c)::value;      // columns per group: 4 or 1
        constexpr int GROUPS = TILE_M * TN / V;          // groups in the tile
        static_assert(GROUPS % THREADS == 0, "tile reduction layout");
        constexpr int PER = GROUPS / THREADS;
        constexpr int E = PER < 4 ? PER : 4;
        using vec = std::conditional_t<V == 4, f32x4, float>;
#pragma unroll 1
        for (int e0 = 0; e0 < PER; e0 += E) {
            uint32_t off[E];
            bool ok[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int q = (e0 + e) * THREADS + tid;
                const int r = m0 + q / (TN / V), c = n0 + V * (q % (TN / V));
                ok[e] = r < M && c < N;
                off[e] = (uint32_t)r * (uint32_t)N + (uint32_t)c;  // element index
            }
            vec acc[E];
#pragma unroll 1
            for (int s0 = 0; s0 < split; s0 += 4) {
                vec v[4][E];
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const uint32_t o = (ok[e] && s0 + j < split) ? ((uint32_t)(s0 + j) * mn + off[e]) * 4u : p_bytes;
                        if constexpr (V == 4)
                            v[j][e] = __builtin_bit_cast(
                                f32x4, __builtin_amdgcn_raw_buffer_load_b128(pr, o, 0, CPOL_COHERENT));
                        else
                            v[j][e] = __builtin_bit_cast(
                                float, __builtin_amdgcn_raw_buffer_load_b32(pr, o, 0, CPOL_COHERENT));
                    }
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[e] = (s0 == 0 && j == 0) ? v[j][e] : acc[e] + v[j][e];
            }
#pragma unroll
            for (int e = 0; e < E; ++e) {
                if (out16) {
                    const uint32_t o = ok[e] ? off[e] * 2u : y_bytes;
                    if constexpr (V == 4) {
                        const f16 h[4] = {(f16)acc[e][0], (f16)acc[e][1], (f16)acc[e][2], (f16)acc[e][3]};
                        u32x2 w;
                        __builtin_memcpy(&w, h, 8);
                        __builtin_amdgcn_raw_buffer_store_b64(w, yr, o, 0, 0);
                    } else {
                        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (f16)acc[e]), yr, o, 0, 0);
                    }
                } else {
                    const uint32_t o = ok[e] ? off[e] * 4u : y_bytes;
                    if constexpr (V == 4)
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[e]), yr, o, 0, 0);
                    else
                        buffer_store_f32(acc[e], yr, o);
                }
            }
        }
    };
    if (N % 4 == 0)
        sum_groups(std::integral_constant<int, 4>{});
    else
        sum_groups(std::integral_constant<int, 1>{});
}


// Tiles a launch of `tiles` work-groups gives each of the 8 XCDs: the XCDs
// take contiguous ranges of tiles (work-group i runs on XCD i % 8).
__device__ __forceinline__ int xcd_tile(int tiles) {
    const int per_xcd = (tiles + 7) / 8;
    return (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
}

// floor(n / d) = (n * mul) >> shift for every n < 2^31: shift = 31 + ceil(log2 d),
// mul = ceil(2^shift / d) (Granlund and Montgomery, "Division by invariant
// integers using multiplication", 1994, the N+1-bit multiplier case).
struct DivMagic {
    uint64_t mul;
    int shift;
};
static DivMagic div_magic(int d) {
    int l = 0;
    while ((1LL << l) < d) ++l;
    const int shift = 31 + l;
    return {((1ULL << shift) + (uint64_t)d - 1) / (uint64_t)d, shift};
}


}  // namespace qmm
