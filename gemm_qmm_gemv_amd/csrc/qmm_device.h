// qmm_device.h -- device-side building blocks shared by the HIP kernels:
// bit extraction of packed codes into fp16 pairs, activation pair set-up and
// the per-unit dot product.
//
// Format (the library's definition; the pages only say "affine quantization
// Q2 to Q8"): code k of a row sits at stream bits [k*b, k*b+b), stream bit i
// is bit i%32 of word i/32; w = s*q + m per group of K.
//
// Inline dequantization ("BaseRT claims fastest Apple Silicon inference",
// section "What BaseRT does differently": weights are dequantized inside the
// compute loop and never written back in full precision) is done here in two
// steps that cost a handful of VALU operations per weight:
//
//  1. Code -> fp16 without a conversion instruction.  OR-ing an integer
//     v < 1024 into the mantissa of the fp16 constant 1024.0 (bit pattern
//     0x6400) gives exactly the fp16 value 1024 + v: in [1024, 2048) the fp16
//     spacing is 1.  A mask over a 32-bit word can place two codes at once,
//     one in each 16-bit half (0x64006400 holds two 1024.0).  Codes may sit
//     at a bit offset f inside the half, which yields 1024 + 2^f * q; that is
//     still exact while 2^f * q < 1024, and the power of two is divided out
//     later, exactly.
//  2. The group-factored product.  For one group,
//        sum_k (s q_k + m) x_k = s * sum_k q_k x_k + m * sum_k x_k,
//     and sum_k (1024 + 2^f q_k) x_k = 1024 sum x_k + 2^f sum q_k x_k.
//     So the inner loop is nothing but v_dot2_f32_f16 on (1024 + 2^f q) pairs
//     against activation pairs, and the constant 1024 * sum x (weighted by
//     2^-f per accumulator) is subtracted once per unit.  The activation-side
//     constants do not depend on the weight row, so a lane computes them once
//     and reuses them for every row it visits.
//
// A "chunk" is 32 consecutive codes of a row (b words).  Each chunk gives 16
// packed pairs; PairFmt<b> lists, for pair i, the two code positions (ka, kb)
// inside the chunk and the accumulator (one per bit offset f) it adds into.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32;
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef u32 u32x4 __attribute__((ext_vector_type(4)));

constexpr u32 MAGIC2 = 0x64006400u;  // two fp16 1024.0

__device__ __forceinline__ f16x2 as_h2(u32 v) { return __builtin_bit_cast(f16x2, v); }
__device__ __forceinline__ u32 as_u32(f16x2 v) { return __builtin_bit_cast(u32, v); }
__device__ __forceinline__ float half_bits_to_float(uint16_t v) {
    return (float)__builtin_bit_cast(f16, v);
}
// ((hi:lo) >> sh) low word, 0 < sh < 32.
__device__ __forceinline__ u32 funnel(u32 hi, u32 lo, u32 sh) {
    return __builtin_amdgcn_alignbit(hi, lo, sh);
}
// (v & mask) | 0x64006400 as one v_and_or_b32.  gfx9 VOP3 encodings take no
// literal operands and at most one scalar register, so the mask comes from
// an SGPR and the fp16 pair constant from a VGPR; left to itself the
// compiler splits this into an AND and an OR with literals.
__device__ __forceinline__ u32 mask_or_magic(u32 v, u32 mask) {
    u32 r;
    const u32 magic = MAGIC2;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "s"(mask), "v"(magic));
    return r;
}
// Raw buffer resources.  A buffer load addresses memory as an SGPR base plus
// a 32-bit VGPR byte offset, and returns zero for offsets at or past the
// resource's size, so row and unit tails need no branches and the per-load
// address arithmetic is one 32-bit multiply-add instead of 64-bit math.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
// Word 3 of the descriptor: 32-bit data format, the setting for raw
// (untyped) buffer access on gfx9-family parts.
constexpr int RSRC_WORD3 = 0x00020000;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, RSRC_WORD3);
}

// NW consecutive words at byte offset off (aligned to A bytes).
template <int NW, int A>
__device__ __forceinline__ void buffer_words(rsrc_t r, uint32_t off, u32 (&w)[NW]) {
    if constexpr (A == 16 && NW % 4 == 0) {
#pragma unroll
        for (int i = 0; i < NW / 4; ++i) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * i, 0, 0);
            w[4 * i + 0] = v[0]; w[4 * i + 1] = v[1]; w[4 * i + 2] = v[2]; w[4 * i + 3] = v[3];
        }
    } else if constexpr (A >= 8 && NW % 2 == 0) {
#pragma unroll
        for (int i = 0; i < NW / 2; ++i) {
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off + 8 * i, 0, 0);
            w[2 * i + 0] = v[0]; w[2 * i + 1] = v[1];
        }
    } else {
#pragma unroll
        for (int i = 0; i < NW; ++i) w[i] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * i, 0, 0);
    }
}

__device__ __forceinline__ void buffer_store_f32(float v, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(u32, v), r, off, 0, 0);
}

// Values the whole wave agrees on, made explicitly scalar.  Loads from a
// descriptor table that the kernel also writes through (outputs) cannot be
// proven invariant, so the compiler would treat them as per-lane values and
// wrap every buffer access in a loop over distinct values.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}
template <class T>
__device__ __forceinline__ T* uniform(T* p) {
    return reinterpret_cast<T*>(uniform(reinterpret_cast<int64_t>(p)));
}

__device__ __forceinline__ u32 buffer_u16(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ u32 buffer_u32(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
// 24-bit field t (codes at bits 0..23) -> low 12 bits kept, bits 12..23 moved
// to 16..27; bits 12..15 and 28..31 of the result are don't-care.
__device__ __forceinline__ u32 spread12(u32 t) {
    return (t & 0xFFFu) | ((t << 4) & 0xFFFFF000u);
}

template <int B> struct PairFmt;

// Q2: word j holds codes 16j..16j+15 at bits 2c.  Mask 0x00030003 << 2t picks
// codes t and t+8 (t < 4); after >> 8 the same masks pick t+4 and t+12.
template <> struct PairFmt<2> {
    static constexpr int NACC = 4;
    static constexpr int ka(int i) { return 16 * (i / 8) + (i % 8); }
    static constexpr int kb(int i) { return ka(i) + 8; }
    static constexpr int acc(int i) { return (i % 8) % 4; }
    static constexpr float inv_factor(int a) { return a == 0 ? 1.f : a == 1 ? 0.25f : a == 2 ? 0.0625f : 0.015625f; }
    __device__ static __forceinline__ void extract(const u32* w, u32* p) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const u32 v = w[j], v8 = w[j] >> 8;
#pragma unroll
            for (int t = 0; t < 8; ++t)
                p[8 * j + t] = mask_or_magic(t < 4 ? v : v8, 0x00030003u << (2 * (t % 4)));
        }
    }
};

// Q3: 3 words = 96 bits = four 24-bit pieces of 8 codes.  Each piece is
// spread so codes 0..3 sit at bits 0,3,6,9 and codes 4..7 at 16,19,22,25;
// then (c0,c4) x1, (c1,c5) x8, (c2,c6) x64 by masks and (c3,c7) x1 after >> 9.
template <> struct PairFmt<3> {
    static constexpr int NACC = 3;
    static constexpr int ka(int i) { return 8 * (i / 4) + (i % 4); }
    static constexpr int kb(int i) { return ka(i) + 4; }
    static constexpr int acc(int i) { return (i % 4) == 3 ? 0 : (i % 4); }
    static constexpr float inv_factor(int a) { return a == 0 ? 1.f : a == 1 ? 0.125f : 0.015625f; }
    __device__ static __forceinline__ void extract(const u32* w, u32* p) {
        const u32 t[4] = {w[0], funnel(w[1], w[0], 24), funnel(w[2], w[1], 16), w[2] >> 8};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32 u = spread12(t[q]);
            p[4 * q + 0] = mask_or_magic(u, 0x00070007u);
            p[4 * q + 1] = mask_or_magic(u, 0x00380038u);
            p[4 * q + 2] = mask_or_magic(u, 0x01C001C0u);
            p[4 * q + 3] = mask_or_magic(u >> 9, 0x00070007u);
        }
    }
};

// Q4: word j holds codes 8j..8j+7 as nibbles.  Mask 0x000F000F picks (c0,c4)
// x1, 0x00F000F0 picks (c1,c5) x16; after >> 8, (c2,c6) x1 and (c3,c7) x16.
template <> struct PairFmt<4> {
    static constexpr int NACC = 2;
    static constexpr int ka(int i) { return 8 * (i / 4) + (i % 4); }
    static constexpr int kb(int i) { return ka(i) + 4; }
    static constexpr int acc(int i) { return (i % 4) & 1; }
    static constexpr float inv_factor(int a) { return a == 0 ? 1.f : 0.0625f; }
    __device__ static __forceinline__ void extract(const u32* w, u32* p) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32 v = w[j], v8 = w[j] >> 8;
            p[4 * j + 0] = mask_or_magic(v, 0x000F000Fu);
            p[4 * j + 1] = mask_or_magic(v, 0x00F000F0u);
            p[4 * j + 2] = mask_or_magic(v8, 0x000F000Fu);
            p[4 * j + 3] = mask_or_magic(v8, 0x00F000F0u);
        }
    }
};

// 20-bit field t (codes at bits 0..19) -> low 10 bits kept, bits 10..19
// moved to 16..25; bits 10..15 and 26..31 of the result are don't-care.
__device__ __forceinline__ u32 spread10(u32 t) {
    return (t & 0x3FFu) | ((t << 6) & 0x03FF0000u);
}

// Q5: 5 words = 160 bits = eight 20-bit pieces of 4 codes.  Spread puts
// codes 0,1 at bits 0,5 and codes 2,3 at 16,21: mask 0x001F001F gives
// (c0,c2) x1 and mask 0x03E003E0 gives (c1,c3) x32 (32 * 31 < 1024, exact).
template <> struct PairFmt<5> {
    static constexpr int NACC = 2;
    static constexpr int ka(int i) { return 4 * (i / 2) + (i % 2); }
    static constexpr int kb(int i) { return ka(i) + 2; }
    static constexpr int acc(int i) { return i % 2; }
    static constexpr float inv_factor(int a) { return a == 0 ? 1.f : 0.03125f; }
    __device__ static __forceinline__ void extract(const u32* w, u32* p) {
        // Piece q starts at stream bit 20q.
        const u32 t[8] = {w[0], funnel(w[1], w[0], 20), w[1] >> 8, funnel(w[2], w[1], 28),
                          funnel(w[3], w[2], 16), w[3] >> 4, funnel(w[4], w[3], 24), w[4] >> 12};
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const u32 u = spread10(t[q]);
            p[2 * q + 0] = mask_or_magic(u, 0x001F001Fu);
            p[2 * q + 1] = mask_or_magic(u, 0x03E003E0u);
        }
    }
};

// Q6: 6 words = 192 bits = eight 24-bit pieces of 4 codes.  Spread puts
// codes 0,1 at bits 0,6 and codes 2,3 at 16,22: mask 0x003F003F gives (c0,c2),
// the same mask after >> 6 gives (c1,c3).
template <> struct PairFmt<6> {
    static constexpr int NACC = 2;
    static constexpr int ka(int i) { return 4 * (i / 2) + (i % 2); }
    static constexpr int kb(int i) { return ka(i) + 2; }
    static constexpr int acc(int i) { return i % 2; }
    static constexpr float inv_factor(int) { return 1.f; }
    __device__ static __forceinline__ void extract(const u32* w, u32* p) {
        const u32 t[8] = {w[0], funnel(w[1], w[0], 24), funnel(w[2], w[1], 16), w[2] >> 8,
                          w[3], funnel(w[4], w[3], 24), funnel(w[5], w[4], 16), w[5] >> 8};
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const u32 u = spread12(t[q]);
            p[2 * q + 0] = mask_or_magic(u, 0x003F003Fu);
            p[2 * q + 1] = mask_or_magic(u >> 6, 0x003F003Fu);
        }
    }
};

// Q8: word j holds codes 4j..4j+3 as bytes: (c0,c2) and, after >> 8, (c1,c3).
template <> struct PairFmt<8> {
    static constexpr int NACC = 2;
    static constexpr int ka(int i) { return 4 * (i / 2) + (i % 2); }
    static constexpr int kb(int i) { return ka(i) + 2; }
    static constexpr int acc(int i) { return i % 2; }
    static constexpr float inv_factor(int) { return 1.f; }
    __device__ static __forceinline__ void extract(const u32* w, u32* p) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            p[2 * j + 0] = mask_or_magic(w[j], 0x00FF00FFu);
            p[2 * j + 1] = mask_or_magic(w[j] >> 8, 0x00FF00FFu);
        }
    }
};

// Unquantized fp16 weights ("Q16"): the stream holds the fp16 values
// themselves, two per word in k order, so a word already is the pair
// (k, k+1).  No offset to remove and no scale or min: scale_value<16> is 1
// and the min arrays are never read.
template <> struct PairFmt<16> {
    static constexpr int NACC = 1;
    static constexpr int ka(int i) { return 2 * i; }
    static constexpr int kb(int i) { return 2 * i + 1; }
    static constexpr int acc(int) { return 0; }
    static constexpr float inv_factor(int) { return 1.f; }
    __device__ static __forceinline__ void extract(const u32* w, u32* p) {
#pragma unroll
        for (int i = 0; i < 16; ++i) p[i] = w[i];
    }
};
// Formats with a scale and a min per group (all but fp16).
template <int B>
constexpr bool has_affine() { return B != 16; }
// The group scale as a float; fp16 weights carry none.
template <int B>
__device__ __forceinline__ float scale_value(u32 bits) {
    if constexpr (has_affine<B>()) return half_bits_to_float((uint16_t)bits);
    return 1.f;
}

// Largest power-of-two alignment (<= 16 bytes) of a unit of `unit` codes at b
// bits, given 16-byte aligned rows... rows start at multiples of the unit's
// byte size, so the unit size alone decides.
constexpr int unit_align(int b, int unit) {
    const int bytes = unit * b / 8;
    return (bytes % 16 == 0) ? 16 : (bytes % 8 == 0) ? 8 : 4;
}

// Load NW consecutive words at p (aligned to A bytes) with the widest loads.
template <int NW, int A>
__device__ __forceinline__ void load_words(const u32* __restrict__ p, u32 (&w)[NW]) {
    if constexpr (A == 16 && NW % 4 == 0) {
#pragma unroll
        for (int i = 0; i < NW / 4; ++i) {
            const u32x4 v = reinterpret_cast<const u32x4*>(p)[i];
            w[4 * i + 0] = v[0]; w[4 * i + 1] = v[1]; w[4 * i + 2] = v[2]; w[4 * i + 3] = v[3];
        }
    } else if constexpr (A >= 8 && NW % 2 == 0) {
#pragma unroll
        for (int i = 0; i < NW / 2; ++i) {
            const u32x2 v = reinterpret_cast<const u32x2*>(p)[i];
            w[2 * i + 0] = v[0]; w[2 * i + 1] = v[1];
        }
    } else {
#pragma unroll
        for (int i = 0; i < NW; ++i) w[i] = p[i];
    }
}

// Activation-side state of one unit (UNIT consecutive codes of a row, inside
// one quantization group): the 16 pairs per chunk in extraction order, the
// offset constant to subtract, and the plain sum of the unit's activations.
template <int B, int UNIT>
struct XUnit {
    static constexpr int NP = UNIT / 2;
    f16x2 xp[NP];
    float corr;  // sum over pairs of 1024 * (x_a + x_b) * 2^-f
    float xsum;  // sum of the UNIT activations
};

// Build an XUnit from the UNIT fp16 activations at byte offset off of the
// activation buffer (16-byte aligned).
// (Split in two below: xunit_from_words converts words already loaded.)
template <int B, int UNIT>
__device__ __forceinline__ void xunit_from_words(const u32 (&xw)[UNIT / 2], XUnit<B, UNIT>& xu);

template <int B, int UNIT>
__device__ __forceinline__ void prep_xunit(rsrc_t xr, uint32_t off, XUnit<B, UNIT>& xu) {
    u32 xw[UNIT / 2];
    buffer_words<UNIT / 2, 16>(xr, off, xw);
    xunit_from_words<B, UNIT>(xw, xu);
}

template <int B, int UNIT>
__device__ __forceinline__ void xunit_from_words(const u32 (&xw)[UNIT / 2], XUnit<B, UNIT>& xu) {
    using F = PairFmt<B>;
    // Both constants come from packed dot products on the pairs themselves:
    // corr += x_a * c + x_b * c with c = 1024 * 2^-f (exact in fp16), and
    // xsum += x_a + x_b.  No per-element conversions, few live registers.
    float corr = 0.f, xsum = 0.f;
    const f16x2 one2 = {(f16)1.0f, (f16)1.0f};
#pragma unroll
    for (int c = 0; c < UNIT / 32; ++c) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int a = 32 * c + F::ka(i), b = 32 * c + F::kb(i);
            const u32 lo = (xw[a / 2] >> (16 * (a % 2))) & 0xFFFFu;
            const u32 hi = (xw[b / 2] >> (16 * (b % 2))) & 0xFFFFu;
            const f16x2 pr = as_h2(lo | (hi << 16));
            xu.xp[16 * c + i] = pr;
            if constexpr (has_affine<B>()) {
                const f16 cf = (f16)(1024.0f * F::inv_factor(F::acc(i)));
                corr = __builtin_amdgcn_fdot2(pr, f16x2{cf, cf}, corr, false);
            }
            xsum = __builtin_amdgcn_fdot2(pr, one2, xsum, false);
        }
    }
    xu.corr = corr;
    xu.xsum = xsum;
}

template <int B, int UNIT>
__device__ __forceinline__ void zero_xunit(XUnit<B, UNIT>& xu) {
#pragma unroll
    for (int i = 0; i < UNIT / 2; ++i) xu.xp[i] = as_h2(0u);
    xu.corr = 0.f;
    xu.xsum = 0.f;
}

// sum_k q_k x_k over one unit, from its packed words (UNIT*B/32 of them).
template <int B, int UNIT>
__device__ __forceinline__ float unit_qx(const u32* w, const XUnit<B, UNIT>& xu) {
    using F = PairFmt<B>;
    float acc[F::NACC];
#pragma unroll
    for (int a = 0; a < F::NACC; ++a) acc[a] = 0.f;
#pragma unroll
    for (int c = 0; c < UNIT / 32; ++c) {
        u32 p[16];
        F::extract(w + c * B, p);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            acc[F::acc(i)] = __builtin_amdgcn_fdot2(as_h2(p[i]), xu.xp[16 * c + i], acc[F::acc(i)], false);
    }
    float t = acc[0];
#pragma unroll
    for (int a = 1; a < F::NACC; ++a) t = __builtin_fmaf(acc[a], F::inv_factor(a), t);
    return t - xu.corr;
}

// Sum over aligned groups of L lanes (L = 16, 32 or 64); every lane of the
// group gets the total.  Within a 16-lane row the butterfly runs on DPP
// lane swizzles folded into the adds (xor 1, xor 2, then the half-row and
// row mirrors, which pair each lane with one holding the complementary
// partial sum); across rows one ds_swizzle (xor 16) and one cross-lane
// permute (xor 32).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f32<0x141>(v);  // row_half_mirror
    v += dpp_f32<0x140>(v);  // row_mirror
    return v;
}
__device__ __forceinline__ float xor16_add(float v) {
    return v + __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}
__device__ __forceinline__ float xor32_add(float v) { return v + __shfl_xor(v, 32, 64); }

template <int L>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(L == 16 || L == 32 || L == 64, "lanes per row");
    v = row16_sum(v);
    if constexpr (L >= 32) v = xor16_add(v);
    if constexpr (L == 64) v = xor32_add(v);
    return v;
}
// Same with a wave-uniform run-time width (16, 32 or 64).
__device__ __forceinline__ float group_sum_rt(float v, int lanes) {
    v = row16_sum(v);
    if (lanes >= 32) v = xor16_add(v);
    if (lanes == 64) v = xor32_add(v);
    return v;
}

}  // namespace qmm
