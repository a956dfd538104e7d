// unpack.hip -- packed codes to bytes, a bit-exact view of the format used to
// check the GPU's reading of the bitstream against the CPU's.
//
// Format: code k of row n sits at stream bits [k*b, k*b+b) of the row's
// bitstream; stream bit i is bit i%32 of word i/32 (the library's definition;
// the pages only name "affine quantization Q2 to Q8", "Apple Silicon 로컬 LLM
// 추론의 새 기준 BaseRT", section "BaseRT는 무엇인가").
#include "qmm_device.h"
#include "qmm_kernels.h"

namespace qmm {

// One thread per 32-code chunk (b words in, 32 bytes out).
template <int B>
__global__ __launch_bounds__(256) void unpack_kernel(const u32* __restrict__ W,
                                                     uint8_t* __restrict__ codes,
                                                     int64_t chunks, int64_t chunks_per_row) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= chunks) return;
    const int64_t row = t / chunks_per_row;
    const int64_t c = t - row * chunks_per_row;
    const u32* p = W + row * chunks_per_row * B + c * B;
    u32 w[B + 1];
#pragma unroll
    for (int i = 0; i < B; ++i) w[i] = p[i];
    w[B] = 0u;
    u32 out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = 0u;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const int bit = i * B;
        const u32 lo = w[bit / 32], hi = w[bit / 32 + 1];
        const u32 v = (bit % 32) ? ((lo >> (bit % 32)) | (hi << (32 - bit % 32))) : lo;
        out[i / 4] |= (v & ((1u << B) - 1u)) << (8 * (i % 4));
    }
    u32x4* dst = reinterpret_cast<u32x4*>(codes + row * chunks_per_row * 32 + c * 32);
    dst[0] = u32x4{out[0], out[1], out[2], out[3]};
    dst[1] = u32x4{out[4], out[5], out[6], out[7]};
}

hipError_t launch_unpack(const uint32_t* w, uint8_t* codes, int64_t n, int64_t k, int bits,
                         hipStream_t st) {
    const int64_t cpr = k / 32;
    const int64_t chunks = n * cpr;
    const int64_t grid = (chunks + 255) / 256;
    switch (bits) {
#define CASE(B)                                                                                 \
    case B:                                                                                     \
        hipLaunchKernelGGL(unpack_kernel<B>, dim3((unsigned)grid), dim3(256), 0, st, w, codes, \
                           chunks, cpr);                                                        \
        break;
        CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(8)
#undef CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace qmm
