// ceiling.hip -- measured ceilings for the roofline (libqmm_ceiling.so).
//
// Two plain kernels whose rates bound what the library's kernels can reach
// on the machine at hand, reported next to the spec peaks:
//   * a streaming read of a device buffer (16-byte loads, four in flight per
//     thread, XOR-folded so the compiler keeps them): HBM read bandwidth;
//   * a loop of independent v_mfma_f32_32x32x16_f16 on every SIMD: dense fp16
//     matrix-core throughput.
// Measurement only: nothing in the quantized-matmul path uses them.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ p, uint64_t n16,
                                                   uint32_t* __restrict__ sink) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        const u32x4 a = p[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    // Never true for the buffers the caller fills; keeps the loads live.
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

__global__ __launch_bounds__(256) void mfma_kernel(int iters, float* __restrict__ sink) {
    f16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (_Float16)(1.0f / (float)(threadIdx.x + j + 1));
        b[j] = (_Float16)(1.0f / (float)(threadIdx.x + 2 * j + 3));
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c3, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) s += c0[v] + c1[v] + c2[v] + c3[v];
    if (s == -1.0f) sink[0] = s;  // the sums are positive: never taken
}

}  // namespace

extern "C" {

// Streaming read of `bytes` (a multiple of 16) from a 16-byte aligned device
// buffer with `blocks` work-groups of 256 threads.  `sink`: a device word the
// kernel never writes for buffers filled with anything but one pattern.
__attribute__((visibility("default"))) int qmm_ceiling_read(const void* buf, uint64_t bytes, int blocks,
                                                            void* sink, void* stream) {
    if (!buf || !sink || bytes % 16 || blocks <= 0) return 1;
    hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const u32x4*>(buf), bytes / 16, static_cast<uint32_t*>(sink));
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

// `blocks` work-groups of four waves, each wave issuing 4 * iters
// 32x32x16 fp16 MFMAs (32768 flops each).
__attribute__((visibility("default"))) int qmm_ceiling_mfma(int blocks, int iters, void* sink, void* stream) {
    if (!sink || blocks <= 0 || iters <= 0) return 1;
    hipLaunchKernelGGL(mfma_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters,
                       static_cast<float*>(sink));
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
