// Measurement helpers (not part of the layer): the achievable ceilings the
// layer's kernels are compared with beside the vendor peaks.
//  * a matrix-core loop: every wavefront issues v_mfma_f32_32x32x16_bf16 back
//    to back on register operands, four independent accumulators round robin
//    (enough to keep the pipeline full), no memory traffic;
//  * a streaming copy and a streaming read of large buffers with 16-byte
//    accesses, the HBM ceilings of copy-like and read-like kernels.
#include "common.hpp"
#include "moe_ceiling.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* __restrict__ sink)
{
    typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
    const int lane = threadIdx.x & 63;
    bf8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (lane + i));
        b[i] = (__bf16)(0.002f * (lane - i));
    }
    f32x16 acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[q][r] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[q], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[q][r];
    // one store per block keeps the accumulators live
    if (s == 12345.678f || threadIdx.x == 0) sink[blockIdx.x] = s;
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, long long n)
{
    const long long stride = (long long)gridDim.x * 256 * 4;
    for (long long i = (long long)blockIdx.x * 1024 + threadIdx.x; i < n; i += stride) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i + 256 * u < n) v[u] = __builtin_nontemporal_load(src + i + 256 * u);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i + 256 * u < n) __builtin_nontemporal_store(v[u], dst + i + 256 * u);
    }
}

__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, long long n,
                                                   unsigned* __restrict__ sink)
{
    const long long stride = (long long)gridDim.x * 256 * 4;
    unsigned acc = 0;
    for (long long i = (long long)blockIdx.x * 1024 + threadIdx.x; i < n; i += stride) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i + 256 * u < n) {
                const u32x4 v = __builtin_nontemporal_load(src + i + 256 * u);
                acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
            }
    }
    if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;   // practically never: keeps the loads
}

}  // namespace
}  // namespace moe

extern "C" {

long long moe_ceiling_mfma(int blocks, int iters, float* sink, void* stream)
{
    if (blocks <= 0 || iters <= 0 || !sink) return -1;
    moe::mfma_loop_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(iters, sink);
    if (hipGetLastError() != hipSuccess) return -1;
    // 4 wavefronts x iters x 8 MFMAs x 32*32*16*2 flop
    return (long long)blocks * 4 * iters * 8 * (32LL * 32 * 16 * 2);
}

int moe_ceiling_copy(const void* src, void* dst, long long bytes, int blocks, void* stream)
{
    if (!src || !dst || bytes <= 0 || bytes % 16 || blocks <= 0) return -1;
    moe::copy_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const moe::u32x4*>(src), static_cast<moe::u32x4*>(dst), bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int moe_ceiling_read(const void* src, long long bytes, unsigned* sink, int blocks, void* stream)
{
    if (!src || !sink || bytes <= 0 || bytes % 16 || blocks <= 0) return -1;
    moe::read_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const moe::u32x4*>(src), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
