// qknr_bench.hip -- plain streaming kernels used to measure the achievable HBM
// bandwidth of an MI355X (gfx950) beside the QK-Norm + RoPE kernels, an empty
// kernel that measures the cost of a dispatch, and a fill that evicts the
// caches between timed launches.  Not part of the operation; built
// as its own library (libqknr_bench.so) for the benchmark and its tests.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "qknr_bench.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

__global__ __launch_bounds__(256) void bench_stream2_kernel(const u32x4 *__restrict__ a,
                                                           const u32x4 *__restrict__ b,
                                                           u32x4 *__restrict__ dst, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x * 4 + threadIdx.x; i < n; i += stride) {
        u32x4 v[4], w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i + u * 256 < n) {
                v[u] = __builtin_nontemporal_load(a + i + u * 256);
                w[u] = __builtin_nontemporal_load(b + i + u * 256);
            }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i + u * 256 < n)
                __builtin_nontemporal_store(v[u] ^ w[u], dst + i + u * 256);
    }
}

__global__ __launch_bounds__(256) void bench_copy_kernel(const u32x4 *__restrict__ src,
                                                        u32x4 *__restrict__ dst, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x * 4 + threadIdx.x; i < n; i += stride) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i + u * 256 < n)
                v[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i + u * 256 < n)
                __builtin_nontemporal_store(v[u], dst + i + u * 256);
    }
}

__global__ __launch_bounds__(256) void bench_flush_kernel(u32x4 *__restrict__ buf, int64_t n,
                                                         uint32_t seed)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const uint32_t v = (uint32_t)i ^ seed;
        buf[i] = (u32x4){v, v + 1, v + 2, v + 3};
    }
}

// Does nothing: its launch measures the dispatch cost alone.
__global__ __launch_bounds__(64) void bench_empty_kernel() {}

}  // namespace

extern "C" {

int qknr_bench_empty(void *stream)
{
    hipLaunchKernelGGL(bench_empty_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? QKNR_BENCH_OK : QKNR_BENCH_ERR_HIP;
}

int qknr_bench_copy(const void *src, void *dst, size_t bytes, void *stream)
{
    if (bytes == 0)
        return QKNR_BENCH_OK;
    if (!src || !dst)
        return QKNR_BENCH_ERR_INVALID_ARG;
    if (!aligned(src, 16) || !aligned(dst, 16) || bytes % 16 != 0)
        return QKNR_BENCH_ERR_MISALIGNED;
    const int64_t n = (int64_t)(bytes / 16);
    int64_t blocks = (n + 1023) / 1024;
    if (blocks > 256 * 64)
        blocks = 256 * 64;
    hipLaunchKernelGGL(bench_copy_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(src),
                       static_cast<u32x4 *>(dst), n);
    return hipGetLastError() == hipSuccess ? QKNR_BENCH_OK : QKNR_BENCH_ERR_HIP;
}

int qknr_bench_stream2(const void *a, const void *b, void *dst, size_t bytes, void *stream)
{
    if (bytes == 0)
        return QKNR_BENCH_OK;
    if (!a || !b || !dst)
        return QKNR_BENCH_ERR_INVALID_ARG;
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(dst, 16) || bytes % 16 != 0)
        return QKNR_BENCH_ERR_MISALIGNED;
    const int64_t n = (int64_t)(bytes / 16);
    int64_t blocks = (n + 1023) / 1024;
    if (blocks > 256 * 64)
        blocks = 256 * 64;
    hipLaunchKernelGGL(bench_stream2_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(a),
                       static_cast<const u32x4 *>(b), static_cast<u32x4 *>(dst), n);
    return hipGetLastError() == hipSuccess ? QKNR_BENCH_OK : QKNR_BENCH_ERR_HIP;
}

int qknr_bench_flush(void *buf, size_t bytes, uint32_t seed, void *stream)
{
    if (bytes == 0)
        return QKNR_BENCH_OK;
    if (!buf)
        return QKNR_BENCH_ERR_INVALID_ARG;
    if (!aligned(buf, 16) || bytes % 16 != 0)
        return QKNR_BENCH_ERR_MISALIGNED;
    const int64_t n = (int64_t)(bytes / 16);
    int64_t blocks = (n + 255) / 256;
    if (blocks > 256 * 64)
        blocks = 256 * 64;
    hipLaunchKernelGGL(bench_flush_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<u32x4 *>(buf), n, seed);
    return hipGetLastError() == hipSuccess ? QKNR_BENCH_OK : QKNR_BENCH_ERR_HIP;
}

}  // extern "C"
