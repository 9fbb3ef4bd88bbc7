// hbm_probe.hip -- host side and kernels of include/epdc_probe.h: streaming
// read, write and copy kernels that measure the card's HBM rates in each
// direction.  They move bytes and nothing else; the benchmark compares the
// dispatch and combine kernels with them.
#include "epdc_probe.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kReadVecs = 8;  // loads in flight per thread: 32 KiB per block
constexpr int kCopyVecs = 4;  // vectors per thread: 16 KiB per block

thread_local std::string g_last_error;

epdc_status fail(epdc_status s, const char *fmt, ...)
{
    char buf[256];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

__global__ __launch_bounds__(kThreads) void k_probe_read(const u32x4 *src, int64_t vecs,
                                                         uint32_t magic, uint32_t *flag)
{
    const int64_t base = (int64_t)blockIdx.x * kThreads * kReadVecs + threadIdx.x;
    u32x4 v[kReadVecs];
#pragma unroll
    for (int i = 0; i < kReadVecs; ++i) {
        const int64_t j = base + (int64_t)i * kThreads;
        v[i] = j < vecs ? __builtin_nontemporal_load(src + j) : u32x4{0u, 0u, 0u, 0u};
    }
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < kReadVecs; ++i)
        x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    // fold the block's words so one lane decides
    for (int d = 32; d >= 1; d >>= 1)
        x ^= __shfl_xor(x, d, 64);
    __shared__ uint32_t wave_x[kThreads / 64];
    if ((threadIdx.x & 63) == 0)
        wave_x[threadIdx.x / 64] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t b = 0;
        for (int w = 0; w < kThreads / 64; ++w)
            b ^= wave_x[w];
        if (b == magic)
            flag[0] = magic;
    }
}

__global__ __launch_bounds__(kThreads) void k_probe_write(u32x4 *dst, int64_t vecs, uint32_t value)
{
    const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (j < vecs)
        dst[j] = u32x4{value, value ^ 1u, value ^ 2u, value ^ 3u};
}

__global__ __launch_bounds__(kThreads) void k_probe_copy(const u32x4 *src, u32x4 *dst, int64_t vecs)
{
    const int64_t base = (int64_t)blockIdx.x * kThreads * kCopyVecs + threadIdx.x;
    u32x4 v[kCopyVecs];
#pragma unroll
    for (int i = 0; i < kCopyVecs; ++i) {
        const int64_t j = base + (int64_t)i * kThreads;
        if (j < vecs)
            v[i] = __builtin_nontemporal_load(src + j);
    }
#pragma unroll
    for (int i = 0; i < kCopyVecs; ++i) {
        const int64_t j = base + (int64_t)i * kThreads;
        if (j < vecs)
            dst[j] = v[i];
    }
}

epdc_status check_buffer(const void *p, size_t bytes, const char *name)
{
    if (!p)
        return fail(EPDC_ERR_INVALID_ARGS, "%s is NULL", name);
    if (((uintptr_t)p & 15u) != 0)
        return fail(EPDC_ERR_INVALID_ARGS, "%s must be 16-byte aligned", name);
    if (bytes == 0 || bytes % 16 != 0)
        return fail(EPDC_ERR_INVALID_ARGS, "bytes must be a positive multiple of 16, got %zu",
                    bytes);
    return EPDC_SUCCESS;
}

// Blocks of `vecs_per_block` vectors covering `vecs`, or -1 past one launch.
int64_t grid_for(int64_t vecs, int64_t vecs_per_block)
{
    const int64_t g = (vecs + vecs_per_block - 1) / vecs_per_block;
    return g <= 0x7FFFFFFF ? g : -1;
}

epdc_status launched(const char *what)
{
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(EPDC_ERR_GPU_OP, "%s launch failed: %s", what, hipGetErrorString(e));
    g_last_error.clear();
    return EPDC_SUCCESS;
}

}  // namespace

extern "C" {

epdc_status epdc_probe_read(const void *src, size_t bytes, uint32_t magic, uint32_t *flag,
                            void *stream)
{
    epdc_status s = check_buffer(src, bytes, "src");
    if (s != EPDC_SUCCESS)
        return s;
    if (!flag || ((uintptr_t)flag & 3u) != 0)
        return fail(EPDC_ERR_INVALID_ARGS, "flag must be a 4-byte aligned device pointer");
    const int64_t vecs = (int64_t)(bytes / 16);
    const int64_t grid = grid_for(vecs, (int64_t)kThreads * kReadVecs);
    if (grid < 0)
        return fail(EPDC_ERR_INVALID_ARGS, "%zu bytes do not fit one launch", bytes);
    k_probe_read<<<(unsigned)grid, kThreads, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const u32x4 *>(src), vecs, magic, flag);
    return launched("k_probe_read");
}

epdc_status epdc_probe_write(void *dst, size_t bytes, uint32_t value, void *stream)
{
    epdc_status s = check_buffer(dst, bytes, "dst");
    if (s != EPDC_SUCCESS)
        return s;
    const int64_t vecs = (int64_t)(bytes / 16);
    const int64_t grid = grid_for(vecs, kThreads);
    if (grid < 0)
        return fail(EPDC_ERR_INVALID_ARGS, "%zu bytes do not fit one launch", bytes);
    k_probe_write<<<(unsigned)grid, kThreads, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<u32x4 *>(dst), vecs, value);
    return launched("k_probe_write");
}

epdc_status epdc_probe_copy(const void *src, void *dst, size_t bytes, void *stream)
{
    epdc_status s = check_buffer(src, bytes, "src");
    if (s == EPDC_SUCCESS)
        s = check_buffer(dst, bytes, "dst");
    if (s != EPDC_SUCCESS)
        return s;
    const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
    if (a < b + bytes && b < a + bytes)
        return fail(EPDC_ERR_INVALID_ARGS, "src and dst overlap");
    const int64_t vecs = (int64_t)(bytes / 16);
    const int64_t grid = grid_for(vecs, (int64_t)kThreads * kCopyVecs);
    if (grid < 0)
        return fail(EPDC_ERR_INVALID_ARGS, "%zu bytes do not fit one launch", bytes);
    k_probe_copy<<<(unsigned)grid, kThreads, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), vecs);
    return launched("k_probe_copy");
}

const char *epdc_probe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
