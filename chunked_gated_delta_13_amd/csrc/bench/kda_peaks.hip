// Bandwidth probes for the benchmark harness (libkda_peaks.so, not part of libkda): a read stream,
// a device copy and an in-place read-modify-write of known byte counts, so that the kernels'
// achieved HBM rates can be set against what this GPU streams.  Each workgroup streams one
// contiguous range with 16-byte non-temporal accesses; the workgroups per compute unit are the
// fastest of a sweep on the MI355X (contiguous ranges beat grid-stride order by about 10%).  The
// read-modify-write takes the shape that streamed fastest in a sweep of state-update layouts: one
// 64 KiB block per 1024-thread workgroup, blocks dealt so that each XCD streams one contiguous range.
#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

typedef __attribute__((ext_vector_type(4))) float f4_t;

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int kReadBlocksPerCU = 2;
constexpr int kCopyBlocksPerCU = 8;
constexpr int kRmwThreads = 1024;
constexpr size_t kRmwBlock4 = 4096;   // 16-byte elements per read-modify-write block (64 KiB)

__device__ __forceinline__ void block_range(size_t n4, size_t* b0, size_t* b1) {
    const size_t per = (n4 + gridDim.x - 1) / gridDim.x;
    *b0 = (size_t)blockIdx.x * per;
    *b1 = *b0 + per < n4 ? *b0 + per : n4;
}

__global__ __launch_bounds__(kThreads) void read_stream(const f4_t* __restrict__ src, size_t n4, float* sink) {
    size_t b0, b1;
    block_range(n4, &b0, &b1);
    size_t i = b0 + threadIdx.x;
    f4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (; i + (kUnroll - 1) * kThreads < b1; i += kUnroll * kThreads) {
        f4_t v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc += v[u];
    }
    for (; i < b1; i += kThreads) acc += __builtin_nontemporal_load(src + i);
    // one value per thread keeps the loads live (a vector store per thread)
    sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc[0] + acc[1] + acc[2] + acc[3];
}

__global__ __launch_bounds__(kThreads) void copy_stream(f4_t* __restrict__ dst, const f4_t* __restrict__ src, size_t n4) {
    size_t b0, b1;
    block_range(n4, &b0, &b1);
    size_t i = b0 + threadIdx.x;
    for (; i + (kUnroll - 1) * kThreads < b1; i += kUnroll * kThreads) {
        f4_t v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * kThreads);
    }
    for (; i < b1; i += kThreads) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// x <- a x + b in place (the access pattern of a state read-modify-write).  Workgroups are dealt
// to the 8 XCDs in turn, so workgroup w takes block (w mod 8) * per + w / 8: each XCD's L2 sees
// one contiguous range.  The grid is 8 * per; blocks at or past nblk return at once.  Whole blocks
// run without per-element checks (checks around each access cost a quarter of the rate); only a
// last, partial block checks its bounds.
__global__ __launch_bounds__(kRmwThreads) void rmw_blocks(f4_t* __restrict__ x, size_t n4, size_t nblk, float a, float b) {
    const size_t per = (nblk + 7) / 8;
    const size_t blk = (size_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
    if (blk >= nblk) return;
    constexpr int kPer = (int)(kRmwBlock4 / kRmwThreads);
    f4_t* p = x + blk * kRmwBlock4 + threadIdx.x;
    if ((blk + 1) * kRmwBlock4 <= n4) {
        f4_t v[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) v[u] = __builtin_nontemporal_load(p + u * kRmwThreads);
#pragma unroll
        for (int u = 0; u < kPer; ++u) __builtin_nontemporal_store(v[u] * a + b, p + u * kRmwThreads);
        return;
    }
    const size_t left = n4 - blk * kRmwBlock4;   // 0 < left < kRmwBlock4
    for (size_t i = threadIdx.x; i < left; i += kRmwThreads)
        __builtin_nontemporal_store(__builtin_nontemporal_load(x + blk * kRmwBlock4 + i) * a + b, x + blk * kRmwBlock4 + i);
}

int cu_count() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    return cus;
}

bool ok16(const void* p) { return (uintptr_t)p % 16 == 0; }

}  // namespace

extern "C" {

// Number of floats `sink` must hold for kda_peak_read.
size_t kda_peak_read_sink_floats(void) { return (size_t)cu_count() * kReadBlocksPerCU * kThreads; }

// Reads `bytes` (a multiple of 16, 16-byte aligned) from device memory `src`; writes one float per
// thread to `sink` (kda_peak_read_sink_floats() floats).  0 on success, 1 on bad arguments,
// 2 on a launch failure.
int kda_peak_read(const void* src, size_t bytes, float* sink, void* stream) {
    if (!src || !sink || bytes % 16 != 0 || !ok16(src)) return 1;
    hipLaunchKernelGGL(read_stream, dim3(cu_count() * kReadBlocksPerCU), dim3(kThreads), 0, (hipStream_t)stream,
                       (const f4_t*)src, bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Copies `bytes` (a multiple of 16, both pointers 16-byte aligned, not overlapping) from src to dst.
int kda_peak_copy(void* dst, const void* src, size_t bytes, void* stream) {
    if (!src || !dst || bytes % 16 != 0 || !ok16(src) || !ok16(dst)) return 1;
    const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
    if (a < b + bytes && b < a + bytes) return 1;
    hipLaunchKernelGGL(copy_stream, dim3(cu_count() * kCopyBlocksPerCU), dim3(kThreads), 0, (hipStream_t)stream,
                       (f4_t*)dst, (const f4_t*)src, bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// x <- a x + b over `bytes` (a multiple of 16, 16-byte aligned) of fp32 in place: each byte is
// read once and written once.
int kda_peak_rmw(void* x, size_t bytes, float a, float b, void* stream) {
    if (!x || bytes % 16 != 0 || !ok16(x)) return 1;
    const size_t n4 = bytes / 16, nblk = (n4 + kRmwBlock4 - 1) / kRmwBlock4;
    if (nblk == 0) return 0;
    const size_t grid = 8 * ((nblk + 7) / 8);
    if (grid > 0x7fffffffu) return 1;
    hipLaunchKernelGGL(rmw_blocks, dim3((unsigned)grid), dim3(kRmwThreads), 0, (hipStream_t)stream, (f4_t*)x, n4,
                       nblk, a, b);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
