// On-device prefix scan over sequence segments, and a small state copy.
//
// Sources: "Kimi K3" (meridianbulletin.com), "Parallelizing Sequential State
// Updates" (each piece of the sequence contributes a transition and an
// increment, and a prefix scan over the pieces recovers the same states as
// the token-by-token run); "Kimi K3's architecture" (orkas.ai), "The bill
// comes due in the serving stack" (the per-segment transition and the state
// reached from zero combine exactly across segments).
//
// Entry state of segment s:  S_in(0) = S0,  S_in(s+1) = M_s S_in(s) + H_s.  With s_first = 1 the
// walk starts from S_in(1), already written by the pass that ran segment 0 from S0.
// State columns are independent, so a workgroup owns (head, 16 columns) and
// keeps that column block of S_in in LDS while it walks the segments.  fp32
// throughout; the n_seg - 1 steps are tiny next to the chunk passes around them.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int DK>
__global__ __launch_bounds__(256) void kda_scan_kernel(const ScanArgs a) {
    constexpr int CB = 16;               // columns per workgroup
    constexpr int NCB = DK / CB;
    constexpr int TPR = 256 / DK;        // threads per row
    constexpr int CPT = CB / TPR;        // columns per thread
    const int bh = blockIdx.x / NCB;
    const int cb = blockIdx.x % NCB;
    if (bh >= a.BH) return;
    const int tid = threadIdx.x;
    const int row = tid / TPR;
    const int c0 = cb * CB + (tid % TPR) * CPT;
    constexpr long long SS = (long long)DK * DK;

    __shared__ float sS[DK][CB + 1];
    float cur[CPT];
    float* sin = a.S_in + (long long)bh * a.n_seg * SS;
    if (a.s_first == 0) {
        const float* s0 = a.S0 ? a.S0 + bh * SS : nullptr;
#pragma unroll
        for (int j = 0; j < CPT; ++j) cur[j] = s0 ? s0[(long long)row * DK + c0 + j] : 0.0f;
#pragma unroll
        for (int j = 0; j < CPT; ++j) sin[(long long)row * DK + c0 + j] = cur[j];
    } else {
#pragma unroll
        for (int j = 0; j < CPT; ++j) cur[j] = sin[(long long)a.s_first * SS + (long long)row * DK + c0 + j];
    }

    for (int s = a.s_first; s + 1 < a.n_seg; ++s) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < CPT; ++j) sS[row][c0 - cb * CB + j] = cur[j];
        __syncthreads();
        const float* M = a.M + ((long long)bh * (a.n_seg - 1) + s) * SS + (long long)row * DK;
        const float* Hs = a.Hinc + ((long long)bh * (a.n_seg - 1) + s) * SS + (long long)row * DK;
        float acc[CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j) acc[j] = Hs[c0 + j];
        for (int m = 0; m < DK; m += 4) {
            const f32x4_t mv = *reinterpret_cast<const f32x4_t*>(M + m);
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int j = 0; j < CPT; ++j) acc[j] += mv[u] * sS[m + u][c0 - cb * CB + j];
        }
        float* dst = sin + (long long)(s + 1) * SS + (long long)row * DK + c0;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            cur[j] = acc[j];
            dst[j] = acc[j];
        }
    }
}

__global__ __launch_bounds__(256) void kda_state_copy_kernel(float* dst, const float* src, long long n) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.0f;
}

hipError_t launch_scan(int dk, const ScanArgs& a, hipStream_t stream) {
    if (a.BH <= 0 || a.n_seg <= 0) return hipSuccess;
    if (a.s_first < 0 || a.s_first >= a.n_seg) return hipErrorInvalidValue;
    const long long nblk = (long long)a.BH * (dk / 16);
    if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
    if (dk == 128) hipLaunchKernelGGL(kda_scan_kernel<128>, dim3((unsigned)nblk), dim3(256), 0, stream, a);
    else if (dk == 64) hipLaunchKernelGGL(kda_scan_kernel<64>, dim3((unsigned)nblk), dim3(256), 0, stream, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_state_copy(float* dst, const float* src, long long n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const long long nblk = (n + 255) / 256;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kda_state_copy_kernel, dim3((unsigned)nblk), dim3(256), 0, stream, dst, src, n);
    return hipGetLastError();
}

}  // namespace kda
