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
// keeps that column block of S_in in LDS while it walks the segments; each
// thread holds one row of the step's transition in registers (the next step's
// row is requested before the current step's products).  fp32 throughout, with
// each entry summed over m in order (the same sums as one row-by-row product).
// A step whose transition died out (the transition pass stored it as zeros and
// recorded a chunk count) is S_in(s+1) = H_s: its transition is neither read nor
// multiplied, which gives the same bits.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int DK>
__global__ __launch_bounds__(256) void kda_scan_kernel(const ScanArgs a) {
    constexpr int CB = 16;               // columns per workgroup
    constexpr int NCB = DK / CB;
    constexpr int TPR = 256 / DK;        // threads per row
    constexpr int CPT = CB / TPR;        // columns per thread (8 or 4)
    constexpr int NQ = CPT / 4;          // float4 groups per thread
    static_assert(CPT % 4 == 0, "whole float4 column groups per thread");
    const int bh = blockIdx.x / NCB;
    const int cb = blockIdx.x % NCB;
    if (bh >= a.BH) return;
    const int tid = threadIdx.x;
    const int row = tid / TPR;
    const int cl = (tid % TPR) * CPT;    // first column of this thread inside the block
    const int c0 = cb * CB + cl;
    constexpr long long SS = (long long)DK * DK;

    // the current entry state's column block, rows 16-byte aligned (every lane of a wave reads the
    // same row at a time: broadcast reads)
    __shared__ __attribute__((aligned(16))) float sS[DK][CB];
    f32x4_t cur[NQ];
    float* sin = a.S_in + (long long)bh * a.n_seg * SS;
    if (a.s_first == 0) {
        const float* s0 = a.S0 ? a.S0 + bh * SS : nullptr;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            cur[q] = s0 ? *reinterpret_cast<const f32x4_t*>(s0 + (long long)row * DK + c0 + 4 * q) : zero4();
            *reinterpret_cast<f32x4_t*>(sin + (long long)row * DK + c0 + 4 * q) = cur[q];
        }
    } else {
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            cur[q] = *reinterpret_cast<const f32x4_t*>(sin + (long long)a.s_first * SS + (long long)row * DK + c0 + 4 * q);
    }

    // row `row` of M_s and this thread's columns of H_s, for the step being computed and the next
    auto mrow_of = [&](int s) { return a.M + ((long long)bh * (a.n_seg - 1) + s) * SS + (long long)row * DK; };
    auto hrow_of = [&](int s) { return a.Hinc + ((long long)bh * (a.n_seg - 1) + s) * SS + (long long)row * DK + c0; };
    // a step whose transition died (the transition pass stored it as zeros) adds nothing to H_s:
    // its rows are not read and its product is skipped (workgroup-uniform)
    auto dead = [&](int s) { return a.z != nullptr && split_count(a.z, a.n_seg, a.n_vs, bh, s) >= 0; };
    f32x4_t mr[DK / 4], hr[NQ];
    bool dead_cur = false;
    if (a.s_first + 1 < a.n_seg) {
        dead_cur = dead(a.s_first);
        const float* M = mrow_of(a.s_first);
        const float* Hs = hrow_of(a.s_first);
        if (!dead_cur) {
#pragma unroll
            for (int m = 0; m < DK / 4; ++m) mr[m] = *reinterpret_cast<const f32x4_t*>(M + 4 * m);
        }
#pragma unroll
        for (int q = 0; q < NQ; ++q) hr[q] = *reinterpret_cast<const f32x4_t*>(Hs + 4 * q);
    }
    for (int s = a.s_first; s + 1 < a.n_seg; ++s) {
        __syncthreads();
#pragma unroll
        for (int q = 0; q < NQ; ++q) *reinterpret_cast<f32x4_t*>(&sS[row][cl + 4 * q]) = cur[q];
        __syncthreads();
        // next step's operands requested before this step's products
        f32x4_t mn[DK / 4], hn[NQ];
        const bool more = s + 2 < a.n_seg;
        const bool dead_next = more && dead(s + 1);
        if (more) {
            const float* M = mrow_of(s + 1);
            const float* Hs = hrow_of(s + 1);
            if (!dead_next) {
#pragma unroll
                for (int m = 0; m < DK / 4; ++m) mn[m] = *reinterpret_cast<const f32x4_t*>(M + 4 * m);
            }
#pragma unroll
            for (int q = 0; q < NQ; ++q) hn[q] = *reinterpret_cast<const f32x4_t*>(Hs + 4 * q);
        }
        f32x4_t acc[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) acc[q] = hr[q];
        if (!dead_cur) {
#pragma unroll
        for (int m = 0; m < DK / 4; ++m) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float mv = mr[m][u];
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const f32x4_t sv = *reinterpret_cast<const f32x4_t*>(&sS[4 * m + u][cl + 4 * q]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[q][j] += mv * sv[j];
                }
            }
        }
        }
        float* dst = sin + (long long)(s + 1) * SS + (long long)row * DK + c0;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            cur[q] = acc[q];
            *reinterpret_cast<f32x4_t*>(dst + 4 * q) = acc[q];
        }
        if (more) {
#pragma unroll
            for (int m = 0; m < DK / 4; ++m) mr[m] = mn[m];
#pragma unroll
            for (int q = 0; q < NQ; ++q) hr[q] = hn[q];
            dead_cur = dead_next;
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
