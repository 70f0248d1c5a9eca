// KDA decode step for gfx950: one token per (sequence, head), state updated in place.
//
// Sources: "Inside Kimi K3" (academa.ai lecture), sequence paragraph (each new
// token costs the same: one fixed-size state update); "Kimi K3's
// architecture" (orkas.ai), "The bill comes due in the serving stack" (the
// state updates in place).
//
// The step is HBM-bound (about 7 flops per 8 bytes of state moved), so it is
// written as one streaming pass over the state with no matrix cores:
//   S' = Diag(alpha) S                       alpha = exp(clamp(log_alpha, -5, 0))
//   p  = S'^T k,  r = S'^T q                 both column reductions in the same pass
//   e  = v - p
//   S  = S' + beta k e^T                     written back from registers
//   o  = S^T q = r + beta (k . q) e          no second pass over S
// A workgroup owns (sequence, head, 64 state columns): 16 column groups of 4
// (float4, 256 contiguous bytes per row) x 16 row groups.  Column sums are
// reduced across row groups with lane shuffles, then across the 4 waves in LDS.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int DK, typename TIn>
__global__ __launch_bounds__(256) void kda_decode_kernel(const DecodeArgs a) {
    constexpr int DV = DK;
    constexpr int NVB = DV / 64;     // 64-column blocks per state
    constexpr int RPT = DK / 16;     // state rows per thread
    const long long nh = blockIdx.x / NVB;
    const int vb = blockIdx.x % NVB;
    if (nh >= a.NH) return;
    const int tid = threadIdx.x;
    const int cg = tid & 15, rg = tid >> 4;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = vb * 64 + cg * 4;

    float* Sb = a.S + nh * (long long)(DK * DV) + col;
    const TIn* qn = reinterpret_cast<const TIn*>(a.q) + nh * DK;
    const TIn* kn = reinterpret_cast<const TIn*>(a.k) + nh * DK;
    const float* lan = a.log_alpha + nh * DK;

    f32x4_t s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        s[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(Sb + (long long)(rg + 16 * m) * DV));

    float kk[RPT], qq[RPT], al[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + 16 * m;
        kk[m] = to_f32<TIn>(kn[i]);
        qq[m] = to_f32<TIn>(qn[i]);
        al[m] = __expf(fminf(fmaxf(lan[i], kLogAlphaMin), 0.0f));
    }

    f32x4_t p = zero4(), r = zero4();
    float kq = 0.0f;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            s[m][j] *= al[m];
            p[j] += s[m][j] * kk[m];
            r[j] += s[m][j] * qq[m];
        }
        kq += kk[m] * qq[m];
    }
    // reduce over the 4 row groups of this wave (lanes 16 apart) ...
#pragma unroll
    for (int off = 16; off < 64; off <<= 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            p[j] += __shfl_xor(p[j], off);
            r[j] += __shfl_xor(r[j], off);
        }
        kq += __shfl_xor(kq, off);
    }
    // ... then over the 4 waves
    __shared__ f32x4_t sp[4][16], sr[4][16];
    __shared__ float skq[4];
    if (lane < 16) {
        sp[wave][cg] = p;
        sr[wave][cg] = r;
    }
    if (lane == 0) skq[wave] = kq;
    __syncthreads();
    p = sp[0][cg] + sp[1][cg] + sp[2][cg] + sp[3][cg];
    r = sr[0][cg] + sr[1][cg] + sr[2][cg] + sr[3][cg];
    kq = skq[0] + skq[1] + skq[2] + skq[3];

    const float bt = a.beta[nh];
    const TIn* vn = reinterpret_cast<const TIn*>(a.v) + nh * DV + col;
    f32x4_t e;
#pragma unroll
    for (int j = 0; j < 4; ++j) e[j] = to_f32<TIn>(vn[j]) - p[j];

#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const float bk = bt * kk[m];
#pragma unroll
        for (int j = 0; j < 4; ++j) s[m][j] += bk * e[j];
        __builtin_nontemporal_store(s[m], reinterpret_cast<f32x4_t*>(Sb + (long long)(rg + 16 * m) * DV));
    }
    if (rg == 0) {
        TIn* on = reinterpret_cast<TIn*>(a.o) + nh * DV + col;
        const float bkq = bt * kq;
#pragma unroll
        for (int j = 0; j < 4; ++j) on[j] = from_f32<TIn>(r[j] + bkq * e[j]);
    }
}

hipError_t launch_decode(int dk, bool f32, const DecodeArgs& a, hipStream_t stream) {
    if (a.NH <= 0) return hipSuccess;
    const long long nblk = a.NH * (dk / 64);
    if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)nblk), block(256);
    if (dk == 128 && !f32) hipLaunchKernelGGL((kda_decode_kernel<128, __bf16>), grid, block, 0, stream, a);
    else if (dk == 128 && f32) hipLaunchKernelGGL((kda_decode_kernel<128, float>), grid, block, 0, stream, a);
    else if (dk == 64 && !f32) hipLaunchKernelGGL((kda_decode_kernel<64, __bf16>), grid, block, 0, stream, a);
    else if (dk == 64 && f32) hipLaunchKernelGGL((kda_decode_kernel<64, float>), grid, block, 0, stream, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace kda
