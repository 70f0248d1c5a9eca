// KDA decode for gfx950: one token (decode step) or a short block of m tokens (speculative
// verify / commit) per (sequence, head), run from the state held in registers.
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
// For an m-token block the state is read once, the m tokens run in order on
// chip, and the state is written back only when the block is committed
// ("Kimi K3's architecture", "The bill comes due in the serving stack": the
// drafted tokens' inputs are kept and the state rebuilt from them).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// MM = most tokens per block this instantiation stages (1 for the decode step).
template <int DK, typename TIn, int MM>
__global__ __launch_bounds__(256) void kda_decode_kernel(const DecodeArgs a) {
    constexpr int DV = DK;
    constexpr int NVB = DV / 64;     // 64-column blocks per state
    constexpr int RPT = DK / 16;     // state rows per thread
    const long long nh = blockIdx.x / NVB;
    const int vb = blockIdx.x % NVB;
    if (nh >= a.NH) return;
    const long long n = nh / a.H;
    const int h = (int)(nh % a.H);
    int mt = a.m < MM ? a.m : MM;    // tokens this sequence runs (uniform over the workgroup)
    if (a.lens) {
        const int l = a.lens[n];
        mt = l < 0 ? 0 : (l > mt ? mt : l);
    }
    if (mt == 0) return;             // nothing to run: the state stays as it is
    const int tid = threadIdx.x;
    const int cg = tid & 15, rg = tid >> 4;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = vb * 64 + cg * 4;

    float* Sb = a.S + nh * (long long)(DK * DV) + col;
    f32x4_t s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        s[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(Sb + (long long)(rg + 16 * m) * DV));

    // A block's token inputs are staged in LDS once, while the state loads are in flight; a
    // single token (the decode step) is read straight from memory.
    constexpr int MS = MM > 1 ? MM : 1;
    __shared__ float skk[MS][DK], sqq[MS][DK], sal[MS][DK], sv[MS][64], sbt[MS];
    auto tok_of = [&](int t) { return (n * a.m + t) * a.H + h; };   // token row of [N, m, H, *]
    auto alpha_of = [](float la) { return __expf(fminf(fmaxf(la, kLogAlphaMin), 0.0f)); };
    if constexpr (MM > 1) {
        for (int e = tid; e < mt * DK; e += 256) {
            const int t = e / DK, i = e % DK;
            const long long base = tok_of(t) * DK + i;
            skk[t][i] = to_f32<TIn>(reinterpret_cast<const TIn*>(a.k)[base]);
            sqq[t][i] = to_f32<TIn>(reinterpret_cast<const TIn*>(a.q)[base]);
            sal[t][i] = alpha_of(a.log_alpha[base]);
        }
        for (int e = tid; e < mt * 64; e += 256) {
            const int t = e / 64, c = e % 64;
            sv[t][c] = to_f32<TIn>(reinterpret_cast<const TIn*>(a.v)[tok_of(t) * DV + vb * 64 + c]);
        }
        if (tid < mt) sbt[tid] = a.beta[tok_of(tid)];
    }

    // column sums of the 4 waves, double-buffered over tokens so one barrier per token suffices
    __shared__ f32x4_t sp[2][4][16], sr[2][4][16];
    __shared__ float skq[2][4];
    if constexpr (MM > 1) __syncthreads();

    for (int t = 0; t < mt; ++t) {
        float kk[RPT], qq[RPT], al[RPT];
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg + 16 * m;
            if constexpr (MM > 1) {
                kk[m] = skk[t][i];
                qq[m] = sqq[t][i];
                al[m] = sal[t][i];
            } else {
                const long long base = tok_of(t) * DK + i;
                kk[m] = to_f32<TIn>(reinterpret_cast<const TIn*>(a.k)[base]);
                qq[m] = to_f32<TIn>(reinterpret_cast<const TIn*>(a.q)[base]);
                al[m] = alpha_of(a.log_alpha[base]);
            }
        }
        f32x4_t p = zero4(), r = zero4();
        float kq = 0.0f;
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const float al_m = al[m];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                s[m][j] *= al_m;
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
        const int bsel = t & 1;
        if (lane < 16) {
            sp[bsel][wave][cg] = p;
            sr[bsel][wave][cg] = r;
        }
        if (lane == 0) skq[bsel][wave] = kq;
        __syncthreads();
        p = sp[bsel][0][cg] + sp[bsel][1][cg] + sp[bsel][2][cg] + sp[bsel][3][cg];
        r = sr[bsel][0][cg] + sr[bsel][1][cg] + sr[bsel][2][cg] + sr[bsel][3][cg];
        kq = skq[bsel][0] + skq[bsel][1] + skq[bsel][2] + skq[bsel][3];

        float bt;
        f32x4_t e;
        if constexpr (MM > 1) {
            bt = sbt[t];
#pragma unroll
            for (int j = 0; j < 4; ++j) e[j] = sv[t][cg * 4 + j] - p[j];
        } else {
            bt = a.beta[tok_of(t)];
            const TIn* vn = reinterpret_cast<const TIn*>(a.v) + tok_of(t) * DV + col;
#pragma unroll
            for (int j = 0; j < 4; ++j) e[j] = to_f32<TIn>(vn[j]) - p[j];
        }
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const float bk = bt * kk[m];
#pragma unroll
            for (int j = 0; j < 4; ++j) s[m][j] += bk * e[j];
        }
        if (a.o && rg == 0) {
            TIn* on = reinterpret_cast<TIn*>(a.o) + tok_of(t) * DV + col;
            const float bkq = bt * kq;
#pragma unroll
            for (int j = 0; j < 4; ++j) on[j] = from_f32<TIn>(r[j] + bkq * e[j]);
        }
    }
    if (a.write_state) {
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            __builtin_nontemporal_store(s[m], reinterpret_cast<f32x4_t*>(Sb + (long long)(rg + 16 * m) * DV));
    }
}

template <int MM>
static hipError_t launch_decode_mm(int dk, bool f32, const DecodeArgs& a, dim3 grid, hipStream_t stream) {
    const dim3 block(256);
    if (dk == 128 && !f32) hipLaunchKernelGGL((kda_decode_kernel<128, __bf16, MM>), grid, block, 0, stream, a);
    else if (dk == 128 && f32) hipLaunchKernelGGL((kda_decode_kernel<128, float, MM>), grid, block, 0, stream, a);
    else if (dk == 64 && !f32) hipLaunchKernelGGL((kda_decode_kernel<64, __bf16, MM>), grid, block, 0, stream, a);
    else if (dk == 64 && f32) hipLaunchKernelGGL((kda_decode_kernel<64, float, MM>), grid, block, 0, stream, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_decode(int dk, bool f32, const DecodeArgs& a, hipStream_t stream) {
    if (a.NH <= 0) return hipSuccess;
    if (a.m < 1 || a.m > kDecodeMaxTokens) return hipErrorInvalidValue;
    const long long nblk = a.NH * (dk / 64);
    if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)nblk);
    if (a.m == 1) return launch_decode_mm<1>(dk, f32, a, grid, stream);
    if (a.m <= 4) return launch_decode_mm<4>(dk, f32, a, grid, stream);
    return launch_decode_mm<kDecodeMaxTokens>(dk, f32, a, grid, stream);
}

}  // namespace kda
