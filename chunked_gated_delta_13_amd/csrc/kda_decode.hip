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
// A workgroup owns one whole (sequence, head) state: DV/4 column groups of 4 (float4, so
// each state row is read as one contiguous run) x 16 row groups.  Column sums are reduced
// across the row groups of a wave with lane shuffles, then across the waves in LDS (one
// barrier per token).  The
// state a workgroup takes is chosen so that each of the 8 XCDs (which receive workgroups
// round-robin) streams one contiguous range of states: a whole-state, XCD-contiguous
// pattern moves measurably more bytes per second through HBM than half-state workgroups.
// For an m-token block the state is read once, the m tokens run in order on
// chip, and the state is written back only when the block is committed
// ("Kimi K3's architecture", "The bill comes due in the serving stack": the
// drafted tokens' inputs are kept and the state rebuilt from them).  A verify
// block of at most 4 tokens (outputs only) takes all its state reductions in
// one pass instead (kda_verify_block_kernel).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// MM = most tokens per block this instantiation stages (1 for the decode step).  TWO = reduce
// across the waves through workgroup totals with two barriers per token (blocks that write
// outputs: the read-out sums then cost one LDS read per column) instead of one.
template <int DK, typename TIn, int MM, bool TWO>
__global__ __launch_bounds__(4 * DK) void kda_decode_kernel(const DecodeArgs a, int per_xcd) {
    constexpr int DV = DK;
    constexpr int NCG = DV / 4;      // float4 column groups per state row
    constexpr int NRG = 16;          // row groups
    constexpr int NTH = NCG * NRG;   // threads per workgroup (4 * DK)
    constexpr int NW = NTH / 64;     // waves per workgroup
    constexpr int RPT = DK / NRG;    // state rows per thread
    static_assert(NCG <= 64 && 64 % NCG == 0, "a wave holds whole row groups");
    const long long nh = (long long)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
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
    const int cg = tid % NCG, rg = tid / NCG;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = cg * 4;

    auto tok_of = [&](int t) { return (n * a.m + t) * a.H + h; };   // token row of [N, m, H, *]
    auto alpha_of = [](float la) { return __expf(fminf(fmaxf(la, kLogAlphaMin), 0.0f)); };
    // Blocks of at most NTH / DK tokens hold one element of each input per thread: those are
    // requested ahead of the state, so that staging them overlaps the state's arrival.  Threads
    // past the block's last element read element 0 and discard it.
    constexpr bool EARLY = MM > 1 && MM * DK <= NTH;
    const bool has_in = EARLY && tid < mt * DK;
    const int te = has_in ? tid / DK : 0, ie = has_in ? tid % DK : 0;
    TIn kin{}, qin{}, vin{};
    float lin = 0.0f, bin = 0.0f;
    if constexpr (EARLY) {
        const long long ibase = tok_of(te) * DK + ie;   // DV == DK
        kin = reinterpret_cast<const TIn*>(a.k)[ibase];
        qin = reinterpret_cast<const TIn*>(a.q)[ibase];
        vin = reinterpret_cast<const TIn*>(a.v)[ibase];
        lin = a.log_alpha[ibase];
        bin = a.beta[tok_of(tid < mt ? tid : 0)];
        __builtin_amdgcn_sched_barrier(0);   // keep these requests ahead of the state's
    }

    float* Sb = a.S + nh * (long long)(DK * DV) + col;
    f32x4_t s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        s[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(Sb + (long long)(rg + NRG * m) * DV));

    // A block's token inputs are staged in LDS once, while the state loads are in flight; a
    // single token (the decode step) is read straight from memory.
    constexpr int MS = MM > 1 ? MM : 1;
    __shared__ float skk[MS][DK], sqq[MS][DK], sal[MS][DK], sv[MS][DV], sbt[MS];
    if constexpr (EARLY) {
        if (has_in) {
            skk[te][ie] = to_f32<TIn>(kin);
            sqq[te][ie] = to_f32<TIn>(qin);
            sal[te][ie] = alpha_of(lin);
            sv[te][ie] = to_f32<TIn>(vin);
        }
        if (tid < mt) sbt[tid] = bin;
    } else if constexpr (MM > 1) {
        for (int e = tid; e < mt * DK; e += NTH) {
            const int t = e / DK, i = e % DK;
            const long long base = tok_of(t) * DK + i;
            skk[t][i] = to_f32<TIn>(reinterpret_cast<const TIn*>(a.k)[base]);
            sqq[t][i] = to_f32<TIn>(reinterpret_cast<const TIn*>(a.q)[base]);
            sal[t][i] = alpha_of(a.log_alpha[base]);
        }
        for (int e = tid; e < mt * DV; e += NTH) {
            const int t = e / DV, c = e % DV;
            sv[t][c] = to_f32<TIn>(reinterpret_cast<const TIn*>(a.v)[tok_of(t) * DV + c]);
        }
        if (tid < mt) sbt[tid] = a.beta[tok_of(tid)];
    }

    // per-wave column sums (p, then r, then k.q), one buffer per token parity; workgroup totals
    __shared__ __attribute__((aligned(16))) float spart[2][NW][2 * DV + 4];
    __shared__ float stot[TWO ? 2 * DV + 1 : 1];
    if constexpr (MM > 1) __syncthreads();

    for (int t = 0; t < mt; ++t) {
        float kk[RPT], qq[RPT], al[RPT];
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg + NRG * m;
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
        // reduce over the row groups of this wave (lanes NCG apart) ...
#pragma unroll
        for (int off = NCG; off < 64; off <<= 1) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                p[j] += __shfl_xor(p[j], off);
                r[j] += __shfl_xor(r[j], off);
            }
            kq += __shfl_xor(kq, off);
        }
        // ... then over the waves, in wave order.  With one barrier, every thread sums its own
        // columns; the partials are double-buffered by token parity, so a wave writes token
        // t+1's partials only after the barrier of token t, which every wave reaches after
        // reading token t-1's.  With two, thread i <= 2 DV sums value i into the totals.
        const int pb = TWO ? 0 : t & 1;
        if (lane < NCG) {
            *reinterpret_cast<f32x4_t*>(&spart[pb][wave][col]) = p;
            *reinterpret_cast<f32x4_t*>(&spart[pb][wave][DV + col]) = r;
        }
        if (lane == 0) spart[pb][wave][2 * DV] = kq;
        __syncthreads();
        const bool writes_o = a.o && rg == 0;
        if constexpr (TWO) {
            if (tid <= 2 * DV) {
                float acc = spart[0][0][tid];
#pragma unroll
                for (int w = 1; w < NW; ++w) acc += spart[0][w][tid];
                stot[tid] = acc;
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < 4; ++j) p[j] = stot[col + j];
            if (writes_o) {
#pragma unroll
                for (int j = 0; j < 4; ++j) r[j] = stot[DV + col + j];
                kq = stot[2 * DV];
            }
        } else {
            p = *reinterpret_cast<const f32x4_t*>(&spart[pb][0][col]);
#pragma unroll
            for (int w = 1; w < NW; ++w) {
                const f32x4_t x = *reinterpret_cast<const f32x4_t*>(&spart[pb][w][col]);
#pragma unroll
                for (int j = 0; j < 4; ++j) p[j] += x[j];
            }
            if (writes_o) {
                r = *reinterpret_cast<const f32x4_t*>(&spart[pb][0][DV + col]);
                kq = spart[pb][0][2 * DV];
#pragma unroll
                for (int w = 1; w < NW; ++w) {
                    const f32x4_t x = *reinterpret_cast<const f32x4_t*>(&spart[pb][w][DV + col]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) r[j] += x[j];
                    kq += spart[pb][w][2 * DV];
                }
            }
        }

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
        if (writes_o) {
            TIn* on = reinterpret_cast<TIn*>(a.o) + tok_of(t) * DV + col;
            const float bkq = bt * kq;
#pragma unroll
            for (int j = 0; j < 4; ++j) on[j] = from_f32<TIn>(r[j] + bkq * e[j]);
        }
    }
    if (a.write_state) {
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            __builtin_nontemporal_store(s[m], reinterpret_cast<f32x4_t*>(Sb + (long long)(rg + NRG * m) * DV));
    }
}

// Speculative verify of a block of m <= MB tokens in one pass over the state (outputs only, the
// state is not written).  With a_t = alpha_0 * ... * alpha_t (per key channel, t = 0 .. m-1) the
// recurrence unrolls over the block to
//   S_t = Diag(a_t) S + sum_{j <= t} beta_j Diag(a_t / a_j) k_j e_j^T,
//   e_t = v_t - S^T (a_t . k_t) - sum_{j < t} G_tj e_j,     G_tj = beta_j sum_i (a_t/a_j)_i k_j,i k_t,i
//   o_t = S^T (a_t . q_t) + sum_{j <= t} H_tj e_j,           H_tj = beta_j sum_i (a_t/a_j)_i k_j,i q_t,i
// so the state is read once for 2m column sums, the m x m products G and H (independent of the
// state) are formed while its loads are in flight, and e_t, o_t follow by forward substitution
// per column.  a_t / a_j is formed as the product alpha_{j+1} ... alpha_t (no division); every
// factor lies in [e^{-5 m}, 1].
template <int DK, typename TIn, int MB>
__global__ __launch_bounds__(4 * DK) __attribute__((amdgpu_waves_per_eu(8))) void kda_verify_block_kernel(const DecodeArgs a, int per_xcd) {
    constexpr int DV = DK;
    constexpr int NCG = DV / 4, NRG = 16, NTH = NCG * NRG, NW = NTH / 64, RPT = DK / NRG;
    constexpr int NP = MB * (MB + 1) / 2;   // (t, j) pairs with j <= t
    constexpr int CPL = DK / 64;            // key channels per lane in the pair products
    static_assert(NCG <= 64 && 64 % NCG == 0 && DK % 64 == 0, "a wave holds whole row groups");
    const long long nh = (long long)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (nh >= a.NH) return;
    const long long n = nh / a.H;
    const int h = (int)(nh % a.H);
    const int mt = a.m < MB ? a.m : MB;
    const int tid = threadIdx.x;
    const int cg = tid % NCG, rg = tid / NCG;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = cg * 4;

    // The block's token inputs (one element of each per thread) are requested before the state,
    // so that staging them and the pair products, which need nothing else, run while the state
    // is still arriving.  Threads past the block's last element read element 0 and discard it.
    static_assert(MB * DK <= NTH, "one input element per thread");
    auto tok_of = [&](int t) { return (n * a.m + t) * a.H + h; };   // token row of [N, m, H, *]
    const bool has_in = tid < mt * DK;
    const int te = has_in ? tid / DK : 0, ie = has_in ? tid % DK : 0;
    const long long ibase = tok_of(te) * DK + ie;                   // DV == DK
    const TIn kin = reinterpret_cast<const TIn*>(a.k)[ibase];
    const TIn qin = reinterpret_cast<const TIn*>(a.q)[ibase];
    const TIn vin = reinterpret_cast<const TIn*>(a.v)[ibase];
    const float lin = a.log_alpha[ibase];
    const float bin = a.beta[tok_of(tid < mt ? tid : 0)];
    __builtin_amdgcn_sched_barrier(0);   // keep these requests ahead of the state's

    const float* Sb = a.S + nh * (long long)(DK * DV) + col;
    f32x4_t s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        s[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(Sb + (long long)(rg + NRG * m) * DV));

    __shared__ float skk[MB][DK], sqq[MB][DK], sal[MB][DK], sv[MB][DV], sbt[MB];
    __shared__ float skt[MB][DK], sqt[MB][DK];   // a_t . k_t, a_t . q_t
    __shared__ float sG[MB][MB], sH[MB][MB];
    constexpr int HB = MB < 2 ? MB : 2;   // tokens per group of column sums
    __shared__ __attribute__((aligned(16))) float spart[NW][2 * HB][DV];
    __shared__ __attribute__((aligned(16))) float stot[2 * MB][DV];
    if (has_in) {
        skk[te][ie] = to_f32<TIn>(kin);
        sqq[te][ie] = to_f32<TIn>(qin);
        sal[te][ie] = __expf(fminf(fmaxf(lin, kLogAlphaMin), 0.0f));
        sv[te][ie] = to_f32<TIn>(vin);
    }
    if (tid < mt) sbt[tid] = bin;
    barrier_lds();   // the state loads stay in flight

    // decay-weighted keys and queries, and the pair products (wave w takes pairs w, w + NW, ...)
    if (tid < DK) {
        float at = 1.0f;
        for (int t = 0; t < mt; ++t) {
            at *= sal[t][tid];
            skt[t][tid] = at * skk[t][tid];
            sqt[t][tid] = at * sqq[t][tid];
        }
    }
    for (int pp = wave; pp < NP; pp += NW) {
        int t = 0;
        while ((t + 1) * (t + 2) / 2 <= pp) ++t;
        const int j = pp - t * (t + 1) / 2;   // j <= t
        if (t >= mt) continue;                 // wave-uniform
        float gs = 0.0f, hs = 0.0f;
#pragma unroll
        for (int u = 0; u < CPL; ++u) {
            const int i = lane + 64 * u;
            float c = sbt[j] * skk[j][i];
            for (int l = j + 1; l <= t; ++l) c *= sal[l][i];
            gs += c * skk[t][i];
            hs += c * sqq[t][i];
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            gs += __shfl_xor(gs, off);
            hs += __shfl_xor(hs, off);
        }
        if (lane == 0) {
            sH[t][j] = hs;
            if (j < t) sG[t][j] = gs;
        }
    }

    // column sums of the state against the decay-weighted keys and queries, HB tokens at a time
    // (the per-wave partials of a group are summed into the totals before the next group's are
    // written, which keeps the partials buffer, and so the workgroup's LDS, small)
    barrier_lds();   // skt, sqt (and sG, sH) complete; the state loads may still be in flight
#pragma unroll
    for (int t0 = 0; t0 < MB; t0 += HB) {
        if (t0 >= mt) break;   // uniform
#pragma unroll
        for (int u = 0; u < HB; ++u) {
            const int t = t0 + u;
            if (t < mt) {
                f32x4_t pk = zero4(), pq = zero4();
#pragma unroll
                for (int m = 0; m < RPT; ++m) {
                    const float kv = skt[t][rg + NRG * m], qv = sqt[t][rg + NRG * m];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        pk[jj] += s[m][jj] * kv;
                        pq[jj] += s[m][jj] * qv;
                    }
                }
#pragma unroll
                for (int off = NCG; off < 64; off <<= 1) {
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        pk[jj] += __shfl_xor(pk[jj], off);
                        pq[jj] += __shfl_xor(pq[jj], off);
                    }
                }
                if (lane < NCG) {
                    *reinterpret_cast<f32x4_t*>(&spart[wave][2 * u][col]) = pk;
                    *reinterpret_cast<f32x4_t*>(&spart[wave][2 * u + 1][col]) = pq;
                }
            }
        }
        barrier_lds();
        const int nt = mt - t0 < HB ? mt - t0 : HB;
        for (int e = tid; e < 2 * nt * DV; e += NTH) {
            const int r = e / DV, c = e % DV;
            float acc = spart[0][r][c];
#pragma unroll
            for (int w = 1; w < NW; ++w) acc += spart[w][r][c];
            stot[2 * t0 + r][c] = acc;
        }
        barrier_lds();
    }

    // forward substitution per column: e_t, then o_t
    if (rg == 0) {
        f32x4_t ev[MB];
#pragma unroll
        for (int t = 0; t < MB; ++t) {
            if (t < mt) {
                const f32x4_t pt = *reinterpret_cast<const f32x4_t*>(&stot[2 * t][col]);
                const f32x4_t qt = *reinterpret_cast<const f32x4_t*>(&stot[2 * t + 1][col]);
                f32x4_t e4, o4;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) e4[jj] = sv[t][col + jj] - pt[jj];
#pragma unroll
                for (int j = 0; j < t; ++j) {
                    const float g = sG[t][j];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) e4[jj] -= g * ev[j][jj];
                }
                ev[t] = e4;
                o4 = qt;
#pragma unroll
                for (int j = 0; j <= t; ++j) {
                    const float hh = sH[t][j];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) o4[jj] += hh * ev[j][jj];
                }
                TIn* on = reinterpret_cast<TIn*>(a.o) + tok_of(t) * DV + col;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) on[jj] = from_f32<TIn>(o4[jj]);
            }
        }
    }
}

template <int MB>
static hipError_t launch_verify_block(int dk, bool f32, const DecodeArgs& a, dim3 grid, int per_xcd,
                                      hipStream_t stream) {
    const dim3 block(4 * dk);
    if (dk == 128 && !f32) hipLaunchKernelGGL((kda_verify_block_kernel<128, __bf16, MB>), grid, block, 0, stream, a, per_xcd);
    else if (dk == 128 && f32) hipLaunchKernelGGL((kda_verify_block_kernel<128, float, MB>), grid, block, 0, stream, a, per_xcd);
    else if (dk == 64 && !f32) hipLaunchKernelGGL((kda_verify_block_kernel<64, __bf16, MB>), grid, block, 0, stream, a, per_xcd);
    else if (dk == 64 && f32) hipLaunchKernelGGL((kda_verify_block_kernel<64, float, MB>), grid, block, 0, stream, a, per_xcd);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

template <int MM, bool TWO>
static hipError_t launch_decode_mm(int dk, bool f32, const DecodeArgs& a, dim3 grid, int per_xcd,
                                   hipStream_t stream) {
    const dim3 block(4 * dk);
    if (dk == 128 && !f32) hipLaunchKernelGGL((kda_decode_kernel<128, __bf16, MM, TWO>), grid, block, 0, stream, a, per_xcd);
    else if (dk == 128 && f32) hipLaunchKernelGGL((kda_decode_kernel<128, float, MM, TWO>), grid, block, 0, stream, a, per_xcd);
    else if (dk == 64 && !f32) hipLaunchKernelGGL((kda_decode_kernel<64, __bf16, MM, TWO>), grid, block, 0, stream, a, per_xcd);
    else if (dk == 64 && f32) hipLaunchKernelGGL((kda_decode_kernel<64, float, MM, TWO>), grid, block, 0, stream, a, per_xcd);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_decode(int dk, bool f32, const DecodeArgs& a, hipStream_t stream) {
    if (a.NH <= 0) return hipSuccess;
    if (a.m < 1 || a.m > kDecodeMaxTokens) return hipErrorInvalidValue;
    // one workgroup per state; workgroup b takes state (b % 8) * per_xcd + b / 8
    const long long per_xcd = (a.NH + 7) / 8;
    if (per_xcd > 0x7fffffffLL / 8) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(8 * per_xcd));
    // verify blocks (outputs, m > 1) reduce with two barriers per token, everything else with one
    if (a.m == 1) return launch_decode_mm<1, false>(dk, f32, a, grid, (int)per_xcd, stream);
    if (a.m <= 4) {
        // a verify block (outputs, state untouched, every sequence runs all m tokens) in one pass
        if (a.o && !a.write_state && !a.lens) return launch_verify_block<4>(dk, f32, a, grid, (int)per_xcd, stream);
        return a.o ? launch_decode_mm<4, true>(dk, f32, a, grid, (int)per_xcd, stream)
                   : launch_decode_mm<4, false>(dk, f32, a, grid, (int)per_xcd, stream);
    }
    return a.o ? launch_decode_mm<kDecodeMaxTokens, true>(dk, f32, a, grid, (int)per_xcd, stream)
               : launch_decode_mm<kDecodeMaxTokens, false>(dk, f32, a, grid, (int)per_xcd, stream);
}

}  // namespace kda
