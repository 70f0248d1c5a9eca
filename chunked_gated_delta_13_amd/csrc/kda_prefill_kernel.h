// Fused chunked KDA prefill kernel for gfx950.
//
// One workgroup of 256 threads (4 wave64s) owns one unit = (sequence b, head h,
// segment s, state-column slice) and walks the unit's chunks of C tokens in
// order, carrying the fp32 state slice S (DK x 64*NCT) in registers.  Sources:
// "Kimi K3" (meridianbulletin.com), "Parallelizing Sequential State Updates"
// (the tokens of a chunk are processed in parallel, then the state is handed to
// the next chunk); "Kimi K3's architecture" (orkas.ai), "A lower bound that
// deleted a GPU code path" (with log alpha >= -5 the accumulated log-decay of a
// 16-token tile stays inside (-80, 0), so its reciprocal fits the 8-bit
// exponent of bf16 and the diagonal tiles use the same dense product as the
// others).
//
// Per chunk, with g_r the inclusive cumulative log2-decay of token r inside the
// chunk (per key channel), row tile a = tokens 16a..16a+15 and its reference
// rho_a = g at the token before the tile:
//   A   scale: Lq = q 2^{g-rho_a}, Lk = k 2^{g-rho_a}    (<= 1)
//              Kd = k 2^{rho_a-g}                        (<= 2^{115.4} = e^80, diagonal tile)
//              K' = k 2^{g_C-g}                          (<= 1, state write)
//   B   A_ri = beta_r <Lk_r, R_i>, Bqk_ri = <Lq_r, R_i>  one dense MFMA tile per (row tile,
//       column tile <= row tile), R_i = Kd_i times 2^{rho_row - rho_col} for earlier tiles;
//       strict / inclusive lower masks by select
//   C   T = (I + A)^{-1}: forward substitution in the 16x16 diagonal blocks, then
//       T_ab = -T_aa sum_c A_ac T_cb band by band
//   D   X = K~ S, P = Q~ S with K~ = Lk 2^{rho_a}, Q~ = Lq 2^{rho_a}
//       U = T (beta (V - X))
//       O = P + Bqk U
//       S <- Diag(2^{g_C}) S + K'^T U
// Every product runs on the matrix cores (bf16 operands / fp32 accumulate, or
// fp32 operands in the fp32 mode); the decay factors are formed in fp32.
// Products of two factors are ordered so that no factor above 1 ever meets an
// underflowed one, so an underflow only drops contributions below FLT_MIN.
#pragma once

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int DK_, int NCT_, int C_, typename TIn_>
struct PrefillCfg {
    static constexpr int DK = DK_;
    static constexpr int NCT = NCT_;             // 16-column tiles per wave
    static constexpr int C = C_;
    using TIn = TIn_;
    using OpT = TIn_;                            // matrix-core operand type
    static constexpr int NT = C / 16;            // 16-token row tiles per chunk
    static constexpr int NTB = (NT + 1) / 2;     // 32-token contraction blocks per chunk
    static constexpr int DVW = 64 * NCT;         // state columns per workgroup
    static constexpr int NPAIR = DK / 2;         // channel pairs (decay phase)
    static constexpr int NSEG = 256 / NPAIR;     // token segments (decay phase)
    static constexpr int TPS = C / NSEG;         // tokens per segment
    static constexpr int SPT = 16 / TPS;         // segments per 16-token tile
    static constexpr int CP = C < 32 ? 32 : C;   // token extent of token-indexed rows
    static constexpr int PADE = sizeof(OpT) == 2 ? 8 : 4;
    static constexpr int PK = DK + PADE;         // pitch of [C][DK] operand arrays
    static constexpr int PT = CP + PADE;         // pitch of sT, sB, sKpT
    static constexpr int PV = DVW + PADE;        // pitch of sV / sO
    static constexpr int PA = C + 1;             // pitch of fp32 sA / sTf
    static constexpr int VEL = 16 / (int)sizeof(TIn);           // elements per 16-byte vector
    static constexpr int VPR = DVW / VEL;                       // vectors per value row
    static constexpr int NV = C * VPR;                          // vectors per value chunk
    static constexpr int NVV = (NV + 255) / 256;                // vectors per thread

    static_assert(TPS >= 1 && 16 % TPS == 0, "segment must sit inside one tile");
    static_assert(DK % 32 == 0 && C % 16 == 0, "shape");

    static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
    static constexpr size_t oLq = 0;
    static constexpr size_t oLk = oLq + al(sizeof(OpT) * C * PK);
    static constexpr size_t oKd = oLk + al(sizeof(OpT) * C * PK);
    static constexpr size_t oKpT = oKd + al(sizeof(OpT) * C * PK);
    static constexpr size_t oV = oKpT + al(sizeof(OpT) * DK * PT);
    static constexpr size_t oT = oV + al(sizeof(TIn) * C * PV);
    static constexpr size_t oB = oT + al(sizeof(OpT) * C * PT);
    static constexpr size_t oA = oB + al(sizeof(OpT) * C * PT);
    static constexpr size_t oTf = oA + al(4 * C * PA);
    static constexpr size_t oM = oTf + al(4 * C * PA);
    static constexpr size_t oE = oM + al(4 * 3 * 16 * 17);
    static constexpr size_t oD = oE + al(4 * (NT + 1) * DK);
    static constexpr size_t oBeta = oD + al(4 * NT * DK);
    static constexpr size_t oTot = oBeta + al(4 * C);
    static constexpr size_t LDS = oTot + al(4 * NSEG * DK);
    static_assert(sizeof(TIn) * PV <= sizeof(OpT) * PK, "output staging aliases sLk");
};

template <class Cfg>
__global__ __launch_bounds__(256, 1) void kda_prefill_kernel(const PrefillArgs a) {
    using TIn = typename Cfg::TIn;
    using OpT = typename Cfg::OpT;
    using P2 = Pair<TIn>;
    constexpr int DK = Cfg::DK, C = Cfg::C, NT = Cfg::NT, NTB = Cfg::NTB, NCT = Cfg::NCT;
    constexpr int DVW = Cfg::DVW, NPAIR = Cfg::NPAIR, NSEG = Cfg::NSEG, TPS = Cfg::TPS;
    constexpr int SPT = Cfg::SPT, CP = Cfg::CP, PK = Cfg::PK, PT = Cfg::PT, PV = Cfg::PV;
    constexpr int PA = Cfg::PA, VEL = Cfg::VEL, VPR = Cfg::VPR, NV = Cfg::NV, NVV = Cfg::NVV;
    constexpr int NIT = DK / 16;   // 16-row tiles of the state
    constexpr int NKB = DK / 32;   // 32-channel contraction blocks

    __shared__ __align__(16) char smem[Cfg::LDS];
    OpT* sLq = reinterpret_cast<OpT*>(smem + Cfg::oLq);
    OpT* sLk = reinterpret_cast<OpT*>(smem + Cfg::oLk);
    OpT* sKd = reinterpret_cast<OpT*>(smem + Cfg::oKd);
    OpT* sKpT = reinterpret_cast<OpT*>(smem + Cfg::oKpT);
    TIn* sV = reinterpret_cast<TIn*>(smem + Cfg::oV);
    OpT* sT = reinterpret_cast<OpT*>(smem + Cfg::oT);
    OpT* sB = reinterpret_cast<OpT*>(smem + Cfg::oB);
    float* sA = reinterpret_cast<float*>(smem + Cfg::oA);
    float* sTf = reinterpret_cast<float*>(smem + Cfg::oTf);
    float* sM = reinterpret_cast<float*>(smem + Cfg::oM);
    float* sE = reinterpret_cast<float*>(smem + Cfg::oE);
    float* sD = reinterpret_cast<float*>(smem + Cfg::oD);
    float* sBeta = reinterpret_cast<float*>(smem + Cfg::oBeta);
    float* sTot = reinterpret_cast<float*>(smem + Cfg::oTot);
    TIn* sO = reinterpret_cast<TIn*>(smem + Cfg::oLk);  // aliases sLk after the X/P products

    // ---- unit of this workgroup; sibling column slices share an XCD (blockIdx % 8) ----
    const int bid = blockIdx.x;
    const int xcd = bid & 7;
    const int rr = bid >> 3;
    const int vs = rr % a.n_vs;
    const int unit = (rr / a.n_vs) * 8 + xcd;
    if (unit >= a.n_units) return;
    const int sl = unit % a.n_seg_launch;
    const int bh = unit / a.n_seg_launch;
    const int h = bh % a.H;
    const int b = bh / a.H;
    const int s = a.seg0 + sl;
    const long long t_begin = (long long)s * a.seg_len;
    const long long t_end = (t_begin + a.seg_len < a.T) ? t_begin + a.seg_len : a.T;
    const int col0 = vs * DVW;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, lr = lane & 15, lg = lane >> 4;

    const long long HD = (long long)a.H * DK;  // token stride of every [B, T, H, d] tensor
    const long long base_tok = (long long)b * a.T * HD + (long long)h * DK;
    const TIn* gq = reinterpret_cast<const TIn*>(a.q) + base_tok;
    const TIn* gk = reinterpret_cast<const TIn*>(a.k) + base_tok;
    const float* gla = a.log_alpha + base_tok;
    const TIn* gv = reinterpret_cast<const TIn*>(a.v) + base_tok + col0;
    TIn* go = a.o ? reinterpret_cast<TIn*>(a.o) + base_tok + col0 : nullptr;
    const float* gbeta = a.beta + (long long)b * a.T * a.H + h;
    const bool has_o = go != nullptr;
    const bool zero_v = a.zero_values != 0;

    // ---- initial state: lane holds S[16*it + 4*lg + j][colw(ct)] ----
    f32x4_t st[NIT][NCT];
    {
        const float* sin = (a.init_mode == 1)
            ? a.s_in + (long long)bh * a.sin_bh_stride + (long long)s * a.sin_seg_stride
            : nullptr;
#pragma unroll
        for (int it = 0; it < NIT; ++it)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const int col = col0 + wave * 16 * NCT + ct * 16 + lr;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = 16 * it + 4 * lg + j;
                    float x = 0.0f;
                    if (a.init_mode == 1) x = sin[(long long)row * DK + col];
                    else if (a.init_mode == 2) x = (row == col) ? 1.0f : 0.0f;
                    st[it][ct][j] = x;
                }
            }
    }

    // ---- zero the token-padded operand arrays once (never-written parts stay zero) ----
    for (int e = tid; e < C * PT; e += 256) {
        sT[e] = from_f32<OpT>(0.0f);
        sB[e] = from_f32<OpT>(0.0f);
    }
    for (int e = tid; e < DK * PT; e += 256) sKpT[e] = from_f32<OpT>(0.0f);

    // ---- decay-phase thread mapping: channel pair cp, token segment sg ----
    const int cp = tid % NPAIR;
    const int sg = tid / NPAIR;
    const int ch0 = 2 * cp;

    // ---- prefetch registers for the next chunk ----
    typename P2::raw pq[TPS], pk[TPS];
    float2 pl[TPS];
    float pbeta = 0.0f;
    uint4 pv[NVV];

    auto load_chunk = [&](long long c0) {
#pragma unroll
        for (int i = 0; i < TPS; ++i) {
            const long long t = c0 + sg * TPS + i;
            if (t < t_end) {
                const long long off = t * HD + ch0;
                pl[i] = *reinterpret_cast<const float2*>(gla + off);
                pq[i] = P2::load(gq + off);
                pk[i] = P2::load(gk + off);
            } else {
                pl[i] = make_float2(0.0f, 0.0f);
                pq[i] = P2::zero();
                pk[i] = P2::zero();
            }
        }
        if (tid < C) {
            const long long t = c0 + tid;
            pbeta = (t < t_end) ? gbeta[t * a.H] : 0.0f;
        }
#pragma unroll
        for (int m = 0; m < NVV; ++m) {
            const int e = tid + 256 * m;
            uint4 x = make_uint4(0u, 0u, 0u, 0u);
            if (e < NV) {
                const int row = e / VPR, cv = e % VPR;
                const long long t = c0 + row;
                if (t < t_end && !zero_v)
                    x = *reinterpret_cast<const uint4*>(gv + t * HD + cv * VEL);
            }
            pv[m] = x;
        }
    };

    const long long ntok = t_end - t_begin;
    const int nchunks = ntok > 0 ? (int)((ntok + C - 1) / C) : 0;
    if (nchunks > 0) load_chunk(t_begin);

    for (int c = 0; c < nchunks; ++c) {
        const long long c0 = t_begin + (long long)c * C;
        __syncthreads();  // every read of the previous chunk's LDS is done

        // ================= A: commit prefetch, per-segment cumulative decay =================
#pragma unroll
        for (int m = 0; m < NVV; ++m) {
            const int e = tid + 256 * m;
            if (e < NV) {
                const int row = e / VPR, cv = e % VPR;
                *reinterpret_cast<uint4*>(sV + row * PV + cv * VEL) = pv[m];
            }
        }
        if (tid < C) sBeta[tid] = pbeta;

        float g0[TPS], g1[TPS], kx0[TPS], kx1[TPS], qx0[TPS], qx1[TPS];
        {
            float run0 = 0.0f, run1 = 0.0f;
#pragma unroll
            for (int i = 0; i < TPS; ++i) {
                const float l0 = fminf(fmaxf(pl[i].x, kLogAlphaMin), 0.0f) * kLog2e;
                const float l1 = fminf(fmaxf(pl[i].y, kLogAlphaMin), 0.0f) * kLog2e;
                run0 += l0;
                run1 += l1;
                g0[i] = run0;
                g1[i] = run1;
                qx0[i] = P2::lo(pq[i]);
                qx1[i] = P2::hi(pq[i]);
                kx0[i] = P2::lo(pk[i]);
                kx1[i] = P2::hi(pk[i]);
            }
            sTot[sg * DK + ch0] = run0;
            sTot[sg * DK + ch0 + 1] = run1;
        }
        __syncthreads();
        if (c + 1 < nchunks) load_chunk(c0 + C);  // overlaps with everything below

        // ================= A': references and decay-scaled operands =================
        {
            // prefix over segments, summed in the same order by every thread
            float P0[NSEG + 1], P1[NSEG + 1];
            P0[0] = 0.0f;
            P1[0] = 0.0f;
#pragma unroll
            for (int q2 = 0; q2 < NSEG; ++q2) {
                P0[q2 + 1] = P0[q2] + sTot[q2 * DK + ch0];
                P1[q2 + 1] = P1[q2] + sTot[q2 * DK + ch0 + 1];
            }
            const int at = (sg * TPS) / 16;       // this segment's row tile
            float off0 = 0.0f, off1 = 0.0f, rho0 = 0.0f, rho1 = 0.0f, nx0 = 0.0f, nx1 = 0.0f;
#pragma unroll
            for (int q2 = 0; q2 <= NSEG; ++q2) {
                if (q2 == sg) { off0 = P0[q2]; off1 = P1[q2]; }
                if (q2 == at * SPT) { rho0 = P0[q2]; rho1 = P1[q2]; }
                if (q2 == (at + 1) * SPT) { nx0 = P0[q2]; nx1 = P1[q2]; }
            }
            const float gC0 = P0[NSEG], gC1 = P1[NSEG];
            const float fd0 = fast_exp2(nx0 - rho0), fd1 = fast_exp2(nx1 - rho1);  // [2^-115.4, 1]
            const float fc0 = fast_exp2(gC0 - nx0), fc1 = fast_exp2(gC1 - nx1);    // (0, 1]
#pragma unroll
            for (int i = 0; i < TPS; ++i) {
                const int r = sg * TPS + i;
                const float gg0 = g0[i] + off0, gg1 = g1[i] + off1;
                const float x0 = fast_exp2(gg0 - rho0), x1 = fast_exp2(gg1 - rho1);  // <= 1
                const float y0 = fast_exp2(rho0 - gg0), y1 = fast_exp2(rho1 - gg1);  // >= 1
                st_pair(sLq + r * PK + ch0, qx0[i] * x0, qx1[i] * x1);
                st_pair(sLk + r * PK + ch0, kx0[i] * x0, kx1[i] * x1);
                st_pair(sKd + r * PK + ch0, kx0[i] * y0, kx1[i] * y1);
                sKpT[ch0 * PT + r] = from_f32<OpT>(kx0[i] * ((y0 * fd0) * fc0));
                sKpT[(ch0 + 1) * PT + r] = from_f32<OpT>(kx1[i] * ((y1 * fd1) * fc1));
            }
            if (sg == 0) {
#pragma unroll
                for (int t2 = 0; t2 <= NT; ++t2) {
                    sE[t2 * DK + ch0] = fast_exp2(P0[t2 * SPT]);
                    sE[t2 * DK + ch0 + 1] = fast_exp2(P1[t2 * SPT]);
                    if (t2 < NT) {
                        sD[t2 * DK + ch0] = fast_exp2(P0[(t2 + 1) * SPT] - P0[t2 * SPT]);
                        sD[t2 * DK + ch0 + 1] = fast_exp2(P1[(t2 + 1) * SPT] - P1[t2 * SPT]);
                    }
                }
            }
        }
        __syncthreads();

        // ================= B: decay-weighted KK^T and QK^T tiles =================
        {
            constexpr int NP = NT * (NT + 1) / 2;
            for (int pi = wave; pi < NP; pi += 4) {
                int ar = 0, rem = pi;
                while (rem > ar) { rem -= ar + 1; ++ar; }
                const int ac = rem;
                f32x4_t accA = zero4(), accB = zero4();
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    Frag<OpT> fk, fq, fr;
                    lds_row_frag(fk, sLk + (16 * ar + lr) * PK + 32 * kb, lg);
                    lds_row_frag(fq, sLq + (16 * ar + lr) * PK + 32 * kb, lg);
                    lds_row_frag(fr, sKd + (16 * ac + lr) * PK + 32 * kb, lg);
                    if (ac < ar) {
                        float val[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j) val[j] = fr.get(j);
                        for (int m = ac; m < ar; ++m) {
                            float d8[8];
                            lds_row_f32x8(d8, sD + m * DK + 32 * kb, lg);
#pragma unroll
                            for (int j = 0; j < 8; ++j) val[j] *= d8[j];
                        }
#pragma unroll
                        for (int j = 0; j < 8; ++j) fr.set(j, val[j]);
                    }
                    accA = mma(fk, fr, accA);
                    accB = mma(fq, fr, accB);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * ar + 4 * lg + j;
                    const int i = 16 * ac + lr;
                    float av = accA[j] * sBeta[r];
                    float bv = accB[j];
                    if (ac == ar) {
                        av = (i < r) ? av : 0.0f;
                        bv = (i <= r) ? bv : 0.0f;
                    }
                    sA[r * PA + i] = av;
                    sB[r * PT + i] = from_f32<OpT>(bv);
                }
            }
        }
        __syncthreads();

        // ================= C: T = (I + A)^{-1} =================
        if (wave == 0) {
            const int ab = lane >> 4, jj = lane & 15;
            if (ab < NT) {
                const float* Ab = sA + (16 * ab) * PA + 16 * ab;
                float col[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float acc = (r == jj) ? 1.0f : 0.0f;
#pragma unroll
                    for (int i = 0; i < r; ++i) acc -= Ab[r * PA + i] * col[i];
                    col[r] = acc;
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) sTf[(16 * ab + r) * PA + 16 * ab + jj] = col[r];
            }
        }
        __syncthreads();
#pragma unroll
        for (int d = 1; d < NT; ++d) {
            const int nb = NT - d;
            for (int e = tid; e < nb * 256; e += 256) {
                const int bi = e >> 8, r = (e >> 4) & 15, jj = e & 15;
                const int ar = d + bi, bc = bi;
                float acc = 0.0f;
                for (int cc = bc; cc < ar; ++cc) {
                    const float* Ar = sA + (16 * ar + r) * PA + 16 * cc;
                    const float* Tc = sTf + (16 * cc) * PA + 16 * bc + jj;
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc += Ar[i] * Tc[i * PA];
                }
                sM[(bi * 16 + r) * 17 + jj] = acc;
            }
            __syncthreads();
            for (int e = tid; e < nb * 256; e += 256) {
                const int bi = e >> 8, r = (e >> 4) & 15, jj = e & 15;
                const int ar = d + bi, bc = bi;
                const float* Tr = sTf + (16 * ar + r) * PA + 16 * ar;
                float acc = 0.0f;
#pragma unroll
                for (int m = 0; m < 16; ++m) acc += Tr[m] * sM[(bi * 16 + m) * 17 + jj];
                sTf[(16 * ar + r) * PA + 16 * bc + jj] = -acc;
            }
            __syncthreads();
        }
        for (int e = tid; e < C * C; e += 256) {
            const int r = e / C, cc = e % C;
            sT[r * PT + cc] = from_f32<OpT>(cc <= r ? sTf[r * PA + cc] : 0.0f);
        }
        __syncthreads();

        // ================= D: state-dependent products =================
        f32x4_t X[NT][NCT], Pq[NT][NCT];
        {
            Frag<OpT> fs[NKB][NCT];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) acc_pair_frag(fs[kb][ct], st[2 * kb][ct], st[2 * kb + 1][ct], true);
#pragma unroll
            for (int ar = 0; ar < NT; ++ar) {
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) { X[ar][ct] = zero4(); Pq[ar][ct] = zero4(); }
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    Frag<OpT> fk, fq;
                    float e8[8];
                    lds_row_frag(fk, sLk + (16 * ar + lr) * PK + 32 * kb, lg);
                    lds_row_frag(fq, sLq + (16 * ar + lr) * PK + 32 * kb, lg);
                    lds_row_f32x8(e8, sE + ar * DK + 32 * kb, lg);
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        fk.set(j, fk.get(j) * e8[j]);
                        fq.set(j, fq.get(j) * e8[j]);
                    }
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        X[ar][ct] = mma(fk, fs[kb][ct], X[ar][ct]);
                        Pq[ar][ct] = mma(fq, fs[kb][ct], Pq[ar][ct]);
                    }
                }
            }
        }
        __syncthreads();  // sLk / sLq reads done: sO may now overwrite sLk

        // RHS = beta (V - X), then U = T RHS
        Frag<OpT> fU[NTB][NCT];
        {
            f32x4_t Rh[NT][NCT];
#pragma unroll
            for (int ar = 0; ar < NT; ++ar)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    const int wc = wave * 16 * NCT + ct * 16 + lr;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int r = 16 * ar + 4 * lg + j;
                        const float vv = zero_v ? 0.0f : to_f32<TIn>(sV[r * PV + wc]);
                        Rh[ar][ct][j] = sBeta[r] * (vv - X[ar][ct][j]);
                    }
                }
            Frag<OpT> fR[NTB][NCT];
#pragma unroll
            for (int kb = 0; kb < NTB; ++kb)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    const bool hi = 2 * kb + 1 < NT;
                    acc_pair_frag(fR[kb][ct], Rh[2 * kb][ct], Rh[hi ? 2 * kb + 1 : 2 * kb][ct], hi);
                }
            f32x4_t U[NT][NCT];
#pragma unroll
            for (int ar = 0; ar < NT; ++ar) {
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) U[ar][ct] = zero4();
#pragma unroll
                for (int kb = 0; kb <= ar / 2; ++kb) {
                    Frag<OpT> ft;
                    lds_row_frag(ft, sT + (16 * ar + lr) * PT + 32 * kb, lg);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) U[ar][ct] = mma(ft, fR[kb][ct], U[ar][ct]);
                }
            }
#pragma unroll
            for (int kb = 0; kb < NTB; ++kb)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    const bool hi = 2 * kb + 1 < NT;
                    acc_pair_frag(fU[kb][ct], U[2 * kb][ct], U[hi ? 2 * kb + 1 : 2 * kb][ct], hi);
                }
        }

        // O = P + Bqk U
        if (has_o) {
#pragma unroll
            for (int ar = 0; ar < NT; ++ar)
#pragma unroll
                for (int kb = 0; kb <= ar / 2; ++kb) {
                    Frag<OpT> fb;
                    lds_row_frag(fb, sB + (16 * ar + lr) * PT + 32 * kb, lg);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) Pq[ar][ct] = mma(fb, fU[kb][ct], Pq[ar][ct]);
                }
        }

        // S <- Diag(2^{g_C}) S + K'^T U
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const f32x4_t gam = *reinterpret_cast<const f32x4_t*>(sE + NT * DK + 16 * it + 4 * lg);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int j = 0; j < 4; ++j) st[it][ct][j] *= gam[j];
#pragma unroll
            for (int kb = 0; kb < NTB; ++kb) {
                Frag<OpT> fkp;
                lds_row_frag(fkp, sKpT + (16 * it + lr) * PT + 32 * kb, lg);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) st[it][ct] = mma(fkp, fU[kb][ct], st[it][ct]);
            }
        }

        // stage O through LDS and write whole rows
        if (has_o) {
#pragma unroll
            for (int ar = 0; ar < NT; ++ar)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    const int wc = wave * 16 * NCT + ct * 16 + lr;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        sO[(16 * ar + 4 * lg + j) * PV + wc] = from_f32<TIn>(Pq[ar][ct][j]);
                }
            __syncthreads();
#pragma unroll
            for (int m = 0; m < NVV; ++m) {
                const int e = tid + 256 * m;
                if (e < NV) {
                    const int row = e / VPR, cv = e % VPR;
                    const long long t = c0 + row;
                    if (t < t_end)
                        *reinterpret_cast<uint4*>(go + t * HD + cv * VEL) =
                            *reinterpret_cast<const uint4*>(sO + row * PV + cv * VEL);
                }
            }
        }
    }

    // ---- final state ----
    if (a.s_out && (a.out_seg < 0 || a.out_seg == s)) {
        float* so = a.s_out + (long long)bh * a.sout_bh_stride + (long long)s * a.sout_seg_stride;
#pragma unroll
        for (int it = 0; it < NIT; ++it)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const int col = col0 + wave * 16 * NCT + ct * 16 + lr;
#pragma unroll
                for (int j = 0; j < 4; ++j) so[(long long)(16 * it + 4 * lg + j) * DK + col] = st[it][ct][j];
            }
    }
}

template <class Cfg>
hipError_t launch_prefill_cfg(const PrefillArgs& a, hipStream_t stream) {
    const long long groups = ((long long)a.n_units + 7) / 8;
    const long long nblk = groups * 8 * a.n_vs;
    if (nblk <= 0) return hipSuccess;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kda_prefill_kernel<Cfg>, dim3((unsigned)nblk), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kda
