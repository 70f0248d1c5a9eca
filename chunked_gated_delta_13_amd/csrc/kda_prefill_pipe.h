// Two-role chunked KDA prefill for gfx950: one chunk of look-ahead.
//
// The kernel in kda_prefill_kernel.h runs every phase of a chunk on all of its waves, one after
// the other, with a workgroup barrier between phases; the state-independent work of a chunk
// (decay, decay-scaled operands, tile pairs, diagonal inverses: VALU-heavy) and the
// state-dependent work (state products: matrix cores and LDS) never overlap.  Here the waves of
// a workgroup take two roles and two chunks are in flight:
//   NCW "chunk waves" (4 or 8) prepare chunk c+1: decay sums (A and a prefix pass), decay-scaled
//   operands (A'), tile pairs (B) and the diagonal inverses;
//   4 "state waves" hold the fp32 state, 32 columns each, and run chunk c:
//   X = K~S and RHS (from the state after chunk c-1), U, O, state update.
// Every SIMD hosts waves of both roles, so VALU work of one role issues while the other waits on
// the matrix cores or LDS.  Per loop iteration there are four barrier intervals, the same for
// both roles:
//   1: prefix(c+1)             | U(c)
//   2: A'(c+1)                 | O(c)            chunk waves hand over V, beta of c+1
//   3: B(c+1)                  | state update(c) chunk waves hand over K~, Q~ of c+1
//   4: inverses(c+1), A(c+2)   | X, RHS(c+1)     chunk waves hand over K'^T, 2^{g_C} of c+1
// An operand array of chunk c is overwritten for c+1 only in an interval after the last state
// wave read it, so it needs one copy.  The arithmetic of every phase is that of
// kda_prefill_kernel.h (same decay summation order, same products); sources as cited there:
// "Kimi K3" (meridianbulletin.com), "Parallelizing Sequential State Updates"; "Kimi K3's
// architecture" (orkas.ai), "A lower bound that deleted a GPU code path".
#pragma once

#include "kda_prefill_kernel.h"

namespace kda {

// Byte sizes rounded up to 16 (LDS arrays start on 16-byte boundaries).
constexpr size_t pipe_al(size_t x) { return (x + 15) & ~size_t(15); }

template <int NCW_>
struct PipeCfg {
    static constexpr int NCW = NCW_;             // chunk waves (4 or 8); the state waves are 4
    static constexpr int DK = 128;
    static constexpr int C = 64;
    static constexpr int NT = C / 16;            // 16-token row tiles
    static constexpr int NTB = NT / 2;           // 32-token contraction blocks
    static constexpr int NTH = 64 * (NCW + 4);   // threads per workgroup
    static constexpr int NCTH = 64 * NCW;        // chunk-wave threads
    static constexpr int NQ = DK / 4;            // channel quads
    static constexpr int NSEG = NCTH / NQ;       // token segments of the chunk waves
    static constexpr int TPS = C / NSEG;         // tokens per segment
    static constexpr int G = C / 16;             // tokens per decay group
    static constexpr int GPT = TPS / G;          // decay groups per segment
    static constexpr int SPT = 16 / G;           // decay groups per tile
    static constexpr int NCT = 2;                // 16-column tiles per state wave
    // Pitches (elements).  Fragment loads are pairs of 8-byte reads 32 bytes apart; measured on
    // gfx950 they are bank-conflict free at row pitches of 66 or 34 dwords and two-way conflicted
    // at 68 or 36 (and four-way at 72 or 40).  K'^T keeps 72 elements: its rows are permuted
    // (below), which makes both its transposed stores and its fragment loads conflict free.
    static constexpr int PK = DK + 4;            // pitch of [C][DK] operand arrays (66 dwords)
    static constexpr int PT = C + 8;             // pitch of K'^T rows
    static constexpr int PTB = C + 4;            // pitch of the T/A and Bqk rows (34 dwords)
    static constexpr int PV = DK + 8;            // pitch of the value rows
    static constexpr int PD = 20;
    static constexpr int PDB = 16 * PD + 16;
    static constexpr int VROWS = NCTH / 16;      // value rows per pass of the chunk threads
    static constexpr int NVV = C / VROWS;        // 16-byte value vectors per chunk thread
    // Interval (1..4, at its end) of the current chunk in which each row of the next chunk's
    // inputs is requested, 4 bits per row (row i in bits 4i..4i+3): decay input (consumed by
    // phase A in interval 4: 1..3), q and k (consumed by A' in the next interval 2: 2..4), the
    // value vectors and beta (handed over in the next interval 2: 2..4).  Spreading the requests
    // keeps the vector-memory queue from filling in one burst; measured on the model-width
    // workload (values and beta at the end of interval 3 rather than 4: 6-9% per launch).
    static constexpr uint32_t LD_LA = 0x11111111u;
    static constexpr uint32_t LD_Q = 0x44444444u;
    static constexpr uint32_t LD_K = 0x44444444u;
    static constexpr uint32_t LD_V = 0x33333333u;
    static constexpr int LD_B = 3;

    // state-wave operands of one chunk (written by the chunk waves, read by the state waves)
    static constexpr size_t oQt = 0;
    static constexpr size_t oKt = oQt + pipe_al(2 * C * PK);
    static constexpr size_t oKpT = oKt + pipe_al(2 * C * PK);
    static constexpr size_t oTA = oKpT + pipe_al(2 * DK * PT);
    static constexpr size_t oB = oTA + pipe_al(2 * C * PTB);
    static constexpr size_t oV = oB + pipe_al(2 * C * PTB);
    static constexpr size_t oBeta = oV + pipe_al(2 * C * PV);
    static constexpr size_t oGam = oBeta + pipe_al(4 * C);
    // chunk-wave scratch
    static constexpr size_t oLq = oGam + pipe_al(4 * DK);
    static constexpr size_t oLk = oLq + pipe_al(2 * C * PK);
    static constexpr size_t oKd = oLk + pipe_al(2 * C * PK);
    static constexpr size_t oTot = oKd + pipe_al(2 * C * PK);
    static constexpr size_t oD = oTot + pipe_al(4 * 16 * DK);
    static constexpr size_t oE = oD + pipe_al(4 * (NT + 3) * DK);   // D rows, then the products
    static constexpr size_t oF = oE + pipe_al(4 * (NT + 1) * DK);
    static constexpr size_t oAd = oF + pipe_al(4 * NT * DK);
    static constexpr size_t LDS = oAd + pipe_al(4 * NT * PDB);
    static_assert(LDS <= 160 * 1024, "LDS budget of one gfx950 workgroup");
    static_assert(NT == 4, "the D table's product rows cover pairs up to three tiles apart");
    static_assert((NCW == 4 && TPS == 8) || (NCW == 8 && TPS == 4), "segment layout of the chunk waves");
    static_assert(TPS % G == 0 && NSEG % NT == 0, "segments hold whole decay groups");
    static_assert(oB + 2 * C * PTB - oTA < 65536 && oKd + 2 * C * PK - oLq < 65536, "immediate offsets");
    static_assert(PK % 4 == 0 && PTB % 4 == 0 && PT % 4 == 0 && PV % 8 == 0, "8-byte rows (16 for values)");
};

// Chunk wave that forms the pi-th tile pair (pairs enumerated row by row), and the interval it
// does so in.  Diagonal pairs are the cheapest, pairs far below the diagonal the dearest.  The
// diagonal pairs feed the inverses of interval 4 and stay in interval 3; with 8 chunk waves two
// off-diagonal pairs move to interval 4 on waves that do not invert, so that interval 3 holds
// one pair per wave.
template <int NCW>
constexpr int pipe_pair_owner(int pi) {
    constexpr int own4[10] = {0, 2, 3, 1, 2, 3, 0, 1, 3, 2};
    constexpr int own8[10] = {0, 4, 1, 6, 5, 2, 4, 5, 7, 3};
    return NCW == 4 ? own4[pi] : own8[pi];
}
template <int NCW>
constexpr int pipe_pair_interval(int pi) {
    constexpr int iv8[10] = {3, 4, 3, 3, 4, 3, 3, 3, 3, 3};
    return NCW == 4 ? 3 : iv8[pi];
}

// Unit (sequence b, head h, segment s) of one workgroup and its token range.
struct PipeUnit {
    int b, h, s, bh;
    long long t_begin, t_end;
    int nchunks;
    bool cut;              // the sequence split's limit ran fewer chunks than the segment holds
    long long HD;          // token stride of every [B, T, H, d] tensor
    long long base_tok;    // element offset of (b, token 0, h, 0)
};

// Chunk waves (0 .. NCW-1): for each chunk in order, phases A, A', B and the diagonal inverses
// (waves 0..3, one block each), handing the state waves every operand they read.  Four barriers
// per chunk, then four more while the state waves run the last chunk.
template <int NCW, bool GATE>
__device__ __forceinline__ void pipe_chunk_waves(const PrefillArgs& a, const PipeUnit& u, KDA_LDS char* smem,
                                                 const int tid, const int wave) {
    using Cfg = PipeCfg<NCW>;
    using OpT = __bf16;
    using TIn = __bf16;
    using QI = Quad<TIn>;
    using QO = Quad<OpT>;
    constexpr int DK = Cfg::DK, C = Cfg::C, NT = Cfg::NT, NQ = Cfg::NQ;
    constexpr int TPS = Cfg::TPS, G = Cfg::G, GPT = Cfg::GPT, SPT = Cfg::SPT;
    constexpr int PK = Cfg::PK, PT = Cfg::PT, PTB = Cfg::PTB, PV = Cfg::PV, PD = Cfg::PD, PDB = Cfg::PDB, NVV = Cfg::NVV;
    constexpr int NSEG = Cfg::NSEG, VROWS = Cfg::VROWS;
    constexpr int NKB = DK / 32;
    constexpr int eLk = (int)((Cfg::oLk - Cfg::oLq) / 2);
    constexpr int eKd = (int)((Cfg::oKd - Cfg::oLq) / 2);
    constexpr int eKt = (int)((Cfg::oKt - Cfg::oQt) / 2);
    constexpr int eBw = (int)((Cfg::oB - Cfg::oTA) / 2);

    KDA_LDS OpT* sQt = reinterpret_cast<KDA_LDS OpT*>(smem + Cfg::oQt);
    KDA_LDS OpT* sKpT = reinterpret_cast<KDA_LDS OpT*>(smem + Cfg::oKpT);
    KDA_LDS OpT* sTA = reinterpret_cast<KDA_LDS OpT*>(smem + Cfg::oTA);
    KDA_LDS TIn* sV = reinterpret_cast<KDA_LDS TIn*>(smem + Cfg::oV);
    KDA_LDS float* sBeta = reinterpret_cast<KDA_LDS float*>(smem + Cfg::oBeta);
    KDA_LDS float* sGam = reinterpret_cast<KDA_LDS float*>(smem + Cfg::oGam);
    KDA_LDS OpT* sLq = reinterpret_cast<KDA_LDS OpT*>(smem + Cfg::oLq);
    KDA_LDS float* sTot = reinterpret_cast<KDA_LDS float*>(smem + Cfg::oTot);
    KDA_LDS float* sD = reinterpret_cast<KDA_LDS float*>(smem + Cfg::oD);
    KDA_LDS float* sE = reinterpret_cast<KDA_LDS float*>(smem + Cfg::oE);
    KDA_LDS float* sF = reinterpret_cast<KDA_LDS float*>(smem + Cfg::oF);
    KDA_LDS float* sAd = reinterpret_cast<KDA_LDS float*>(smem + Cfg::oAd);

    const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int cq = tid % NQ, sg = tid / NQ;   // channel quad, token segment
    const int ch0 = 4 * cq;
    KDA_LDS OpT* const pA = lds_pin(sLq + sg * TPS * PK + ch0);         // rows of Lq, Lk, Kd
    KDA_LDS OpT* const pQK = lds_pin(sQt + sg * TPS * PK + ch0);        // rows of Q~, K~
    // K'^T rows hold their 4-token groups permuted by row, column c at c ^ 4 ((row >> 3) & 15):
    // the transposed stores below then hit distinct LDS banks (the plain layout serialises them
    // about 4-fold), and the state waves' fragment loads stay conflict-free
    const int kswz = 4 * ((cq >> 1) & 15);                              // ((ch0 + e) >> 3) == cq >> 1
    KDA_LDS OpT* const pKp0 = lds_pin(sKpT + ch0 * PT + ((sg * TPS) ^ kswz));
    KDA_LDS OpT* const pKp1 = lds_pin(sKpT + ch0 * PT + ((sg * TPS + 4) ^ kswz));   // TPS == 8
    KDA_LDS float* const pTotW = lds_pin(sTot + sg * GPT * DK + ch0);
    KDA_LDS OpT* const pK = lds_pin(sLq + lr * PK + 4 * lg);            // fragment rows (tile pairs)
    KDA_LDS float* const pG = lds_pin(sD + 4 * lg);                     // D table by accumulator row
    KDA_LDS float* const pBe = lds_pin(sBeta + 4 * lg);                 // beta by accumulator row
    KDA_LDS OpT* const pW = lds_pin(sTA + 4 * lg * PTB + lr);           // accumulator element of TA, B
    KDA_LDS float* const pAd = lds_pin(sAd + 4 * lg * PD + lr);         // diagonal block, row-major
    const int wi = wave & (NT - 1);                                     // diagonal block (waves < NT)
    KDA_LDS float* const pAi = lds_pin(sAd + wi * PDB + (lane & 15) * PD);
    KDA_LDS OpT* const pTi = lds_pin(sTA + 16 * wi * (PTB + 1) + (lane & 15) * PTB + (lane >> 4));
    const int v_row = tid / 16, v_off = (tid % 16) * 8;                 // value rows: 16 vectors each
    KDA_LDS TIn* const pVc = lds_pin(sV + v_row * PV + v_off);

    const long long HD = u.HD, t_end = u.t_end;
    const TIn* gq = reinterpret_cast<const TIn*>(a.q) + u.base_tok;
    const TIn* gk = reinterpret_cast<const TIn*>(a.k) + u.base_tok;
    constexpr int LAE = GATE ? 2 : 4;                          // bytes per decay-input element
    const char* gla = GATE ? reinterpret_cast<const char*>(a.gate) + u.base_tok * 2
                           : reinterpret_cast<const char*>(a.log_alpha + u.base_tok);
    const long long HDL = HD * LAE;
    const TIn* gv = reinterpret_cast<const TIn*>(a.v) + u.base_tok;
    const float* gbeta = a.beta + (long long)u.b * a.T * a.H + u.h;
    const uint32_t HD2 = (uint32_t)(HD * 2), HDL32 = (uint32_t)HDL;   // token strides in bytes

    // Prefetch of a chunk into registers.  Every address is a uniform row base plus a 32-bit lane
    // offset; rows past the end of the unit re-read its last row (in bounds).  Such rows need no
    // zeroing: their decay, beta and value are zeroed where they are consumed, so their U rows are
    // exactly zero and they add nothing to the state or to earlier outputs.
    using LaRaw = std::conditional_t<GATE, u32x2_t, f32x4_t>;
    typename QI::raw pq[TPS], pk[TPS];
    LaRaw pla[TPS];
    u32x4_t pv[NVV];
    float pbeta = 0.0f;
    auto last_row = [&](long long c0) { return (int)(t_end - 1 - c0 < C - 1 ? t_end - 1 - c0 : C - 1); };
    // requests for the rows of chunk c0 whose schedule entry is iv
    auto load_rows = [&](long long c0, int iv) {
        const int last = last_row(c0);
        const char* bl = gla + c0 * HDL;
        const TIn* bq = gq + c0 * HD;
        const TIn* bk = gk + c0 * HD;
        const TIn* bv = gv + c0 * HD;
#pragma unroll
        for (int i = 0; i < TPS; ++i) {
            const uint32_t r = (uint32_t)min(sg * TPS + i, last);
            if (((Cfg::LD_LA >> (4 * i)) & 15) == (uint32_t)iv)
                pla[i] = *reinterpret_cast<const LaRaw*>(at_byte(bl, pinned_u(r * HDL32 + (uint32_t)(ch0 * LAE))));
            if (((Cfg::LD_Q >> (4 * i)) & 15) == (uint32_t)iv) pq[i] = QI::load(at_byte(bq, pinned_u(r * HD2 + (uint32_t)(ch0 * 2))));
            if (((Cfg::LD_K >> (4 * i)) & 15) == (uint32_t)iv) pk[i] = QI::load(at_byte(bk, pinned_u(r * HD2 + (uint32_t)(ch0 * 2))));
        }
#pragma unroll
        for (int m = 0; m < NVV; ++m) {
            if (((Cfg::LD_V >> (4 * m)) & 15) == (uint32_t)iv) {
                const uint32_t r = (uint32_t)min(v_row + VROWS * m, last);
                pv[m] = *reinterpret_cast<const u32x4_t*>(at_byte(bv, pinned_u(r * HD2 + (uint32_t)(v_off * 2))));
            }
        }
        if (Cfg::LD_B == iv)
            pbeta = *at_byte(gbeta + c0 * a.H, pinned_u((uint32_t)min(tid % C, last) * (uint32_t)(a.H * 4)));
    };
    // next chunk's inputs due for request at the end of interval iv
    auto prefetch = [&](int iv, int c, long long c0) {
        if (c + 1 < u.nchunks) load_rows(c0 + C, iv);
    };

    // A: log2-decay summed inside decay groups of G tokens (g, kept in registers until A');
    // group totals to LDS
    float g[TPS][4];
    auto phase_a = [&](long long c0) {
        const int lastr = last_row(c0);
        bool okt[TPS];
#pragma unroll
        for (int i = 0; i < TPS; ++i) okt[i] = sg * TPS + i <= lastr;
        float run[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < TPS; ++i) {
            f32x4_t l4;
            if constexpr (GATE) {
                // log alpha = -5 sigmoid(x) = -5 / (1 + 2^{-x log2 e})
                const u32x2_t xr = pla[i];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t w = e < 2 ? xr[0] : xr[1];
                    const float x = __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
                    l4[e] = kLogAlphaMin * __builtin_amdgcn_rcpf(1.0f + fast_exp2(-x * kLog2e));
                }
            } else {
                l4 = pla[i];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float l = okt[i] ? __builtin_amdgcn_fmed3f(l4[e], kLogAlphaMin, 0.0f) : 0.0f;
                run[e] = (i % G == 0) ? l * kLog2e : fmaf(l, kLog2e, run[e]);
                g[i][e] = run[e];
            }
            if (i % G == G - 1)
                *reinterpret_cast<KDA_LDS f32x4_t*>(pTotW + (i / G) * DK) = f32x4_t{run[0], run[1], run[2], run[3]};
        }
    };
    // Prefix pass, one channel per thread (threads 0..DK-1): from the group totals, in the
    // canonical order (group totals in order inside a tile, tile totals in order across the
    // chunk), rho_a for every tile and, in place of each group total, the sum of the groups
    // before it inside its tile; then the tables 2^{rho_a} (a = 0..NT), D_a = 2^{rho_{a+1} - rho_a}
    // and 2^{g_C - rho_{a+1}}, and after the D rows the products D_0 D_1, D_1 D_2, (D_0 D_1) D_2
    // that scale the tile pairs two and three tiles below the diagonal.
    auto prefix_pass = [&]() {
        const int ch = tid;
        float tot[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) tot[j] = sTot[j * DK + ch];
        float Rt[NT + 1];
        Rt[0] = 0.0f;
#pragma unroll
        for (int a2 = 0; a2 < NT; ++a2) {
            float run = 0.0f;
#pragma unroll
            for (int j = 0; j < SPT; ++j) {
                sTot[(a2 * SPT + j) * DK + ch] = run;
                if (j + 1 < SPT) run = run + tot[a2 * SPT + j];
            }
            float tt = tot[a2 * SPT];
#pragma unroll
            for (int j = 1; j < SPT; ++j) tt = tt + tot[a2 * SPT + j];
            Rt[a2 + 1] = Rt[a2] + tt;
        }
#pragma unroll
        for (int a2 = 0; a2 <= NT; ++a2) sE[a2 * DK + ch] = fast_exp2(Rt[a2]);
        float dd[NT];
#pragma unroll
        for (int a2 = 0; a2 < NT; ++a2) {
            dd[a2] = fast_exp2(Rt[a2 + 1] - Rt[a2]);
            sD[a2 * DK + ch] = dd[a2];
            sF[a2 * DK + ch] = fast_exp2(Rt[NT] - Rt[a2 + 1]);
        }
        const float d01 = dd[0] * dd[1];
        sD[NT * DK + ch] = d01;
        sD[(NT + 1) * DK + ch] = dd[1] * dd[2];
        sD[(NT + 2) * DK + ch] = d01 * dd[2];
    };
    static_assert(16 / G == Cfg::SPT && NT * Cfg::SPT == 16, "16 decay groups per chunk");
    static_assert(TPS <= 8 && NVV <= 8, "4-bit schedule entries per row");

    // B: decay-weighted KK^T and QK^T tiles of the pairs this wave forms in interval iv, one
    // dense product per tile pair
    auto tile_pairs = [&](int iv) {
            constexpr int NP = NT * (NT + 1) / 2;
            static_for<0, NP>([&](auto PIc) {
                constexpr int pi = decltype(PIc)::value;
                constexpr int ar = pair_row(pi);
                constexpr int ac = pi - ar * (ar + 1) / 2;
                if (pipe_pair_owner<NCW>(pi) != wave || pipe_pair_interval<NCW>(pi) != iv) return;   // wave-uniform
                f32x4_t accA = zero4(), accB = zero4();
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    Frag<OpT> fk, fq, fr;
                    frag_ld(fk, pK + eLk + 16 * ar * PK + 32 * kb);
                    frag_ld(fq, pK + 16 * ar * PK + 32 * kb);
                    frag_ld(fr, pK + eKd + 16 * ac * PK + 32 * kb);
                    if constexpr (ac < ar) {
                        // R = Kd 2^{rho_ar - rho_ac}: one multiply by D_ac or by a product row
                        constexpr int prow = (ar - ac == 1) ? ac : (ar - ac == 2 ? NT + ac : NT + 2);
                        float val[8], d8[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j) val[j] = fr.get(j);
                        f32x8_ld(d8, pG + prow * DK + 32 * kb);
#pragma unroll
                        for (int j = 0; j < 8; ++j) val[j] *= d8[j];
#pragma unroll
                        for (int j = 0; j < 8; ++j) fr.set(j, val[j]);
                    }
                    accA = mma(fk, fr, accA);
                    accB = mma(fq, fr, accB);
                }
                const f32x4_t bt4 = *reinterpret_cast<const KDA_LDS f32x4_t*>(pBe + 16 * ar);
                if constexpr (ac == ar) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int rl = 4 * lg + j;
                        pAd[ar * PDB + j * PD] = (lr < rl) ? accA[j] * bt4[j] : 0.0f;
                        pW[eBw + 16 * ar * PTB + 16 * ac + j * PTB] = from_f32<OpT>((lr <= rl) ? accB[j] : 0.0f);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        pW[16 * ar * PTB + 16 * ac + j * PTB] = from_f32<OpT>(-accA[j] * bt4[j]);
                        pW[eBw + 16 * ar * PTB + 16 * ac + j * PTB] = from_f32<OpT>(accB[j]);
                    }
                }
            });
    };

    const int nchunks = u.nchunks;
    if (nchunks > 0) {
#pragma unroll
        for (int iv = 1; iv <= 4; ++iv) load_rows(u.t_begin, iv);
        phase_a(u.t_begin);
    }
    for (int c = 0; c < nchunks; ++c) {
        const long long c0 = u.t_begin + (long long)c * C;
        barrier_lds();

        // ---- interval 1: prefix pass over this chunk's group totals (written by phase A in the
        //      previous interval 4, or before the loop) ----
        if (tid < DK) prefix_pass();
        prefetch(1, c, c0);
        barrier_lds();

        // ---- interval 2, A': decay-scaled operands ----
        typename QO::raw qtr[TPS], ktr[TPS];   // Q~, K~ of own rows
        uint32_t kp[4][TPS / 2];               // K' of own channels, bf16 pairs of tokens
        {
            // hand over v and beta of this chunk first (the state waves read the previous chunk's
            // in interval 4 of the previous iteration), freeing their registers
#pragma unroll
            for (int m = 0; m < NVV; ++m) {
                const bool ok = c0 + v_row + VROWS * m < t_end;
                const u32x4_t x = pv[m];
                *reinterpret_cast<KDA_LDS u32x4_t*>(pVc + VROWS * m * PV) =
                    u32x4_t{ok ? x[0] : 0u, ok ? x[1] : 0u, ok ? x[2] : 0u, ok ? x[3] : 0u};
            }
            if (tid < C) sBeta[tid] = (c0 + tid < t_end) ? pbeta : 0.0f;

            const int at = (sg * TPS) / 16;    // this segment's row tile
            f32x4_t gp[GPT];                   // in-tile sums before own groups
#pragma unroll
            for (int m = 0; m < GPT; ++m) gp[m] = *reinterpret_cast<const KDA_LDS f32x4_t*>(pTotW + m * DK);
            const f32x4_t er4 = *reinterpret_cast<const KDA_LDS f32x4_t*>(sE + at * DK + ch0);   // 2^{rho_a}
            const f32x4_t fd4 = *reinterpret_cast<const KDA_LDS f32x4_t*>(sD + at * DK + ch0);   // 2^{rho_{a+1} - rho_a}
            const f32x4_t fc4 = *reinterpret_cast<const KDA_LDS f32x4_t*>(sF + at * DK + ch0);   // 2^{g_C - rho_{a+1}}
            float fd[4], fc[4], er[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                fd[e] = fd4[e];
                fc[e] = fc4[e];
                er[e] = er4[e];
            }
#pragma unroll
            for (int i = 0; i < TPS; ++i) {
                float lq[4], lk[4], kd[4], qt[4], kt[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float loc = gp[i / G][e] + g[i][e];   // g - rho_a, in [-115.4, 0]
                    const float x = fast_exp2(loc);
                    const float y = fast_exp2(-loc);
                    const float kv = QI::get(pk[i], e);
                    const float qv = QI::get(pq[i], e);
                    lq[e] = qv * x;
                    qt[e] = lq[e] * er[e];   // q 2^{g} = (q 2^{g - rho_a}) 2^{rho_a}
                    lk[e] = kv * x;
                    kt[e] = lk[e] * er[e];
                    kd[e] = kv * y;
                    const float kpv = (kd[e] * fd[e]) * fc[e];
                    if (i & 1) kp[e][i / 2] |= (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)kpv) << 16;
                    else kp[e][i / 2] = __builtin_bit_cast(uint16_t, (__bf16)kpv);
                }
                QO::store(pA + i * PK, lq[0], lq[1], lq[2], lq[3]);
                QO::store(pA + eLk + i * PK, lk[0], lk[1], lk[2], lk[3]);
                QO::store(pA + eKd + i * PK, kd[0], kd[1], kd[2], kd[3]);
                qtr[i] = QO::pack(qt[0], qt[1], qt[2], qt[3]);
                ktr[i] = QO::pack(kt[0], kt[1], kt[2], kt[3]);
            }
        }
        prefetch(2, c, c0);
        barrier_lds();

        // ---- interval 3: hand over K~ and Q~ (the state waves read the previous chunk's in
        //      intervals 1 and 2), then the tile pairs of B due in this interval ----
#pragma unroll
        for (int i = 0; i < TPS; ++i) {
            QO::store_raw(pQK + i * PK, qtr[i]);
            QO::store_raw(pQK + eKt + i * PK, ktr[i]);
        }
        tile_pairs(3);
        prefetch(3, c, c0);
        barrier_lds();

        // ---- interval 4: diagonal blocks T_aa = (I + A_aa)^{-1}, wave a inverting block a by
        //      forward substitution with the pivot row broadcast inside 16-lane rows (DPP) ----
        if (wave < NT) {
            const int p = lane & 15, cgp = lane >> 4;
            float na[16];   // -A_aa[p][i]
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4_t v4 = *reinterpret_cast<const KDA_LDS f32x4_t*>(pAi + 4 * q4);
                na[4 * q4] = -v4[0]; na[4 * q4 + 1] = -v4[1]; na[4 * q4 + 2] = -v4[2]; na[4 * q4 + 3] = -v4[3];
            }
            float t[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) t[r] = (p == cgp + 4 * r) ? 1.0f : 0.0f;
            static_for<0, 15>([&](auto I) {
                constexpr int i = decltype(I)::value;
#pragma unroll
                for (int r = 0; r < 4; ++r) t[r] = fmaf(row_bcast<i>(t[r]), na[i], t[r]);
            });
#pragma unroll
            for (int r = 0; r < 4; ++r) pTi[4 * r] = from_f32<OpT>(t[r]);
        }
        // hand over K'^T and 2^{g_C} (the state waves read the previous chunk's in interval 3)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            *reinterpret_cast<KDA_LDS u32x2_t*>(pKp0 + e * PT) = u32x2_t{kp[e][0], kp[e][1]};
            if constexpr (TPS == 8)
                *reinterpret_cast<KDA_LDS u32x2_t*>(pKp1 + e * PT) = u32x2_t{kp[e][2], kp[e][3]};
        }
        if (sg == 0)
            *reinterpret_cast<KDA_LDS f32x4_t*>(sGam + ch0) = *reinterpret_cast<const KDA_LDS f32x4_t*>(sE + NT * DK + ch0);
        tile_pairs(4);
        // A of the next chunk (its prefix pass opens the next iteration)
        if (c + 1 < nchunks) {
#pragma unroll
            for (int i = 0; i < TPS; ++i) reg_pin(pla[i]);
            phase_a(c0 + C);
        }
        prefetch(4, c, c0);
    }
    // the state waves run the last chunk
#pragma unroll
    for (int i = 0; i < 4; ++i) barrier_lds();
}

// Operand sequence of the state waves' output product: for each row tile ar, the NKB blocks of
// Q~ (bqk = false, kb = block), then the blocks kb = 0 .. ar/2 of Bqk (bqk = true).
struct PipeOStep {
    int ar, kb;
    bool bqk;
};
constexpr PipeOStep pipe_o_step(int i, int nt, int nkb) {
    for (int ar = 0; ar < nt; ++ar) {
        const int n = nkb + ar / 2 + 1;
        if (i < n) return PipeOStep{ar, i < nkb ? i : i - nkb, i >= nkb};
        i -= n;
    }
    return PipeOStep{-1, 0, false};
}
constexpr int pipe_o_steps(int nt, int nkb) {
    int n = 0;
    for (int ar = 0; ar < nt; ++ar) n += nkb + ar / 2 + 1;
    return n;
}

// State waves (NCW .. NCW+3): state wave sw holds state columns 32 sw .. 32 sw + 31 in
// fp32 registers and runs the state-dependent products of each chunk.  Four barriers while the
// chunk waves prepare the first chunk, then four per chunk.
template <int NCW>
__device__ __forceinline__ void pipe_state_waves(const PrefillArgs& a, const PipeUnit& u, KDA_LDS char* smem,
                                                 const int tid, const int sw) {
    using Cfg = PipeCfg<NCW>;
    using OpT = __bf16;
    using TIn = __bf16;
    constexpr int DK = Cfg::DK, C = Cfg::C, NT = Cfg::NT, NTB = Cfg::NTB, NCT = Cfg::NCT;
    constexpr int PK = Cfg::PK, PT = Cfg::PT, PTB = Cfg::PTB, PV = Cfg::PV;
    constexpr int NIT = DK / 16, NKB = DK / 32;
    constexpr int eKt = (int)((Cfg::oKt - Cfg::oQt) / 2);
    constexpr int eBs = (int)((Cfg::oB - Cfg::oTA) / 2);

    KDA_LDS OpT* sQt = reinterpret_cast<KDA_LDS OpT*>(smem + Cfg::oQt);
    KDA_LDS OpT* sKpT = reinterpret_cast<KDA_LDS OpT*>(smem + Cfg::oKpT);
    KDA_LDS OpT* sTA = reinterpret_cast<KDA_LDS OpT*>(smem + Cfg::oTA);
    KDA_LDS TIn* sV = reinterpret_cast<KDA_LDS TIn*>(smem + Cfg::oV);
    KDA_LDS float* sBeta = reinterpret_cast<KDA_LDS float*>(smem + Cfg::oBeta);
    KDA_LDS float* sGam = reinterpret_cast<KDA_LDS float*>(smem + Cfg::oGam);

    const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int colw = 32 * sw;   // first state column of this wave

    // lane holds S[16 it + 4 lg + j][colw + 16 ct + lr]; its byte offset in a DK x DK state, formed
    // where it is used (kept opaque so that no 64-bit addresses are held across the chunk loop)
    auto st_off = [&](int it, int ct, int j) {
        return pinned_u((uint32_t)(((16 * it + 4 * lg + j) * DK + colw + 16 * ct + lr) * 4));
    };
    f32x4_t st[NIT][NCT];
    if (a.init_mode == 1 || (a.init_mode == 3 && u.s == 0)) {
        const float* sin = a.s_in + (long long)u.bh * a.sin_bh_stride + (long long)u.s * a.sin_seg_stride;
#pragma unroll
        for (int it = 0; it < NIT; ++it)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    st[it][ct][j] = *at_byte(sin, st_off(it, ct, j));
    } else {
        const bool ident = a.init_mode == 2;
#pragma unroll
        for (int it = 0; it < NIT; ++it)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    st[it][ct][j] = (ident && 16 * it + 4 * lg + j == colw + 16 * ct + lr) ? 1.0f : 0.0f;
    }

    KDA_LDS OpT* const pQs = lds_pin(sQt + lr * PK + 4 * lg);             // fragment rows of Q~, K~
    KDA_LDS OpT* const pTs = lds_pin(sTA + lr * PTB + 4 * lg);            // fragment rows of TA, B
    // fragment rows of the permuted K'^T (row 16 it + lr holds column c at c ^ (8 it + 4 (lr >> 3))):
    // one base for even and one for odd it, the rest of the permutation is an immediate offset
    const int hsw = lr >> 3;
    KDA_LDS OpT* const pKs0 = lds_pin(sKpT + lr * PT + 4 * (lg ^ hsw));
    KDA_LDS OpT* const pKs1 = lds_pin(sKpT + lr * PT + ((4 * (lg ^ hsw)) ^ 8));
    KDA_LDS TIn* const pVs = lds_pin(sV + 4 * lg * PV + colw + lr);       // value in accumulator layout
    KDA_LDS float* const pBs = lds_pin(sBeta + 4 * lg);
    KDA_LDS float* const pGs = lds_pin(sGam + 4 * lg);
    TIn* const go = a.o ? reinterpret_cast<TIn*>(a.o) + u.base_tok : nullptr;
    // outputs are formed transposed (O^T = S^T Q~^T + U^T Bqk^T: the same fragments with the
    // operands swapped), so a lane holds 4 adjacent outputs of one token: token lr of the tile,
    // columns colw + 16 ct + 4 lg .. + 3, stored with one 8-byte store
    const uint32_t boO = (uint32_t)((lr * u.HD + colw + 4 * lg) * 2);
    const long long HD = u.HD, t_end = u.t_end;

    // S as an operand, one 32-row block at a time: B operand of K~ S and Q~ S, or equally the A
    // operand of S^T Q~^T (the fragment layout is the same for both roles)
    auto s_frag = [&](Frag<OpT> (&fs)[NCT], int kb) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) acc_pair_frag(fs[ct], st[2 * kb][ct], st[2 * kb + 1][ct], true);
    };
    // X = K~ S and RHS = beta (V - X) of a chunk, from the state before it
    f32x4_t Rh[NT][NCT];
    auto x_rhs = [&]() {
#pragma unroll
        for (int ar = 0; ar < NT; ++ar)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) Rh[ar][ct] = zero4();
        // K~ fragments one contraction block ahead: the loads of block kb + 1 are issued before
        // the products of block kb, so their LDS latency overlaps the matrix-core work
        Frag<OpT> fk[2][NT];
#pragma unroll
        for (int ar = 0; ar < NT; ++ar) frag_ld(fk[0][ar], pQs + eKt + 16 * ar * PK);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            if (kb + 1 < NKB) {
#pragma unroll
                for (int ar = 0; ar < NT; ++ar) frag_ld(fk[(kb + 1) & 1][ar], pQs + eKt + 16 * ar * PK + 32 * (kb + 1));
            }
            __builtin_amdgcn_sched_barrier(0);
            Frag<OpT> fs[NCT];
            s_frag(fs, kb);
#pragma unroll
            for (int ar = 0; ar < NT; ++ar)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) Rh[ar][ct] = mma(fk[kb & 1][ar], fs[ct], Rh[ar][ct]);
        }
#pragma unroll
        for (int ar = 0; ar < NT; ++ar) {
            const f32x4_t bt4 = *reinterpret_cast<const KDA_LDS f32x4_t*>(pBs + 16 * ar);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    Rh[ar][ct][j] = bt4[j] * (to_f32<TIn>(pVs[(16 * ar + j) * PV + 16 * ct]) - Rh[ar][ct][j]);
        }
    };

    // the chunk waves prepare the first chunk; its X and RHS run beside their diagonal inverses
#pragma unroll
    for (int i = 0; i < 4; ++i) barrier_lds();
    if (u.nchunks > 0) x_rhs();

    for (int c = 0; c < u.nchunks; ++c) {
        const long long c0 = u.t_begin + (long long)c * C;
        barrier_lds();

        // ---- interval 1: U_a = T_aa (RHS_a - sum_{b<a} A_ab U_b) ----
        f32x4_t U[NT][NCT];
        Frag<OpT> fU[NTB][NCT];
        // every T/A fragment of the solve is requested up front (they were written in the previous
        // interval 4), so the chain of dependent products below waits on LDS at most once
        static_assert(NT == 4, "fragment list of the blocked solve");
        Frag<OpT> fsol[8];   // T00 | A10, T11 | A2(0..31), T22 | A3(0..31), A32, T33
        frag_ld_lo(fsol[0], pTs);
        frag_ld_lo(fsol[1], pTs + 16 * PTB);
        frag_ld_lo(fsol[2], pTs + 16 * PTB + 16);
        frag_ld(fsol[3], pTs + 32 * PTB);
        frag_ld_lo(fsol[4], pTs + 32 * PTB + 32);
        frag_ld(fsol[5], pTs + 48 * PTB);
        frag_ld_lo(fsol[6], pTs + 48 * PTB + 32);
        frag_ld_lo(fsol[7], pTs + 48 * PTB + 48);
        __builtin_amdgcn_sched_barrier(0);
        constexpr int sol_first[NT] = {0, 1, 3, 5};
#pragma unroll
        for (int ar = 0; ar < NT; ++ar) {
            int fi = sol_first[ar];
            f32x4_t W[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) W[ct] = Rh[ar][ct];
#pragma unroll
            for (int kb = 0; kb < ar / 2; ++kb) {
                const Frag<OpT>& fa = fsol[fi++];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) W[ct] = mma(fa, fU[kb][ct], W[ct]);
            }
            if (ar & 1) {
                const Frag<OpT>& fa = fsol[fi++];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    Frag<OpT> fb;
                    acc_pair_frag(fb, U[ar - 1][ct], U[ar - 1][ct], false);
                    W[ct] = mma(fa, fb, W[ct]);
                }
            }
            const Frag<OpT>& ft = fsol[fi];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                Frag<OpT> fw;
                acc_pair_frag(fw, W[ct], W[ct], false);
                U[ar][ct] = mma(ft, fw, zero4());
            }
            if (ar & 1) {
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) acc_pair_frag(fU[ar / 2][ct], U[ar - 1][ct], U[ar][ct], true);
            }
        }
        barrier_lds();

        // ---- interval 2: O^T = S^T Q~^T + U^T Bqk^T, stored from the accumulators ----
        // One row tile at a time: its four Q~ blocks, then its Bqk blocks kb = 0 .. ar/2, with the
        // operand fragments loaded OLA steps ahead of their products (a rolling buffer), so the
        // LDS latency overlaps the matrix-core work.  The accumulation order per output element is
        // the same as block by block over all row tiles.
        if (go) {
            Frag<OpT> fsa[NKB][NCT];   // S as the A operand, all 128 rows
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) s_frag(fsa[kb], kb);
            constexpr int NS = pipe_o_steps(NT, NKB);
            constexpr int OLA = 3;
            Frag<OpT> fb[OLA + 1];
            auto o_load = [&](auto Ic) {
                constexpr int i = decltype(Ic)::value;
                constexpr PipeOStep st_i = pipe_o_step(i, NT, NKB);
                if constexpr (st_i.bqk) frag_ld(fb[i % (OLA + 1)], pTs + eBs + 16 * st_i.ar * PTB + 32 * st_i.kb);
                else frag_ld(fb[i % (OLA + 1)], pQs + 16 * st_i.ar * PK + 32 * st_i.kb);
            };
            static_for<0, OLA>([&](auto Ic) { o_load(Ic); });
            f32x4_t O[NCT];
            static_for<0, NS>([&](auto Ic) {
                constexpr int i = decltype(Ic)::value;
                constexpr PipeOStep st_i = pipe_o_step(i, NT, NKB);
                constexpr int ar = st_i.ar;
                if constexpr (i + OLA < NS) o_load(std::integral_constant<int, i + OLA>{});
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (!st_i.bqk && st_i.kb == 0) {
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) O[ct] = zero4();
                }
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    O[ct] = st_i.bqk ? mma(fU[st_i.kb][ct], fb[i % (OLA + 1)], O[ct])
                                     : mma(fsa[st_i.kb][ct], fb[i % (OLA + 1)], O[ct]);
                if constexpr (st_i.bqk && st_i.kb == ar / 2) {
                    if (c0 + 16 * ar + lr < t_end) {
                        TIn* const orow = go + (c0 + 16 * ar) * HD;
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct)
                            *reinterpret_cast<u32x2_t*>(at_byte(orow, pinned_u(boO + 32 * ct))) =
                                Quad<TIn>::pack(O[ct][0], O[ct][1], O[ct][2], O[ct][3]);
                    }
                }
            });
        }
        barrier_lds();

        // ---- interval 3: S <- Diag(2^{g_C}) S + K'^T U ----
        // 16 steps (row tile it, contraction block kb); the K'^T fragment of step i is requested
        // ULA steps ahead and the decay row of tile it one tile ahead, so that their LDS latency
        // overlaps the products of the steps between
        {
            constexpr int NUS = NIT * NTB, ULA = 4;
            Frag<OpT> fkb[ULA + 1];
            f32x4_t gmv[2];
            auto u_load = [&](auto Ic) {
                constexpr int i = decltype(Ic)::value;
                constexpr int it = i / NTB, kb = i % NTB;
                constexpr int hi = (8 * it) & 48;
                const KDA_LDS OpT* const kb0 = ((it & 1) ? pKs1 : pKs0) + 16 * it * PT;
                frag_ld2(fkb[i % (ULA + 1)], kb0 + ((32 * kb) ^ hi), kb0 + ((32 * kb + 16) ^ hi));
            };
            gmv[0] = *reinterpret_cast<const KDA_LDS f32x4_t*>(pGs);
            static_for<0, ULA>([&](auto Ic) { u_load(Ic); });
            static_for<0, NUS>([&](auto Ic) {
                constexpr int i = decltype(Ic)::value;
                constexpr int it = i / NTB, kb = i % NTB;
                if constexpr (i + ULA < NUS) u_load(std::integral_constant<int, i + ULA>{});
                if constexpr (kb == 0 && it + 1 < NIT)
                    gmv[(it + 1) & 1] = *reinterpret_cast<const KDA_LDS f32x4_t*>(pGs + 16 * (it + 1));
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (kb == 0) {
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                        for (int j = 0; j < 4; ++j) st[it][ct][j] *= gmv[it & 1][j];
                }
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) st[it][ct] = mma(fkb[i % (ULA + 1)], fU[kb][ct], st[it][ct]);
            });
        }
        if (a.s_ckpt) {   // the state after a full chunk ending on a multiple of ckpt_every
            const long long pend = c0 + C;
            if (pend <= t_end && pend % a.ckpt_every == 0) {
                const long long ci = pend / a.ckpt_every - 1;
                float* sc = a.s_ckpt + (((long long)u.b * a.n_ckpt + ci) * a.H + u.h) * (long long)(DK * DK);
#pragma unroll
                for (int it = 0; it < NIT; ++it)
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            *at_byte(sc, st_off(it, ct, j)) = st[it][ct][j];
            }
        }
        barrier_lds();

        // ---- interval 4: X and RHS of the next chunk (the chunk waves handed over its K~, V and
        //      beta in intervals 2 and 3 and invert its diagonal blocks meanwhile) ----
        if (c + 1 < u.nchunks) x_rhs();
    }

    // destination: s_out (when this segment's state is wanted), s_head for segment 0, s_tail for
    // the last segment; a cut unit has no final state of its own, except the last segment, whose
    // final state is then its increment, copied from s_tail
    float* so = (a.s_out && (a.out_seg < 0 || a.out_seg == u.s))
                    ? a.s_out + (long long)u.bh * a.sout_bh_stride + (long long)u.s * a.sout_seg_stride
                    : nullptr;
    const float* from = nullptr;
    if (u.s == 0 && a.s_head) so = a.s_head + (long long)u.bh * a.shead_bh_stride;
    if (u.s == a.tail_seg) {
        float* tail = a.s_tail ? a.s_tail + (long long)u.bh * a.stail_bh_stride : nullptr;
        if (!a.z_limit) so = tail;
        else if (u.cut) from = tail;
    }
    if (u.cut && !from) so = nullptr;
    if (so) {
#pragma unroll
        for (int it = 0; it < NIT; ++it)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *at_byte(so, st_off(it, ct, j)) = from ? *at_byte(from, st_off(it, ct, j)) : st[it][ct][j];
    }
}

// One workgroup per unit (sequence, head, segment), all 128 state columns.  The two roles run
// separate loops with the same number of workgroup barriers (4 per chunk plus 4), so every
// barrier is met by all eight waves; the registers of each role are allocated on its own.
template <int NCW, bool GATE>
__global__ __launch_bounds__(64 * (NCW + 4)) void kda_prefill_pipe_kernel(const PrefillArgs a) {
    using Cfg = PipeCfg<NCW>;
    constexpr int C = Cfg::C, PT = Cfg::PT, PTB = Cfg::PTB, DK = Cfg::DK, NTH = Cfg::NTH;
    __shared__ __align__(16) char smem_[Cfg::LDS];
    KDA_LDS char* smem = (KDA_LDS char*)smem_;

    const int bid = blockIdx.x;
    const int unit = (bid >> 3) * 8 + (bid & 7);
    if (unit >= a.n_units) return;
    PipeUnit u;
    const int sl = unit % a.n_seg_launch;
    u.bh = unit / a.n_seg_launch;
    u.h = u.bh % a.H;
    u.b = u.bh / a.H;
    u.s = a.seg0 + sl;
    u.t_begin = (long long)u.s * a.seg_len + (u.s > 0 ? a.seg_shift : 0);
    const long long t_next = (long long)(u.s + 1) * a.seg_len + a.seg_shift;
    u.t_end = t_next < a.T ? t_next : a.T;
    const long long ntok = u.t_end - u.t_begin;
    u.nchunks = ntok > 0 ? (int)((ntok + C - 1) / C) : 0;
    u.cut = false;
    // sequence split: skip a unit whose increment the transition pass already formed, or run only
    // the chunks over which the entry state still matters (unit-uniform, before any barrier)
    if (u.s > 0 && (a.z_gate || a.z_limit)) {
        const int z = split_count(a.z_in, a.n_seg_total, a.n_vs, u.bh, u.s);
        if (a.z_gate && z < 0) return;
        if (a.z_limit && z >= 0 && z < u.nchunks) {
            u.nchunks = z;
            u.cut = true;
        }
    }
    u.HD = (long long)a.H * DK;
    u.base_tok = (long long)u.b * a.T * u.HD + (long long)u.h * DK;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // zero the token-padded operand arrays once (parts never written stay zero)
    {
        KDA_LDS __bf16* sKpT = reinterpret_cast<KDA_LDS __bf16*>(smem + Cfg::oKpT);
        KDA_LDS __bf16* sTA = reinterpret_cast<KDA_LDS __bf16*>(smem + Cfg::oTA);
        KDA_LDS __bf16* sB = reinterpret_cast<KDA_LDS __bf16*>(smem + Cfg::oB);
        for (int e = tid; e < C * PTB; e += NTH) {
            sTA[e] = from_f32<__bf16>(0.0f);
            sB[e] = from_f32<__bf16>(0.0f);
        }
        for (int e = tid; e < DK * PT; e += NTH) sKpT[e] = from_f32<__bf16>(0.0f);
    }
    if (wave < NCW) pipe_chunk_waves<NCW, GATE>(a, u, smem, tid, wave);
    else pipe_state_waves<NCW>(a, u, smem, tid, wave - NCW);
}

template <int NCW, bool GATE>
hipError_t launch_prefill_pipe(const PrefillArgs& a, hipStream_t stream) {
    if (a.n_vs != 1 || a.lens || a.zero_values || (a.gate != nullptr) != GATE) return hipErrorInvalidValue;
    const long long nblk = ((long long)a.n_units + 7) / 8 * 8;
    if (nblk <= 0) return hipSuccess;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((kda_prefill_pipe_kernel<NCW, GATE>), dim3((unsigned)nblk), dim3(64 * (NCW + 4)), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kda
