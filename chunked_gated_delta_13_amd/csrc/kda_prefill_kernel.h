// Fused chunked KDA prefill kernel for gfx950.
//
// One workgroup of NW wave64s (4 or 8) owns one unit = (sequence b, head h,
// segment s, state-column slice) and walks the unit's chunks of C tokens in
// order, carrying the fp32 state slice S (DK x 16*NCT*NW) in registers, 16*NCT
// columns per wave.  Sources:
// "Kimi K3" (meridianbulletin.com), "Parallelizing Sequential State Updates"
// (the tokens of a chunk are processed in parallel, then the state is handed to
// the next chunk); "Kimi K3's architecture" (orkas.ai), "A lower bound that
// deleted a GPU code path" (with log alpha >= -5, 16 tokens can decay by at
// most e^-80 in total, so the inverse of that decay still fits the 8-bit
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
//   C   T_aa = (I + A_aa)^{-1} for the 16x16 diagonal blocks, by forward substitution
//   D   X = K~ S, P = Q~ S with K~ = Lk 2^{rho_a}, Q~ = Lq 2^{rho_a}
//       U = (I + A)^{-1} (beta (V - X)) by blocked forward substitution:
//           U_a = T_aa (RHS_a - sum_{b<a} A_ab U_b)
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

template <int DK_, int NCT_, int C_, typename TIn_, int NW_ = 4>
struct PrefillCfg {
    static constexpr int DK = DK_;
    static constexpr int NCT = NCT_;             // 16-column tiles per wave
    static constexpr int NW = NW_;               // waves per workgroup
    static constexpr int NTH = 64 * NW_;         // threads per workgroup
    static constexpr int C = C_;
    using TIn = TIn_;
    using OpT = TIn_;                            // matrix-core operand type
    static constexpr int NT = C / 16;            // 16-token row tiles per chunk
    static constexpr int NTB = (NT + 1) / 2;     // 32-token contraction blocks per chunk
    static constexpr int DVW = 16 * NCT * NW;    // state columns per workgroup
    static constexpr int NQ = DK / 4;            // channel quads (decay phase)
    static constexpr int NSEG = NTH / NQ;        // token segments (decay phase)
    static constexpr int TPS = C / NSEG;         // tokens per segment
    static constexpr int G = C / 16;             // tokens per decay group (16 groups per chunk)
    static constexpr int GPT = TPS / G;          // decay groups per segment
    static constexpr int SPT = 16 / G;           // decay groups per 16-token tile
    static constexpr int CP = C < 32 ? 32 : C;   // token extent of token-indexed rows
    static constexpr int PADE = sizeof(OpT) == 2 ? 8 : 4;
    // Row pitches: a bf16 fragment load is two 8-byte reads 32 bytes apart, bank-conflict free
    // on gfx950 at row pitches of 66 or 34 dwords (two-way conflicted at 68 or 36).
    static constexpr int PK = DK + 4;            // pitch of [C][DK] operand arrays
    static constexpr int PT = CP + (sizeof(OpT) == 2 && CP == 64 ? 4 : PADE);   // pitch of sTA, sB, sKpT
    static constexpr int PV = DVW + PADE;        // pitch of sV
    static constexpr int PW = 16 * NCT + PADE;   // pitch of a wave's output staging
    static constexpr int PD = 20;                // pitch of the transposed fp32 diagonal A blocks
    static constexpr int PDB = 16 * PD + 16;     // stride between diagonal blocks (bank offset 16)
    static constexpr int VEL = 16 / (int)sizeof(TIn);           // elements per 16-byte vector
    static constexpr int VPR = DVW / VEL;                       // vectors per value row
    static constexpr int NV = C * VPR;                          // vectors per value chunk
    static constexpr int NVV = (NV + NTH - 1) / NTH;            // vectors per thread
    static constexpr int VPRW = 16 * NCT / VEL;                 // vectors per wave output row
    static constexpr int NOT = 16 * VPRW;                       // vectors per wave output tile
    static constexpr int NOTL = (NOT + 63) / 64;                // per lane
    static constexpr int NDMA = C * DK * 4 / 1024;              // 1 KiB fp32 log-decay loads per chunk
    static constexpr int NQT = C * DK / 4;                      // quads per [C][DK] array

    static_assert(TPS >= 1 && 16 % TPS == 0, "segment must sit inside one tile");
    static_assert(TPS % G == 0, "segment holds whole decay groups");
    static_assert(DK % 32 == 0 && C % 16 == 0 && NT <= 4, "shape");
    static_assert(NTH % VPR == 0, "value rows split evenly over the threads");
    static_assert(NT <= NW, "one wave per diagonal block");

    static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
    static constexpr size_t oLq = 0;
    static constexpr size_t oLk = oLq + al(sizeof(OpT) * C * PK);
    static constexpr size_t oKd = oLk + al(sizeof(OpT) * C * PK);
    static constexpr size_t oKpT = oKd + al(sizeof(OpT) * C * PK);
    static constexpr size_t oV = oKpT + al(sizeof(OpT) * DK * PT);
    static constexpr size_t oTA = oV + al(sizeof(TIn) * C * PV);
    static constexpr size_t oB = oTA + al(sizeof(OpT) * C * PT);
    static constexpr size_t oAd = oB + al(sizeof(OpT) * C * PT);
    static constexpr size_t oE = oAd + al(4 * NT * PDB);
    static constexpr size_t oD = oE + al(4 * (NT + 1) * DK);
    static constexpr size_t oBeta = oD + al(4 * (NT == 4 ? NT + 3 : NT) * DK);   // D rows (+ products)
    static constexpr size_t oTot = oBeta + al(4 * C);
    static constexpr size_t oO = oTot + al(4 * 16 * DK);
    static constexpr size_t oFlag = oO + al(sizeof(TIn) * NW * 16 * PW);   // early-stop flags [2][NW]
    static constexpr size_t LDS = oFlag + al(4 * 2 * NW);
    static_assert(LDS <= 160 * 1024, "LDS budget of one gfx950 workgroup");
};

// Row tile of the pi-th (row, column <= row) tile pair, pairs enumerated row by row.
constexpr int pair_row(int pi) {
    int ar = 0;
    while ((ar + 1) * (ar + 2) / 2 <= pi) ++ar;
    return ar;
}

// Wave that forms the pi-th tile pair.  With 8 waves and 4 row tiles the two pairs beyond the
// eighth go to waves that hold a diagonal (cheaper) pair; wave 0 keeps one pair because it also
// inverts the diagonal blocks.
constexpr int pair_owner(int pi, int nw) {
    if (nw == 8 && pi == 8) return 5;
    if (nw == 8 && pi == 9) return 2;
    return pi % nw;
}

// Four adjacent elements (a channel quad) of an input or operand array.
template <typename T> struct Quad;
template <> struct Quad<__bf16> {
    typedef u32x2_t raw;
    __device__ __forceinline__ static raw load(const __bf16* p) { return *reinterpret_cast<const u32x2_t*>(p); }
    __device__ __forceinline__ static raw zero() { return u32x2_t{0u, 0u}; }
    __device__ __forceinline__ static raw load(const KDA_LDS __bf16* p) { return *reinterpret_cast<const KDA_LDS u32x2_t*>(p); }
    __device__ __forceinline__ static float get(raw r, int i) {
        const uint32_t w = i < 2 ? r[0] : r[1];
        return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
    }
    __device__ __forceinline__ static void store(KDA_LDS __bf16* p, float a, float b, float c, float d) {
        bf16x4_t v;
        v[0] = (__bf16)a; v[1] = (__bf16)b; v[2] = (__bf16)c; v[3] = (__bf16)d;
        *reinterpret_cast<KDA_LDS bf16x4_t*>(p) = v;
    }
    __device__ __forceinline__ static raw pack(float a, float b, float c, float d) {
        bf16x4_t v;
        v[0] = (__bf16)a; v[1] = (__bf16)b; v[2] = (__bf16)c; v[3] = (__bf16)d;
        return __builtin_bit_cast(raw, v);
    }
    __device__ __forceinline__ static void store_raw(KDA_LDS __bf16* p, raw r) {
        *reinterpret_cast<KDA_LDS u32x2_t*>(p) = r;
    }
};
template <> struct Quad<float> {
    typedef f32x4_t raw;
    __device__ __forceinline__ static raw load(const float* p) { return *reinterpret_cast<const f32x4_t*>(p); }
    __device__ __forceinline__ static raw zero() { return f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}; }
    __device__ __forceinline__ static raw load(const KDA_LDS float* p) { return *reinterpret_cast<const KDA_LDS f32x4_t*>(p); }
    __device__ __forceinline__ static float get(raw r, int i) { return r[i]; }
    __device__ __forceinline__ static void store(KDA_LDS float* p, float a, float b, float c, float d) {
        *reinterpret_cast<KDA_LDS f32x4_t*>(p) = f32x4_t{a, b, c, d};
    }
    __device__ __forceinline__ static raw pack(float a, float b, float c, float d) { return f32x4_t{a, b, c, d}; }
    __device__ __forceinline__ static void store_raw(KDA_LDS float* p, raw r) {
        *reinterpret_cast<KDA_LDS f32x4_t*>(p) = r;
    }
};

// DUAL: one pass yields both the transition of each unit (identity columns, zero values, kept in
// `sm`) and its increment (zero start, real values, kept in `st`); the decay and intra-chunk work
// is shared and no output rows are formed.
// GATE: the decay input is the raw gate pre-activation x (bf16) and log alpha = -5 sigmoid(x) is
// formed on load, in place of an fp32 log alpha.
// PROBE: a transition pass that stops once its transition columns have died (every entry below
// 2^-126), stores the transition as zeros and records the chunks it ran (the sequence split's
// short cut); the dual pass always runs this way.
template <class Cfg, bool DUAL, bool GATE, bool PROBE>
__global__ __launch_bounds__(Cfg::NTH) void kda_prefill_kernel(const PrefillArgs a) {
    using TIn = typename Cfg::TIn;
    using OpT = typename Cfg::OpT;
    using QI = Quad<TIn>;
    using QO = Quad<OpT>;
    constexpr int DK = Cfg::DK, C = Cfg::C, NT = Cfg::NT, NTB = Cfg::NTB, NCT = Cfg::NCT;
    constexpr int DVW = Cfg::DVW, NQ = Cfg::NQ, NSEG = Cfg::NSEG, TPS = Cfg::TPS;
    constexpr int SPT = Cfg::SPT, G = Cfg::G, GPT = Cfg::GPT, PK = Cfg::PK, PT = Cfg::PT, PV = Cfg::PV, PW = Cfg::PW;
    constexpr int PD = Cfg::PD, PDB = Cfg::PDB, VEL = Cfg::VEL, VPR = Cfg::VPR, NV = Cfg::NV, NVV = Cfg::NVV;
    constexpr int VPRW = Cfg::VPRW, NOT = Cfg::NOT, NOTL = Cfg::NOTL;
    constexpr int NQT = Cfg::NQT, NW = Cfg::NW, NTH = Cfg::NTH;
    constexpr int NIT = DK / 16;   // 16-row tiles of the state
    constexpr int NKB = DK / 32;   // 32-channel contraction blocks

    __shared__ __align__(16) char smem_[Cfg::LDS];
    KDA_LDS char* smem = (KDA_LDS char*)smem_;
    KDA_LDS OpT* sLq = reinterpret_cast<KDA_LDS OpT*>(smem + Cfg::oLq);     // q 2^{g - rho}, then Q~ = q 2^{g}
    KDA_LDS OpT* sLk = reinterpret_cast<KDA_LDS OpT*>(smem + Cfg::oLk);     // k 2^{g - rho}, then K~ = k 2^{g}
    KDA_LDS OpT* sKd = reinterpret_cast<KDA_LDS OpT*>(smem + Cfg::oKd);     // k 2^{rho - g}
    KDA_LDS OpT* sKpT = reinterpret_cast<KDA_LDS OpT*>(smem + Cfg::oKpT);   // (k 2^{g_C - g})^T
    KDA_LDS TIn* sV = reinterpret_cast<KDA_LDS TIn*>(smem + Cfg::oV);
    KDA_LDS OpT* sTA = reinterpret_cast<KDA_LDS OpT*>(smem + Cfg::oTA);     // diagonal blocks T_aa, below them -beta A
    KDA_LDS OpT* sB = reinterpret_cast<KDA_LDS OpT*>(smem + Cfg::oB);       // decay-weighted Q K^T, inclusive lower
    KDA_LDS float* sAd = reinterpret_cast<KDA_LDS float*>(smem + Cfg::oAd); // beta A of the diagonal blocks, transposed
    KDA_LDS float* sE = reinterpret_cast<KDA_LDS float*>(smem + Cfg::oE);
    KDA_LDS float* sD = reinterpret_cast<KDA_LDS float*>(smem + Cfg::oD);
    KDA_LDS float* sBeta = reinterpret_cast<KDA_LDS float*>(smem + Cfg::oBeta);
    KDA_LDS float* sTot = reinterpret_cast<KDA_LDS float*>(smem + Cfg::oTot);
    KDA_LDS TIn* sO = reinterpret_cast<KDA_LDS TIn*>(smem + Cfg::oO);
    KDA_LDS int* sFlag = reinterpret_cast<KDA_LDS int*>(smem + Cfg::oFlag);

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
    const long long t_begin = (long long)s * a.seg_len + (s > 0 ? a.seg_shift : 0);
    const long long t_next = (long long)(s + 1) * a.seg_len + a.seg_shift;
    long long t_end = t_next < a.T ? t_next : a.T;
    if (a.lens) {   // ragged: this sequence stops after lens[b] tokens
        const long long l = a.lens[b];
        const long long lc = l < 0 ? 0 : (l > a.T ? a.T : l);
        if (t_end > lc) t_end = lc;
    }
    const int col0 = vs * DVW;

    const int tid = threadIdx.x;
    const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, kept in a scalar register

    const long long HD = (long long)a.H * DK;  // token stride of every [B, T, H, d] tensor
    const long long base_tok = (long long)b * a.T * HD + (long long)h * DK;
    const TIn* gq = reinterpret_cast<const TIn*>(a.q) + base_tok;
    const TIn* gk = reinterpret_cast<const TIn*>(a.k) + base_tok;
    constexpr int LAE = GATE ? 2 : 4;                          // bytes per decay-input element
    const char* gla = GATE ? reinterpret_cast<const char*>(a.gate) + base_tok * 2
                           : reinterpret_cast<const char*>(a.log_alpha + base_tok);
    const long long HDL = HD * LAE;                            // token stride of the decay input, bytes
    const TIn* gv = reinterpret_cast<const TIn*>(a.v) + base_tok + col0;
    TIn* go = a.o ? reinterpret_cast<TIn*>(a.o) + base_tok + col0 : nullptr;
    const float* gbeta = a.beta + (long long)b * a.T * a.H + h;
    const bool has_o = !DUAL && go != nullptr;
    const bool zero_v = a.zero_values != 0;

    // ---- initial state: lane holds S[16*it + 4*lg + j][colw(ct)]; in the dual pass column tiles
    //      NCT..2*NCT-1 hold the transition of the same columns ----
    constexpr int NCD = DUAL ? 2 * NCT : NCT;
    f32x4_t st[NIT][NCD];
    if constexpr (DUAL) {
#pragma unroll
        for (int it = 0; it < NIT; ++it)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const int col = col0 + wave * 16 * NCT + ct * 16 + lr;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    st[it][ct][j] = 0.0f;
                    st[it][NCT + ct][j] = (16 * it + 4 * lg + j == col) ? 1.0f : 0.0f;
                }
            }
    } else if (a.init_mode == 1 || (a.init_mode == 3 && s == 0)) {
        const float* sin = a.s_in + (long long)bh * a.sin_bh_stride + (long long)s * a.sin_seg_stride;
#pragma unroll
        for (int it = 0; it < NIT; ++it)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const int col = col0 + wave * 16 * NCT + ct * 16 + lr;
#pragma unroll
                for (int j = 0; j < 4; ++j) st[it][ct][j] = sin[(long long)(16 * it + 4 * lg + j) * DK + col];
            }
    } else {
        const bool ident = a.init_mode == 2;
#pragma unroll
        for (int it = 0; it < NIT; ++it)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const int col = col0 + wave * 16 * NCT + ct * 16 + lr;
#pragma unroll
                for (int j = 0; j < 4; ++j) st[it][ct][j] = (ident && 16 * it + 4 * lg + j == col) ? 1.0f : 0.0f;
            }
    }

    // ---- zero the token-padded operand arrays once (parts never written stay zero) ----
    for (int e = tid; e < C * PT; e += NTH) {
        sTA[e] = from_f32<OpT>(0.0f);
        sB[e] = from_f32<OpT>(0.0f);
    }
    for (int e = tid; e < DK * PT; e += NTH) sKpT[e] = from_f32<OpT>(0.0f);

    // ---- decay-phase thread mapping: channel quad cq, token segment sg ----
    const int cq = tid % NQ;
    const int sg = tid / NQ;
    const int ch0 = 4 * cq;

    // ---- lane-dependent LDS bases, computed once and kept opaque: every access in the chunk loop
    //      is one of these registers plus an immediate offset (arrays grouped so that the
    //      immediates stay below 64 KiB) ----
    constexpr int eLk = (int)((Cfg::oLk - Cfg::oLq) / sizeof(OpT));   // element distances
    constexpr int eKd = (int)((Cfg::oKd - Cfg::oLq) / sizeof(OpT));
    constexpr int eTA = (int)((Cfg::oTA - Cfg::oKpT) / sizeof(OpT));
    constexpr int eB = (int)((Cfg::oB - Cfg::oKpT) / sizeof(OpT));
    constexpr int eBw = (int)((Cfg::oB - Cfg::oTA) / sizeof(OpT));
    constexpr int fD = (int)((Cfg::oD - Cfg::oE) / 4);
    constexpr int fBeta = (int)((Cfg::oBeta - Cfg::oE) / 4);
    static_assert(Cfg::oB + sizeof(OpT) * C * PT - Cfg::oKpT < 65536, "immediate offsets");
    static_assert(Cfg::oKd + sizeof(OpT) * C * PK - Cfg::oLq < 65536, "immediate offsets");
    KDA_LDS OpT* const pA = lds_pin(sLq + sg * TPS * PK + ch0);      // decay-phase rows of Lq, Lk, Kd
    KDA_LDS OpT* const pKp = lds_pin(sKpT + ch0 * PT + sg * TPS);     // this thread's K'^T entries
    KDA_LDS float* const pTotW = lds_pin(sTot + sg * GPT * DK + ch0); // this segment's decay-group totals
    KDA_LDS float* const pTotR = lds_pin(sTot + ch0);                 // all segments' totals
    KDA_LDS float* const pCh = lds_pin(sE + ch0);                     // sE, sD rows of this thread's quad
    KDA_LDS TIn* const pVc = lds_pin(sV + (tid / VPR) * PV + (tid % VPR) * VEL);  // value commit
    KDA_LDS OpT* const pK = lds_pin(sLq + lr * PK + 4 * lg);          // fragment rows of Lq, Lk, Kd
    KDA_LDS OpT* const pT = lds_pin(sKpT + lr * PT + 4 * lg);         // fragment rows of KpT, TA, B
    KDA_LDS float* const pG = lds_pin(sE + 4 * lg);                   // sE, sD, sBeta by accumulator row
    KDA_LDS OpT* const pW = lds_pin(sTA + 4 * lg * PT + lr);          // accumulator element of TA, B
    KDA_LDS float* const pAd = lds_pin(sAd + 4 * lg * PD + lr);       // diagonal-block store, row-major
    // diagonal-block inverse (wave a inverts block a): lane = (column group lane / 16, row lane % 16)
    KDA_LDS float* const pAi = lds_pin(sAd + wave * PDB + (lane & 15) * PD);   // row of A_aa
    KDA_LDS OpT* const pTi = lds_pin(sTA + 16 * wave * (PT + 1) + (lane & 15) * PT + (lane >> 4));
    KDA_LDS TIn* const pV = lds_pin(sV + 4 * lg * PV + wave * 16 * NCT + lr);  // value in accumulator layout
    KDA_LDS TIn* const pOw = lds_pin(sO + wave * 16 * PW + 4 * lg * PW + lr);  // output staging write
    KDA_LDS TIn* const pOr = lds_pin(sO + wave * 16 * PW + (lane / VPRW) * PW + (lane % VPRW) * VEL);
    // byte offset of this lane's output vector from the uniform row base
    const uint32_t boGo = (uint32_t)(((lane / VPRW) * HD + wave * 16 * NCT + (lane % VPRW) * VEL) * sizeof(TIn));

    // ---- per-lane 32-bit byte offsets: inside the loop every global address is a uniform
    //      (scalar) row base plus one of these, so each lane keeps one register per stream ----
    const uint32_t boQK = (uint32_t)(((sg * TPS) * HD + ch0) * sizeof(TIn));
    const uint32_t boB = (uint32_t)((tid % C) * a.H * sizeof(float));
    const int v_row = tid / VPR, v_off = (tid % VPR) * VEL;
    const uint32_t boV = (uint32_t)((v_row * HD + v_off) * sizeof(TIn));
    const uint32_t boLa = (uint32_t)((sg * TPS) * HDL + ch0 * LAE);

    // ---- prefetch of the next chunk into registers: the decay input, q and k in the layout the
    //      decay phase uses (TPS tokens x one channel quad per thread), v and beta ----
    using LaRaw = std::conditional_t<GATE, u32x2_t, f32x4_t>;
    typename QI::raw pq[TPS], pk[TPS];
    LaRaw pla[TPS];
    float pbeta = 0.0f;
    u32x4_t pv[NVV];
    auto clampt = [&](long long t) { return t < t_end ? t : t_end - 1; };

    // Loads only: in a partial last chunk, rows past the end of the unit read the last valid row
    // (in bounds) and are zeroed when the chunk is consumed, so no select waits on a load in
    // flight.  A zero key, value, query, beta and log-decay is an exact identity on the state.
    // q, k and the decay input: consumed by the decay phases A and A'
    auto load_qk = [&](long long c0) {
        if (c0 + C <= t_end) {
#pragma unroll
            for (int i = 0; i < TPS; ++i) {
                pla[i] = *reinterpret_cast<const LaRaw*>(at_byte(gla + (c0 + i) * HDL, pinned_u(boLa)));
                if constexpr (!DUAL) pq[i] = QI::load(at_byte(gq + (c0 + i) * HD, pinned_u(boQK)));
                pk[i] = QI::load(at_byte(gk + (c0 + i) * HD, pinned_u(boQK)));
            }
        } else {
#pragma unroll
            for (int i = 0; i < TPS; ++i) {
                const long long t = clampt(c0 + sg * TPS + i);
                const long long off = t * HD + ch0;
                pla[i] = *reinterpret_cast<const LaRaw*>(gla + t * HDL + ch0 * LAE);
                if constexpr (!DUAL) pq[i] = QI::load(gq + off);
                pk[i] = QI::load(gk + off);
            }
            // rows past the end act as zero queries and keys (their decay is masked in phase A);
            // this path runs at most once per unit, so the wait these selects imply costs nothing
#pragma unroll
            for (int i = 0; i < TPS; ++i)
                if (c0 + sg * TPS + i >= t_end) {
                    if constexpr (!DUAL) pq[i] = QI::zero();
                    pk[i] = QI::zero();
                }
        }
    };
    // v and beta: consumed when phase A commits them to LDS
    auto load_vb = [&](long long c0) {
        if (c0 + C <= t_end) {
            pbeta = *at_byte(gbeta + c0 * a.H, pinned_u(boB));
            // values are fetched even when a pass ignores them: a conditional load would make the
            // compiler wait for it where the two paths merge
#pragma unroll
            for (int m = 0; m < NVV; ++m)
                if (NV % NTH == 0 || tid + NTH * m < NV)
                    pv[m] = *reinterpret_cast<const u32x4_t*>(at_byte(gv + (c0 + m * (NTH / VPR)) * HD, pinned_u(boV)));
        } else {
            pbeta = gbeta[clampt(c0 + (tid % C)) * a.H];
#pragma unroll
            for (int m = 0; m < NVV; ++m)
                if (NV % NTH == 0 || tid + NTH * m < NV)
                    pv[m] = *reinterpret_cast<const u32x4_t*>(gv + clampt(c0 + v_row + m * (NTH / VPR)) * HD + v_off);
        }
    };

    const long long ntok = t_end - t_begin;
    int nchunks = ntok > 0 ? (int)((ntok + C - 1) / C) : 0;
    // sequence split: skip a unit whose increment the transition pass already formed, or run only
    // the chunks over which the entry state still matters (unit-uniform, before any barrier)
    bool cut = false;
    if (s > 0 && (a.z_gate || a.z_limit)) {
        const int z = split_count(a.z_in, a.n_seg_total, a.n_vs, bh, s);
        if (a.z_gate && z < 0) return;
        if (a.z_limit && z >= 0 && z < nchunks) {
            nchunks = z;
            cut = true;
        }
    }
    if (nchunks > 0) {
        load_qk(t_begin);
        load_vb(t_begin);
    }
    int died_at = -1;   // transition pass with early stop: chunks run before the transition died

    for (int c = 0; c < nchunks; ++c) {
        const long long c0 = t_begin + (long long)c * C;
        barrier_all();  // every wave's log-decay block has landed; the previous chunk's LDS reads are done
        if (PROBE && c > 0) {   // every wave reads the same flags: a workgroup-uniform decision
            bool alive = false;
#pragma unroll
            for (int w = 0; w < NW; ++w) alive |= sFlag[((c - 1) & 1) * NW + w] != 0;
            if (!alive) {
                died_at = c;
                break;
            }
        }

        // ================= A: commit prefetched values, per-segment cumulative decay =================
#pragma unroll
        for (int m = 0; m < NVV; ++m) {
            const int e = tid + NTH * m;
            if (NV % NTH == 0 || e < NV) {
                const bool ok = !zero_v && c0 + e / VPR < t_end;
                const u32x4_t x = pv[m];
                *reinterpret_cast<KDA_LDS u32x4_t*>(pVc + m * (NTH / VPR) * PV) =
                    u32x4_t{ok ? x[0] : 0u, ok ? x[1] : 0u, ok ? x[2] : 0u, ok ? x[3] : 0u};
            }
        }
        if (tid < C) sBeta[tid] = (c0 + tid < t_end) ? pbeta : 0.0f;

        bool okt[TPS];
#pragma unroll
        for (int i = 0; i < TPS; ++i) okt[i] = c0 + sg * TPS + i < t_end;
        // log2-decay summed from the start of the token's decay group (G tokens); group totals to LDS
        float g[TPS][4];
        {
            float run[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int i = 0; i < TPS; ++i) {
                f32x4_t l4;
                if constexpr (GATE) {
                    // log alpha = -5 sigmoid(x) = -5 / (1 + 2^{-x log2 e})
                    const u32x2_t xr = pla[i];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const uint32_t w = u < 2 ? xr[0] : xr[1];
                        const float x = __uint_as_float((u & 1) ? (w & 0xffff0000u) : (w << 16));
                        l4[u] = kLogAlphaMin * __builtin_amdgcn_rcpf(1.0f + fast_exp2(-x * kLog2e));
                    }
                } else {
                    l4 = pla[i];
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    // clamp to [-5, 0] (rows past the end add nothing), then accumulate the
                    // log2-decay in one rounding per token
                    const float l = okt[i] ? __builtin_amdgcn_fmed3f(l4[u], kLogAlphaMin, 0.0f) : 0.0f;
                    run[u] = (i % G == 0) ? l * kLog2e : fmaf(l, kLog2e, run[u]);
                    g[i][u] = run[u];
                }
                if (i % G == G - 1)
                    *reinterpret_cast<KDA_LDS f32x4_t*>(pTotW + (i / G) * DK) = f32x4_t{run[0], run[1], run[2], run[3]};
            }
        }
        barrier_lds();

        // ================= A': references and decay-scaled operands =================
        typename QO::raw qtr[TPS], ktr[TPS];   // Q~, K~ of this thread's rows, stored after phase B
        {
            // One summation order for every thread layout: group totals in order inside each
            // 16-token tile, tile totals in order across the chunk.  Rt[a] = rho_a.
            f32x4_t Rt[NT + 1];
            Rt[0] = zero4();
#pragma unroll
            for (int a2 = 0; a2 < NT; ++a2) {
                f32x4_t tt = *reinterpret_cast<const KDA_LDS f32x4_t*>(pTotR + a2 * SPT * DK);
#pragma unroll
                for (int j = 1; j < SPT; ++j) tt = tt + *reinterpret_cast<const KDA_LDS f32x4_t*>(pTotR + (a2 * SPT + j) * DK);
                Rt[a2 + 1] = Rt[a2] + tt;
            }
            const int at = (sg * TPS) / 16;       // this segment's row tile
            const int jg0 = (sg * GPT) % SPT;     // its first decay group inside the tile
            // gp[m] = sum of the tile's group totals before own group m, in the same order as above
            f32x4_t gp[GPT];
            {
                const KDA_LDS float* tb = pTotR + at * SPT * DK;
                f32x4_t run = zero4();
#pragma unroll
                for (int j = 0; j < SPT; ++j) {
#pragma unroll
                    for (int m = 0; m < GPT; ++m)
                        if (j == jg0 + m) gp[m] = run;
                    if (j + 1 < SPT) run = run + *reinterpret_cast<const KDA_LDS f32x4_t*>(tb + j * DK);
                }
            }
            f32x4_t rho = Rt[0], nx = Rt[1];
#pragma unroll
            for (int a2 = 1; a2 < NT; ++a2)
                if (at == a2) {
                    rho = Rt[a2];
                    nx = Rt[a2 + 1];
                }
            const f32x4_t gC = Rt[NT];
            float fd[4], fc[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                fd[u] = fast_exp2(nx[u] - rho[u]);   // 2^{rho_{a+1} - rho_a} in [2^-115.4, 1]
                fc[u] = fast_exp2(gC[u] - nx[u]);    // 2^{g_C - rho_{a+1}} in (0, 1]
            }
            // tables 2^{rho_a} (a <= NT) and 2^{rho_{a+1} - rho_a}: row a is formed by the segment
            // sg = a * TSTEP, so the exponentials are spread over several waves
            {
                constexpr int TSTEP = NSEG / (NT + 1) > 0 ? NSEG / (NT + 1) : 1;
                static_assert(NSEG >= NT + 1, "one segment per table row");
                if (sg % TSTEP == 0 && sg / TSTEP <= NT) {
                    const int t2 = sg / TSTEP;
                    f32x4_t r0 = Rt[0], r1 = Rt[NT >= 1 ? 1 : 0];
#pragma unroll
                    for (int a2 = 1; a2 <= NT; ++a2)
                        if (t2 == a2) {
                            r0 = Rt[a2];
                            r1 = Rt[a2 < NT ? a2 + 1 : a2];
                        }
                    f32x4_t e4, d4;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        e4[u] = fast_exp2(r0[u]);
                        d4[u] = fast_exp2(r1[u] - r0[u]);
                    }
                    *reinterpret_cast<KDA_LDS f32x4_t*>(pCh + t2 * DK) = e4;
                    if (t2 < NT) *reinterpret_cast<KDA_LDS f32x4_t*>(pCh + fD + t2 * DK) = d4;
                    if constexpr (NT == 4) {
                        // after the D rows: D_0 D_1, D_1 D_2 and (D_0 D_1) D_2, which scale the
                        // tile pairs two and three tiles below the diagonal
                        if (t2 == NT) {
                            f32x4_t p01, p12, p012;
#pragma unroll
                            for (int u = 0; u < 4; ++u) {
                                const float d0 = fast_exp2(Rt[1][u] - Rt[0][u]);
                                const float d1 = fast_exp2(Rt[2][u] - Rt[1][u]);
                                const float d2 = fast_exp2(Rt[3][u] - Rt[2][u]);
                                p01[u] = d0 * d1;
                                p12[u] = d1 * d2;
                                p012[u] = p01[u] * d2;
                            }
                            *reinterpret_cast<KDA_LDS f32x4_t*>(pCh + fD + NT * DK) = p01;
                            *reinterpret_cast<KDA_LDS f32x4_t*>(pCh + fD + (NT + 1) * DK) = p12;
                            *reinterpret_cast<KDA_LDS f32x4_t*>(pCh + fD + (NT + 2) * DK) = p012;
                        }
                    }
                }
            }
            float kp[4][TPS];   // K' of this thread's channels, by channel: one vector store each
            float er[4];        // 2^{rho_a} of this thread's channels (<= 1)
#pragma unroll
            for (int u = 0; u < 4; ++u) er[u] = fast_exp2(rho[u]);
#pragma unroll
            for (int i = 0; i < TPS; ++i) {
                float lq[4], lk[4], kd[4], qt[4], kt[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float loc = gp[i / G][u] + g[i][u];   // g - rho_a, in [-115.4, 0]
                    const float x = fast_exp2(loc);              // <= 1
                    const float y = fast_exp2(-loc);             // >= 1, at most 2^115.4 = e^80
                    const float kv = QI::get(pk[i], u);
                    if constexpr (!DUAL) {
                        const float qv = QI::get(pq[i], u);
                        lq[u] = qv * x;
                        qt[u] = lq[u] * er[u];                  // q 2^{g}: 2^{g - rho_a} 2^{rho_a}
                    }
                    lk[u] = kv * x;
                    kt[u] = lk[u] * er[u];
                    kd[u] = kv * y;
                    // K' = k 2^{g_C - g}: the factor above 1 meets only a factor that cannot underflow
                    kp[u][i] = (kd[u] * fd[u]) * fc[u];
                }
                if constexpr (!DUAL) QO::store(pA + i * PK, lq[0], lq[1], lq[2], lq[3]);
                QO::store(pA + eLk + i * PK, lk[0], lk[1], lk[2], lk[3]);
                QO::store(pA + eKd + i * PK, kd[0], kd[1], kd[2], kd[3]);
                // K~ = k 2^{g}, Q~ = q 2^{g}: kept in registers and written over Lk, Lq once the
                // tile pairs have read those
                if constexpr (!DUAL) qtr[i] = QO::pack(qt[0], qt[1], qt[2], qt[3]);
                ktr[i] = QO::pack(kt[0], kt[1], kt[2], kt[3]);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) lds_store_run<TPS>(pKp + u * PT, kp[u]);
        }
        // this chunk's q, k and decay input are consumed: fetch the next chunk's
        if (c + 1 < nchunks) load_qk(c0 + C);
        barrier_lds();

        // ================= B: decay-weighted KK^T and QK^T tiles =================
        {
            constexpr int NP = NT * (NT + 1) / 2;
            static_for<0, NP>([&](auto PIc) {
                constexpr int pi = decltype(PIc)::value;
                constexpr int ar = pair_row(pi);
                constexpr int ac = pi - ar * (ar + 1) / 2;
                if (pair_owner(pi, NW) != wave) return;   // wave-uniform
                f32x4_t accA = zero4(), accB = zero4();
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    Frag<OpT> fk, fq, fr;
                    frag_ld(fk, pK + eLk + 16 * ar * PK + 32 * kb);
                    if constexpr (!DUAL) frag_ld(fq, pK + 16 * ar * PK + 32 * kb);
                    frag_ld(fr, pK + eKd + 16 * ac * PK + 32 * kb);
                    if constexpr (ac < ar) {
                        // R = Kd 2^{rho_ar - rho_ac}: one multiply by D_ac = 2^{rho_{ac+1} - rho_ac}
                        // or, two or three tiles below the diagonal, by the product row
                        // D_ac ... D_{ar-1} (formed left to right).  Where that product underflows,
                        // the exact R is below 2^{115.4 - 149}: far under the operands' bf16 step.
                        static_assert(ar - ac == 1 || NT == 4, "product rows exist for four row tiles");
                        constexpr int prow = (ar - ac == 1) ? ac : (ar - ac == 2 ? NT + ac : NT + 2);
                        float val[8], d8[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j) val[j] = fr.get(j);
                        f32x8_ld(d8, pG + fD + prow * DK + 32 * kb);
#pragma unroll
                        for (int j = 0; j < 8; ++j) val[j] *= d8[j];
#pragma unroll
                        for (int j = 0; j < 8; ++j) fr.set(j, val[j]);
                    }
                    accA = mma(fk, fr, accA);
                    if constexpr (!DUAL) accB = mma(fq, fr, accB);
                }
                const f32x4_t bt4 = *reinterpret_cast<const KDA_LDS f32x4_t*>(pG + fBeta + 16 * ar);
                if constexpr (ac == ar) {
                    f32x4_t ad;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int rl = 4 * lg + j;
                        ad[j] = (lr < rl) ? accA[j] * bt4[j] : 0.0f;
                        if constexpr (!DUAL) pW[eBw + 16 * ar * PT + 16 * ac + j * PT] = from_f32<OpT>((lr <= rl) ? accB[j] : 0.0f);
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j) pAd[ar * PDB + j * PD] = ad[j];
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        pW[16 * ar * PT + 16 * ac + j * PT] = from_f32<OpT>(-accA[j] * bt4[j]);
                        if constexpr (!DUAL) pW[eBw + 16 * ar * PT + 16 * ac + j * PT] = from_f32<OpT>(accB[j]);
                    }
                }
            });
        }
        barrier_lds();

        // v and beta of this chunk were committed in phase A: fetch the next chunk's (issued here so
        // that the workgroup's loads do not all queue at the same point of the chunk)
        if (c + 1 < nchunks) load_vb(c0 + C);

        // ====== C: K~, Q~ over Lk, Lq; diagonal blocks T_aa = (I + A_aa)^{-1} ======
#pragma unroll
        for (int i = 0; i < TPS; ++i) {
            if constexpr (!DUAL) QO::store_raw(pA + i * PK, qtr[i]);
            QO::store_raw(pA + eLk + i * PK, ktr[i]);
        }
        if (wave < NT) {
            // wave a inverts diagonal block a by right-looking forward substitution: lane (cgp, p)
            // holds rows p of columns j = cgp + 4 r of T_aa; the pivot row i of each column is
            // broadcast inside the 16-lane row by DPP, so no step waits on LDS
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
        barrier_lds();

        // ================= D: state-dependent products =================
        Frag<OpT> fs[NKB][NCD];   // S as B operand
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int ct = 0; ct < NCD; ++ct) acc_pair_frag(fs[kb][ct], st[2 * kb][ct], st[2 * kb + 1][ct], true);

        // X = K~ S, then RHS = beta (V - X)
        f32x4_t Rh[NT][NCD];
#pragma unroll
        for (int ar = 0; ar < NT; ++ar) {
#pragma unroll
            for (int ct = 0; ct < NCD; ++ct) Rh[ar][ct] = zero4();
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                Frag<OpT> fk;
                frag_ld(fk, pK + eLk + 16 * ar * PK + 32 * kb);
#pragma unroll
                for (int ct = 0; ct < NCD; ++ct) Rh[ar][ct] = mma(fk, fs[kb][ct], Rh[ar][ct]);
            }
            const f32x4_t bt4 = *reinterpret_cast<const KDA_LDS f32x4_t*>(pG + fBeta + 16 * ar);
#pragma unroll
            for (int ct = 0; ct < NCD; ++ct) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float vv = (zero_v || ct >= NCT) ? 0.0f : to_f32<TIn>(pV[(16 * ar + j) * PV + ct * 16]);
                    Rh[ar][ct][j] = bt4[j] * (vv - Rh[ar][ct][j]);
                }
            }
        }

        // U by blocked forward substitution: U_a = T_aa (RHS_a - sum_{b<a} A_ab U_b)
        f32x4_t U[NT][NCD];
        Frag<OpT> fU[NTB][NCD];
#pragma unroll
        for (int ar = 0; ar < NT; ++ar) {
            f32x4_t W[NCD];
#pragma unroll
            for (int ct = 0; ct < NCD; ++ct) W[ct] = Rh[ar][ct];
#pragma unroll
            for (int kb = 0; kb < ar / 2; ++kb) {
                Frag<OpT> fa;
                frag_ld(fa, pT + eTA + 16 * ar * PT + 32 * kb);
#pragma unroll
                for (int ct = 0; ct < NCD; ++ct) W[ct] = mma(fa, fU[kb][ct], W[ct]);
            }
            if (ar & 1) {
                Frag<OpT> fa;
                frag_ld_lo(fa, pT + eTA + 16 * ar * PT + 16 * (ar - 1));
#pragma unroll
                for (int ct = 0; ct < NCD; ++ct) {
                    Frag<OpT> fb;
                    acc_pair_frag(fb, U[ar - 1][ct], U[ar - 1][ct], false);
                    W[ct] = mma(fa, fb, W[ct]);
                }
            }
            Frag<OpT> ft;
            frag_ld_lo(ft, pT + eTA + 16 * ar * PT + 16 * ar);
#pragma unroll
            for (int ct = 0; ct < NCD; ++ct) {
                Frag<OpT> fw;
                acc_pair_frag(fw, W[ct], W[ct], false);
                U[ar][ct] = mma(ft, fw, zero4());
            }
            if (ar & 1) {
#pragma unroll
                for (int ct = 0; ct < NCD; ++ct) acc_pair_frag(fU[ar / 2][ct], U[ar - 1][ct], U[ar][ct], true);
            } else if (ar == NT - 1) {
#pragma unroll
                for (int ct = 0; ct < NCD; ++ct) acc_pair_frag(fU[ar / 2][ct], U[ar][ct], U[ar][ct], false);
            }
        }

        // O = Q~ S + Bqk U, one 16-row tile at a time through this wave's own LDS rows
        if (has_o) {
#pragma unroll
            for (int ar = 0; ar < NT; ++ar) {
                f32x4_t O[NCT];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) O[ct] = zero4();
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    Frag<OpT> fq;
                    frag_ld(fq, pK + 16 * ar * PK + 32 * kb);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) O[ct] = mma(fq, fs[kb][ct], O[ct]);
                }
#pragma unroll
                for (int kb = 0; kb <= ar / 2; ++kb) {
                    Frag<OpT> fb;
                    frag_ld(fb, pT + eB + 16 * ar * PT + 32 * kb);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) O[ct] = mma(fb, fU[kb][ct], O[ct]);
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int j = 0; j < 4; ++j) pOw[j * PW + ct * 16] = from_f32<TIn>(O[ct][j]);
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                for (int m = 0; m < NOTL; ++m) {
                    const int e = lane + 64 * m;
                    if (NOT % 64 == 0 || e < NOT) {
                        const int row = e / VPRW;
                        const u32x4_t x = *reinterpret_cast<const KDA_LDS u32x4_t*>(pOr + m * (64 / VPRW) * PW);
                        if (c0 + 16 * ar + row < t_end)
                            *reinterpret_cast<u32x4_t*>(at_byte(go + (c0 + 16 * ar + m * (64 / VPRW)) * HD, pinned_u(boGo))) = x;
                    }
                }
            }
        }

        // S <- Diag(2^{g_C}) S + K'^T U
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const f32x4_t gam = *reinterpret_cast<const KDA_LDS f32x4_t*>(pG + NT * DK + 16 * it);
#pragma unroll
            for (int ct = 0; ct < NCD; ++ct)
#pragma unroll
                for (int j = 0; j < 4; ++j) st[it][ct][j] *= gam[j];
#pragma unroll
            for (int kb = 0; kb < NTB; ++kb) {
                Frag<OpT> fkp;
                frag_ld(fkp, pT + 16 * it * PT + 32 * kb);
#pragma unroll
                for (int ct = 0; ct < NCD; ++ct) st[it][ct] = mma(fkp, fU[kb][ct], st[it][ct]);
            }
        }

        // early stop: does any transition entry of this wave still hold a normal float (exponent
        // field not zero)?  Read at the top of the next chunk, after its barrier; the buffers
        // alternate by chunk parity, so a flag is not overwritten before every wave has read it.
        if constexpr (PROBE) {
            constexpr int T0 = DUAL ? NCT : 0;
            uint32_t ex = 0;
#pragma unroll
            for (int it = 0; it < NIT; ++it)
#pragma unroll
                for (int ct = T0; ct < T0 + NCT; ++ct)
#pragma unroll
                    for (int j = 0; j < 4; ++j) ex |= __float_as_uint(st[it][ct][j]) & 0x7f800000u;
            const bool wave_alive = __ballot(ex != 0) != 0;
            if (lane == 0) sFlag[(c & 1) * NW + wave] = wave_alive ? 1 : 0;
        }

        // checkpoint: the state after a multiple of ckpt_every tokens (full chunks only)
        if constexpr (!DUAL) {
            if (a.s_ckpt) {
                const long long pend = c0 + C;
                if (pend <= t_end && pend % a.ckpt_every == 0) {
                    const long long ci = pend / a.ckpt_every - 1;
                    float* sc = a.s_ckpt + (((long long)b * a.n_ckpt + ci) * a.H + h) * (long long)(DK * DK);
#pragma unroll
                    for (int it = 0; it < NIT; ++it)
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct) {
                            const int col = col0 + wave * 16 * NCT + ct * 16 + lr;
#pragma unroll
                            for (int j = 0; j < 4; ++j) sc[(long long)(16 * it + 4 * lg + j) * DK + col] = st[it][ct][j];
                        }
                }
            }
        }
    }

    // ---- final state ----
    const bool died = PROBE && died_at >= 0;
    if (PROBE && tid == 0)
        a.z_out[((long long)bh * (a.n_seg_total - 1) + (s - 1)) * a.n_vs + vs] = died ? died_at : -1;
    // destination: s_out (when this segment's state is wanted), s_head for segment 0, s_tail for
    // the last segment; a cut unit has no final state of its own, except the last segment, whose
    // final state is then its increment, copied from s_tail
    float* so = (a.s_out && (a.out_seg < 0 || a.out_seg == s))
                    ? a.s_out + (long long)bh * a.sout_bh_stride + (long long)s * a.sout_seg_stride
                    : nullptr;
    const float* from = nullptr;
    if (s == 0 && a.s_head) so = a.s_head + (long long)bh * a.shead_bh_stride;
    if (s == a.tail_seg) {
        float* tail = a.s_tail ? a.s_tail + (long long)bh * a.stail_bh_stride : nullptr;
        if (!a.z_limit) so = tail;
        else if (cut) from = tail;
    }
    if (cut && !from) so = nullptr;
    // element (it, j) of column tile ct of this lane
    auto elem = [&](int it, int ct, int j) {
        return (long long)(16 * it + 4 * lg + j) * DK + col0 + wave * 16 * NCT + ct * 16 + lr;
    };
    if constexpr (DUAL) {
        // the transition (none is kept for the last segment); a transition that died is stored as
        // zeros, and the unit's increment is then formed by the zero-start pass instead
        if (s != a.tail_seg) {
            float* sx = a.s_aux + (long long)bh * a.saux_bh_stride + (long long)s * a.saux_seg_stride;
#pragma unroll
            for (int it = 0; it < NIT; ++it)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int j = 0; j < 4; ++j) sx[elem(it, ct, j)] = died ? 0.0f : st[it][NCT + ct][j];
        }
        if (died) so = nullptr;
    } else if (died) {
        if (so) {   // a transition pass: its transition is stored as zeros
#pragma unroll
            for (int it = 0; it < NIT; ++it)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int j = 0; j < 4; ++j) so[elem(it, ct, j)] = 0.0f;
        }
        so = nullptr;
    }
    if (so && from) {
#pragma unroll
        for (int it = 0; it < NIT; ++it)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int j = 0; j < 4; ++j) so[elem(it, ct, j)] = from[elem(it, ct, j)];
    } else if (so) {
#pragma unroll
        for (int it = 0; it < NIT; ++it)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int j = 0; j < 4; ++j) so[elem(it, ct, j)] = st[it][ct][j];
    }
}

// The dual pass always stops early (PROBE); a plain pass stops early when a.probe is set, which
// only the split's transition pass of 4-wave shapes asks for.
template <class Cfg, bool DUAL = false, bool GATE = false>
hipError_t launch_prefill_cfg(const PrefillArgs& a, hipStream_t stream) {
    const long long groups = ((long long)a.n_units + 7) / 8;
    const long long nblk = groups * 8 * a.n_vs;
    if (nblk <= 0) return hipSuccess;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
    if (a.probe && (!a.z_out || a.seg0 < 1)) return hipErrorInvalidValue;
    if constexpr (DUAL) {
        if (!a.probe) return hipErrorInvalidValue;
        hipLaunchKernelGGL((kda_prefill_kernel<Cfg, true, GATE, true>), dim3((unsigned)nblk), dim3(Cfg::NTH), 0, stream, a);
    } else if (!a.probe) {
        hipLaunchKernelGGL((kda_prefill_kernel<Cfg, false, GATE, false>), dim3((unsigned)nblk), dim3(Cfg::NTH), 0, stream, a);
    } else {
        if constexpr (Cfg::NW == 4)
            hipLaunchKernelGGL((kda_prefill_kernel<Cfg, false, GATE, true>), dim3((unsigned)nblk), dim3(Cfg::NTH), 0, stream, a);
        else
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kda
