// Device-side helpers shared by the KDA kernels (gfx950 / CDNA4, wave64).
//
// Matrix-core convention used throughout.  A 16x16 output tile is produced by
// v_mfma_f32_16x16x32_bf16 (bf16 operands) or by eight v_mfma_f32_16x16x4_f32
// (fp32 operands).  In both cases lane l = 16*g + r (g = l / 16, r = l % 16):
//   * A operand (16 x 32, M x K): row r, eight contraction slots;
//   * B operand (32 x 16, K x N): column r, the same eight slots;
//   * accumulator (16 x 16): column r, rows 4g .. 4g+3.
// Slot j of lane group g stands for contraction index kmap(g, j) inside the
// 32-block: 4g + j for j < 4 and 16 + 4g + (j - 4) for j >= 4.  The hardware
// pairs A and B slot by slot, so any bijection works as long as both operands
// use it; this one is chosen because it is exactly how two vertically stacked
// accumulator tiles sit in a lane (rows 4g..4g+3 of tile 0, then of tile 1).
// An accumulator pair therefore becomes a B operand with no data movement.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kda {

// LDS (address space 3) pointers keep shared-memory addressing in 32 bits.
#define KDA_LDS __attribute__((address_space(3)))

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLogAlphaMin = -5.0f;  // bound on log alpha (natural log)

__device__ __forceinline__ int kmap(int g, int j) { return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4); }

// ---------------------------------------------------------------- scalars
template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<__bf16>(__bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- fragments
template <typename OpT> struct Frag;

template <> struct Frag<__bf16> {
    bf16x8_t v;
    __device__ __forceinline__ void set(int j, float x) { v[j] = (__bf16)x; }
    __device__ __forceinline__ float get(int j) const { return (float)v[j]; }
    __device__ __forceinline__ void zero() {
        for (int j = 0; j < 8; ++j) v[j] = (__bf16)0.0f;
    }
};

template <> struct Frag<float> {
    float v[8];
    __device__ __forceinline__ void set(int j, float x) { v[j] = x; }
    __device__ __forceinline__ float get(int j) const { return v[j]; }
    __device__ __forceinline__ void zero() {
        for (int j = 0; j < 8; ++j) v[j] = 0.0f;
    }
};

__device__ __forceinline__ f32x4_t mma(const Frag<__bf16>& a, const Frag<__bf16>& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mma(const Frag<float>& a, const Frag<float>& b, f32x4_t c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
    return c;
}

// The eight slots of one lane from a row-major LDS array, `p` already pointing
// at element kmap(g, 0) of the lane's row: p[0..3] and p[16..19].
__device__ __forceinline__ void frag_ld(Frag<__bf16>& f, const KDA_LDS __bf16* p) {
    const bf16x4_t lo = *reinterpret_cast<const KDA_LDS bf16x4_t*>(p);
    const bf16x4_t hi = *reinterpret_cast<const KDA_LDS bf16x4_t*>(p + 16);
    f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void frag_ld(Frag<float>& f, const KDA_LDS float* p) {
    const f32x4_t lo = *reinterpret_cast<const KDA_LDS f32x4_t*>(p);
    const f32x4_t hi = *reinterpret_cast<const KDA_LDS f32x4_t*>(p + 16);
    f.v[0] = lo[0]; f.v[1] = lo[1]; f.v[2] = lo[2]; f.v[3] = lo[3];
    f.v[4] = hi[0]; f.v[5] = hi[1]; f.v[6] = hi[2]; f.v[7] = hi[3];
}

// The same eight slots from two separate LDS addresses (slots 0..3 at lo, 4..7 at hi): rows whose
// 4-element groups are stored permuted.
__device__ __forceinline__ void frag_ld2(Frag<__bf16>& f, const KDA_LDS __bf16* lo, const KDA_LDS __bf16* hi) {
    const bf16x4_t a = *reinterpret_cast<const KDA_LDS bf16x4_t*>(lo);
    const bf16x4_t b = *reinterpret_cast<const KDA_LDS bf16x4_t*>(hi);
    f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Only the lower four slots from LDS, the upper four zero: a 16-wide contraction block.
__device__ __forceinline__ void frag_ld_lo(Frag<__bf16>& f, const KDA_LDS __bf16* p) {
    const bf16x4_t lo = *reinterpret_cast<const KDA_LDS bf16x4_t*>(p);
    const bf16x4_t z = {(__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f};
    f.v = __builtin_shufflevector(lo, z, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void frag_ld_lo(Frag<float>& f, const KDA_LDS float* p) {
    const f32x4_t lo = *reinterpret_cast<const KDA_LDS f32x4_t*>(p);
    f.v[0] = lo[0]; f.v[1] = lo[1]; f.v[2] = lo[2]; f.v[3] = lo[3];
    f.v[4] = 0.0f; f.v[5] = 0.0f; f.v[6] = 0.0f; f.v[7] = 0.0f;
}

// Eight fp32 factors for the same slots (per-channel decay factors).
__device__ __forceinline__ void f32x8_ld(float out[8], const KDA_LDS float* p) {
    const f32x4_t lo = *reinterpret_cast<const KDA_LDS f32x4_t*>(p);
    const f32x4_t hi = *reinterpret_cast<const KDA_LDS f32x4_t*>(p + 16);
    out[0] = lo[0]; out[1] = lo[1]; out[2] = lo[2]; out[3] = lo[3];
    out[4] = hi[0]; out[5] = hi[1]; out[6] = hi[2]; out[7] = hi[3];
}

// Direct global -> LDS load of 16 bytes per lane: lane i of the wave writes
// bytes [16 i, 16 i + 16) after `lds` (wave-uniform).  Kept out of templates:
// the host compilation pass drops a template kernel's launch stub when the
// builtin appears in its body.
__device__ __forceinline__ void lds_dma16(const float* src, KDA_LDS void* lds) {
    __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// N consecutive elements of one LDS row, stored with as few instructions as
// the alignment (N elements of type T are N * sizeof(T)-byte aligned) allows.
template <int N>
__device__ __forceinline__ void lds_store_run(KDA_LDS __bf16* p, const float (&v)[N]) {
    if constexpr (N == 1) {
        *p = (__bf16)v[0];
    } else {
        typedef __attribute__((ext_vector_type(N))) __bf16 vec_t;
        vec_t x;
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] = (__bf16)v[i];
        *reinterpret_cast<KDA_LDS vec_t*>(p) = x;
    }
}
template <int N>
__device__ __forceinline__ void lds_store_run(KDA_LDS float* p, const float (&v)[N]) {
    if constexpr (N == 1) {
        *p = v[0];
    } else if constexpr (N <= 4) {
        typedef __attribute__((ext_vector_type(N))) float vec_t;
        vec_t x;
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] = v[i];
        *reinterpret_cast<KDA_LDS vec_t*>(p) = x;
    } else {
#pragma unroll
        for (int i = 0; i < N; i += 4)
            *reinterpret_cast<KDA_LDS f32x4_t*>(p + i) = f32x4_t{v[i], v[i + 1], v[i + 2], v[i + 3]};
    }
}

// A lane-dependent value pinned in a register: the compiler may not recompute
// it where it is used (inside the chunk loop that would reintroduce runtime
// multiplies into LDS addressing).
// p advanced by a 32-bit byte offset: with p uniform this is the scalar-base + vector-offset
// address form, one register per lane instead of a 64-bit pointer.
template <typename T> __device__ __forceinline__ T* at_byte(T* p, uint32_t off) {
    return reinterpret_cast<T*>(reinterpret_cast<char*>(p) + off);
}
template <typename T> __device__ __forceinline__ const T* at_byte(const T* p, uint32_t off) {
    return reinterpret_cast<const T*>(reinterpret_cast<const char*>(p) + off);
}

// An opaque copy of a lane offset, taken where the address is formed: keeps the compiler from
// hoisting "uniform base + offset" out of a loop as a 64-bit per-lane pointer.
__device__ __forceinline__ uint32_t pinned_u(uint32_t x) { asm volatile("" : "+v"(x)); return x; }
// An opaque copy of an LDS address: the compiler keeps it in one register and reaches nearby
// elements through the instruction's immediate offset instead of materialising one address
// register per constant offset.
template <typename T> __device__ __forceinline__ KDA_LDS T* lds_pin(KDA_LDS T* p) {
    uint32_t x = (uint32_t)(size_t)p;
    asm volatile("" : "+v"(x));
    return (KDA_LDS T*)(size_t)x;
}
// Value of x in lane I of this lane's 16-lane row (DPP row broadcast).
template <int I> __device__ __forceinline__ float row_bcast(float x) {
    static_assert(I >= 0 && I < 16, "row lane");
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x150 + I, 0xF, 0xF, true));
}
// Marks a register value as redefined at this point: computation that reads it cannot be moved
// above here (a load into it is waited for here, not earlier).
template <typename T> __device__ __forceinline__ void reg_pin(T& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ int pinned(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Two stacked accumulator tiles (rows 0..15 and 16..31 of a 32-block) as a B
// operand.  `has_hi` = false treats the lower tile as zeros.
template <typename OpT>
__device__ __forceinline__ void acc_pair_frag(Frag<OpT>& f, const f32x4_t& lo, const f32x4_t& hi,
                                              bool has_hi) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f.set(j, lo[j]);
        f.set(4 + j, has_hi ? hi[j] : 0.0f);
    }
}

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}; }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations,
// not for its global loads in flight (a __syncthreads() fence would drain those
// too and expose a prefetch's full latency).  The memory clobber keeps the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Workgroup barrier that also waits for this wave's global loads, including
// loads that write LDS directly.
__device__ __forceinline__ void barrier_all() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Chunk count of the sequence split's unit (bh, segment s >= 1) from the counts of a transition
// pass laid out [bh][n_seg_total - 1][n_vs]: the largest over the unit's column slices, -1 if any
// slice's transition never fell below 2^-126.
__device__ __forceinline__ int split_count(const int* z, int n_seg_total, int n_vs, int bh, int s) {
    const int* p = z + ((long long)bh * (n_seg_total - 1) + (s - 1)) * n_vs;
    int m = 0;
    for (int v = 0; v < n_vs; ++v) {
        const int c = p[v];
        if (c < 0) return -1;
        m = c > m ? c : m;
    }
    return m;
}

}  // namespace kda
