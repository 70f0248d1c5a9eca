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

namespace kda {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

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

// Load the eight slots of one row of a row-major LDS array: elements
// p[kmap(g, 0..3)] and p[kmap(g, 4..7)] relative to the 32-block start.
__device__ __forceinline__ void lds_row_frag(Frag<__bf16>& f, const __bf16* blk, int g) {
    const bf16x4_t lo = *reinterpret_cast<const bf16x4_t*>(blk + 4 * g);
    const bf16x4_t hi = *reinterpret_cast<const bf16x4_t*>(blk + 16 + 4 * g);
    f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ void lds_row_frag(Frag<float>& f, const float* blk, int g) {
    const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(blk + 4 * g);
    const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(blk + 16 + 4 * g);
    f.v[0] = lo[0]; f.v[1] = lo[1]; f.v[2] = lo[2]; f.v[3] = lo[3];
    f.v[4] = hi[0]; f.v[5] = hi[1]; f.v[6] = hi[2]; f.v[7] = hi[3];
}

// Eight fp32 factors for the same slots (used for per-channel decay factors).
__device__ __forceinline__ void lds_row_f32x8(float out[8], const float* blk, int g) {
    const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(blk + 4 * g);
    const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(blk + 16 + 4 * g);
    out[0] = lo[0]; out[1] = lo[1]; out[2] = lo[2]; out[3] = lo[3];
    out[4] = hi[0]; out[5] = hi[1]; out[6] = hi[2]; out[7] = hi[3];
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

// Two adjacent input elements (a channel pair) as fp32.
template <typename T> struct Pair;
template <> struct Pair<__bf16> {
    typedef uint32_t raw;
    __device__ __forceinline__ static raw load(const __bf16* p) { return *reinterpret_cast<const uint32_t*>(p); }
    __device__ __forceinline__ static float lo(raw r) { return __uint_as_float(r << 16); }
    __device__ __forceinline__ static float hi(raw r) { return __uint_as_float(r & 0xffff0000u); }
    __device__ __forceinline__ static raw zero() { return 0u; }
};
template <> struct Pair<float> {
    typedef float2 raw;
    __device__ __forceinline__ static raw load(const float* p) { return *reinterpret_cast<const float2*>(p); }
    __device__ __forceinline__ static float lo(raw r) { return r.x; }
    __device__ __forceinline__ static float hi(raw r) { return r.y; }
    __device__ __forceinline__ static raw zero() { return make_float2(0.0f, 0.0f); }
};

// Store two values as an adjacent pair of OpT in LDS.
__device__ __forceinline__ void st_pair(__bf16* p, float a, float b) {
    bf16x2_t v;
    v[0] = (__bf16)a;
    v[1] = (__bf16)b;
    *reinterpret_cast<bf16x2_t*>(p) = v;
}
__device__ __forceinline__ void st_pair(float* p, float a, float b) {
    *reinterpret_cast<float2*>(p) = make_float2(a, b);
}

}  // namespace kda
