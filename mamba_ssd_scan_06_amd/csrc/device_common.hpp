// Device-side building blocks shared by the SSD kernels (gfx950, wave64).
//
// Matrix-core fragments
// ---------------------
// All contractions use the 16x16 output tile of the CDNA matrix cores:
//   D[16x16] += A[16xK] * B[Kx16]
// Lane l of the 64-wide wave feeds row (l % 16) of A and column (l % 16) of B
// and holds 8 values of the contraction index k for them; D comes back as 4
// fp32 per lane: D[4*(l/16) + r][l % 16], r = 0..3.
// Which k a lane's 8 values stand for is free, provided A and B use the same
// assignment: the sum over k does not depend on how k is spread over lanes
// and slots.  The kernels rely on this to feed one MFMA's output tile
// straight into the next MFMA (see chunk_output).
//
// bf16 inputs use v_mfma_f32_16x16x32_bf16 (K = 32 per instruction, fp32
// accumulate).  fp32 inputs use v_mfma_f32_16x16x4_f32 eight times (K = 4
// each, exact fp32 products), so the fp32 path never rounds to a narrower
// type.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

using bf16 = __bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// exp(x) through the hardware base-2 exponential.  Inputs here are <= 0
// (decays); results below the fp32 normal range flush to zero, which is
// below any output's resolution.
__device__ __forceinline__ float exp_neg(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(float v) { return v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
// fp32 -> bf16 rounds to nearest even (v_cvt_pk_bf16_f32 on gfx950).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }

// 8 k-values of one MFMA operand for one lane.
template <typename T> struct Frag;
template <> struct Frag<bf16> {
    bf16x8 v;
    __device__ __forceinline__ void set(int s, float f) { v[s] = (bf16)f; }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int s = 0; s < 8; ++s) v[s] = (bf16)0.0f;
    }
};
template <> struct Frag<float> {
    f32x4 lo, hi;
    __device__ __forceinline__ void set(int s, float f) {
        if (s < 4) lo[s] = f; else hi[s - 4] = f;
    }
    __device__ __forceinline__ void zero() {
        lo = f32x4{0.f, 0.f, 0.f, 0.f};
        hi = lo;
    }
};

__device__ __forceinline__ void mma(const Frag<bf16> &a, const Frag<bf16> &b, f32x4 &acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}

__device__ __forceinline__ void mma(const Frag<float> &a, const Frag<float> &b, f32x4 &acc) {
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[s], b.lo[s], acc, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[s], b.hi[s], acc, 0, 0, 0);
}

// Eight consecutive elements at p (16-byte aligned) as one fragment.
__device__ __forceinline__ void load8(Frag<bf16> &f, const bf16 *p) { f.v = *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ void load8(Frag<float> &f, const float *p) {
    f.lo = *reinterpret_cast<const f32x4 *>(p);
    f.hi = *reinterpret_cast<const f32x4 *>(p + 4);
}

// Two runs of four consecutive elements (8-byte / 16-byte aligned) as slots 0-3 and 4-7.
__device__ __forceinline__ void load4x2(Frag<bf16> &f, const bf16 *p0, const bf16 *p1) {
    bf16x4 a = *reinterpret_cast<const bf16x4 *>(p0);
    bf16x4 b = *reinterpret_cast<const bf16x4 *>(p1);
    f.v = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ void load4x2(Frag<float> &f, const float *p0, const float *p1) {
    f.lo = *reinterpret_cast<const f32x4 *>(p0);
    f.hi = *reinterpret_cast<const f32x4 *>(p1);
}

// Eight consecutive fp32 values (32-byte aligned) converted to a T fragment.
__device__ __forceinline__ void load8_from_f32(Frag<bf16> &f, const float *p) {
    f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        f.v[s] = (bf16)a[s];
        f.v[s + 4] = (bf16)b[s];
    }
}
__device__ __forceinline__ void load8_from_f32(Frag<float> &f, const float *p) {
    f.lo = *reinterpret_cast<const f32x4 *>(p);
    f.hi = *reinterpret_cast<const f32x4 *>(p + 4);
}

// Vector of 8 / 4 elements of T for global <-> register moves.
template <typename T> struct Vec8;
template <> struct Vec8<bf16> { typedef bf16x8 type; };
template <> struct Vec8<float> { typedef float type __attribute__((ext_vector_type(8))); };
template <typename T> struct Vec4;
template <> struct Vec4<bf16> { typedef bf16x4 type; };
template <> struct Vec4<float> { typedef f32x4 type; };

}  // namespace ssd
