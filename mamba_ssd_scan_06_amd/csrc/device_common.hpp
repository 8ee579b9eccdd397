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

#include <algorithm>
#include <type_traits>
#include <utility>

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
// 2^x through the same hardware instruction (no range reduction: results
// below the fp32 normal range flush to zero).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

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

// Fragment of an operand held in LDS with the contraction index k as the
// row and the fragment's own index m contiguous ("[k][m]", row stride ld
// elements).  Lane (m = col0 + lane%16, group g = lane/16) receives slots
// 0..3 = rows k0+4g .. k0+4g+3 and slots 4..7 = rows k1+4g .. k1+4g+3 of
// column m.
// bf16 uses gfx950's ds_read_b64_tr_b16: within each 16-lane group, lane i
// receives element i%4 of the 8-byte loads of lanes 4k + i/4 (k = 0..3), so
// source lane s points at row (k + s/4), columns col0 + 4*(s%4) .. +3, and
// lane i ends up with column col0 + i of those four rows.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i16x4 ds_read_tr16(const bf16 *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4 *)(const_cast<bf16 *>(p)));
}
__device__ __forceinline__ void load_tr(Frag<bf16> &f, const bf16 *base, int ld, int k0, int k1, int col0) {
    const int lane = threadIdx.x & 63, s = lane & 15, g = lane >> 4;
    const int off = (4 * g + (s >> 2)) * ld + col0 + 4 * (s & 3);
    const i16x4 a = ds_read_tr16(base + k0 * ld + off);
    const i16x4 b = ds_read_tr16(base + k1 * ld + off);
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 v = i16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    f.v = __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ void load_tr(Frag<float> &f, const float *base, int ld, int k0, int k1, int col0) {
    const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        f.lo[r] = base[(k0 + 4 * g + r) * ld + col0 + i];
        f.hi[r] = base[(k1 + 4 * g + r) * ld + col0 + i];
    }
}

// Direct global -> LDS copies (gfx950 global_load_lds_dwordx4): every lane
// of a wave copies 16 bytes from its own global address to
// lds_wave_base + 16 * lane; lds_wave_base must be the same for the whole
// wave.  Completion is tracked by vmcnt like any load; the kernels wait with
// explicit s_waitcnt immediates and synchronise with a bare s_barrier, since
// __syncthreads() would also wait for every copy still in flight.
__device__ __forceinline__ void copy16_to_lds(const void *gsrc, void *lds_wave_base) {
    __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void *)lds_wave_base, 16, 0, 0);
}
// The wait is the s_waitcnt builtin (gfx9 immediate: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4, lgkmcnt 11:8), which the compiler's own wait insertion
// takes into account; the barriers are asm with a memory clobber so that no
// memory access is moved across them.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }
// Barrier after this wave's LDS stores have completed (its other loads may
// still be in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// XOR swizzles of unpadded LDS tiles whose rows are W 16-byte pieces; the
// copying lane of LDS piece `pos` of row r fetches global piece pos ^ swz(r).
// Swizzle of a row of W 16-byte pieces read 16 bytes per lane down 16 rows.
template <int W>
__device__ __forceinline__ int swz_rows16(int r) {
    if constexpr (W >= 16) return r & 15;
    else return (r / (16 / W)) & (W - 1);
}
// Swizzle of a row of W pieces read through the transposing read (per 16 lanes:
// 4 rows, 2 adjacent pieces).
template <int W>
__device__ __forceinline__ int swz_tr(int r) {
    if constexpr (W >= 16) return 2 * (r & 7);
    else if constexpr (W == 8) return 2 * ((r >> 1) & 3);
    else if constexpr (W == 4) return 2 * ((r >> 2) & 1);
    else return 0;
}

// Data handed from one workgroup to another that may run on a different
// XCD.  Each XCD has its own L2, and for ordinary device memory the L2s are
// not kept coherent with each other, so these accesses carry the device-scope
// cache-policy bit (sc1): loads read from the memory side instead of a
// possibly stale line of this XCD's L2, stores write through to it.  A store
// counts as complete (vmcnt) once it is visible device-wide, so a wave that
// waits for its stores and then stores a flag with device scope publishes the
// data before the flag; a reader polls the flag with device scope and only
// then issues its loads.
constexpr int kScDevice = 16;  // cache-policy operand of the buffer builtins: sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
    // Raw buffer (stride 0); word 3 selects 32-bit data, the gfx9 value for untyped accesses.
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ f32x4 load_f4_device(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, kScDevice));
}
__device__ __forceinline__ void store_f4_device(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, const f32x4 &v) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)byte_off, 0, kScDevice);
}
// Polls a device-scope flag until it is nonzero (the same value for every
// lane).  Gives up after `limit` polls and returns false, so that a wait can
// never hang the GPU.
__device__ __forceinline__ bool wait_flag_device(const int *flag, int limit) {
    for (int k = 0; k < limit; ++k) {
        const int v = __hip_atomic_load(const_cast<int *>(flag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (__builtin_amdgcn_readfirstlane(v) != 0) {
            // Later loads stay after the poll in program order.
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            return true;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    return false;
}
__device__ __forceinline__ void set_flag_device(int *flag, int v) {
    __hip_atomic_store(flag, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16-row tile of wave w when each of NIT waves owns one tile of a chunk.
// Waves w, w+4, w+8, w+12 share a SIMD; tile t meets t/2 + 1 causal 32-token
// blocks, and these orders give every SIMD the same number.
template <int NIT>
__device__ __forceinline__ int wide_tile(int w) {
    if constexpr (NIT == 16) {
        constexpr unsigned long long map = 0xdcfeab894567'3210ull;  // nibble w = tile of wave w
        return (int)((map >> (4 * w)) & 15);
    } else if constexpr (NIT == 8) {
        return w < 4 ? w : 11 - w;
    } else {
        return w;
    }
}

// Vector of 8 / 4 elements of T for global <-> register moves.
template <typename T> struct Vec8;
template <> struct Vec8<bf16> { typedef bf16x8 type; };
template <> struct Vec8<float> { typedef float type __attribute__((ext_vector_type(8))); };
template <typename T> struct Vec4;
template <> struct Vec4<bf16> { typedef bf16x4 type; };
template <> struct Vec4<float> { typedef f32x4 type; };

// Calls f(std::integral_constant<int, I>{}) for I = 0 .. N-1 (unrolled, with
// compile-time indices, e.g. for register arrays).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace ssd
