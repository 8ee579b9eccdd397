// State passing over chunks (yellow part of the SSD block decomposition).
//
// "Transformers are SSMs" article (cloud.tencent.com.cn), section "SSD算法":
// the term linking chunks is itself a 1-semiseparable matrix, i.e. a scan
// over chunks with modified decay factors; section "深入解析分块与状态传递机制"
// runs it sequentially over the chunks' final states to obtain each chunk's
// true initial state.  With S_c the state chunk c reaches from a zero start
// and a_c = exp(cs[c][Q-1]) its decay:
//     h_{-1} = init_state (or 0),   h_c = a_c * h_{c-1} + S_c.
// The scan runs in fp32.  It writes
//   prev[c] = h_{c-1}, rounded (to nearest even) to the input type, the form
//             in which the output kernel feeds it to the matrix cores; chunk 0
//             only when there is an initial state (otherwise it is zero and
//             never read);
//   hj      = h_{c_j-1} in fp32 for c_j = the chunk of state_out_idx[b], when
//             the state at that index is requested (the initial state when
//             that index is -1);
//   final_state = h_{nc-1}.
// The chunk states (in the input type: one rounding of each S_c) are left as
// they are.
//
// One lane per 16 bytes of consecutive state elements (b, h, p, n..n+E-1;
// E = 8 for bf16 chunk states, 4 for fp32), sequential over chunks.  The
// chunk states are loaded in batches of kBatchChunks chunks, and the loads of
// the next batch are issued before the current one is combined, so that two
// batches of loads per lane are in flight.  The chunk states are read for
// the last time here: non-temporal loads, so that the entering states this
// kernel writes, which the output kernel reads next, take their place in the
// last-level cache.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

constexpr int kBatchChunks = 8;

// E consecutive elements of one lane, held in fp32.
template <int E> struct Lane { f32x4 v[E / 4]; };
// ... and as loaded (16 bytes in the chunk states' type).
template <typename T> struct Raw16 { typedef bf16x8 type; };
template <> struct Raw16<float> { typedef f32x4 type; };

template <typename T, int E>
__device__ inline Lane<E> widen(const typename Raw16<T>::type &w) {
    Lane<E> r;
    if constexpr (sizeof(T) == 2) {
        r.v[0] = f32x4{(float)w[0], (float)w[1], (float)w[2], (float)w[3]};
        r.v[1] = f32x4{(float)w[4], (float)w[5], (float)w[6], (float)w[7]};
    } else {
        r.v[0] = w;
    }
    return r;
}
template <typename T, int E>
__device__ inline void store_lane(T *dst, const Lane<E> &x) {
    if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<bf16x8 *>(dst) = bf16x8{(bf16)x.v[0][0], (bf16)x.v[0][1], (bf16)x.v[0][2], (bf16)x.v[0][3],
                                                  (bf16)x.v[1][0], (bf16)x.v[1][1], (bf16)x.v[1][2], (bf16)x.v[1][3]};
    } else {
        *reinterpret_cast<f32x4 *>(dst) = x.v[0];
    }
}
template <int E>
__device__ inline void store_f32(float *dst, const Lane<E> &x) {
#pragma unroll
    for (int i = 0; i < E / 4; ++i) reinterpret_cast<f32x4 *>(dst)[i] = x.v[i];
}

template <typename T>
__global__ __launch_bounds__(256) void state_pass_kernel(Params p) {
    constexpr int E = 16 / (int)sizeof(T);
    typedef Lane<E> LaneT;
    const int64_t pne = (int64_t)p.headdim * p.dstate / E;  // lanes per (b, h)
    const int64_t per_b = (int64_t)p.nheads * pne;
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= p.batch * per_b) return;
    const int64_t b = e / per_b;
    const int64_t rem = e - b * per_b;
    const int64_t h = rem / pne;
    const int64_t q = rem - h * pne;
    const int H = p.nheads, nc = p.nchunks, Q = p.chunk;

    LaneT hc;
#pragma unroll
    for (int i = 0; i < E / 4; ++i)
        hc.v[i] = p.init_state ? reinterpret_cast<const f32x4 *>(p.init_state)[e * (E / 4) + i] : f32x4{0.f, 0.f, 0.f, 0.f};
    const float *cs_last = p.cs + (b * H + h) * (int64_t)nc * Q + (Q - 1);
    const int64_t first = ((b * nc * H + h) * pne + q) * E;  // chunk 0's first element
    const int64_t stride = (int64_t)H * pne * E;              // one chunk further
    const T *st = reinterpret_cast<const T *>(p.states) + first;
    T *prev = reinterpret_cast<T *>(p.prev) + first;
    int cj = -2;  // chunk whose entering state the state-at-index step reads
    if (p.hj && p.state_out_idx) {
        const int j = p.state_out_idx[b];
        cj = j < 0 ? -1 : (int)(min((int64_t)j, p.seqlen - 1) / Q);
    }
    float *hj = p.hj ? p.hj + e * E : nullptr;
    // Nothing accepted: the state-at-index step copies the initial state
    // from hj (init_state itself may be overwritten by final_state).
    if (cj == -1) store_f32<E>(hj, hc);

    typedef typename Raw16<T>::type RawT;
    RawT s0[kBatchChunks], s1[kBatchChunks];
    float a0[kBatchChunks], a1[kBatchChunks];
    auto load_batch = [&](int c0, RawT (&s)[kBatchChunks], float (&a)[kBatchChunks]) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < kBatchChunks; ++k) {
            if (c0 + k < nc) {
                s[k] = __builtin_nontemporal_load(reinterpret_cast<const RawT *>(st + (int64_t)(c0 + k) * stride));
                a[k] = exp_neg(cs_last[(int64_t)(c0 + k) * Q]);
            }
        }
    };
    auto combine = [&](int c0, const RawT (&s)[kBatchChunks], const float (&a)[kBatchChunks]) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < kBatchChunks; ++k) {
            const int c = c0 + k;
            if (c < nc) {
                if (c > 0 || p.init_state) store_lane<T, E>(prev + (int64_t)c * stride, hc);
                if (c == cj) store_f32<E>(hj, hc);
                const LaneT sk = widen<T, E>(s[k]);
#pragma unroll
                for (int i = 0; i < E / 4; ++i) hc.v[i] = a[k] * hc.v[i] + sk.v[i];
            }
        }
    };
    load_batch(0, s0, a0);
#pragma unroll 1
    for (int c0 = 0; c0 < nc; c0 += 2 * kBatchChunks) {
        if (c0 + kBatchChunks < nc) load_batch(c0 + kBatchChunks, s1, a1);
        combine(c0, s0, a0);
        if (c0 + kBatchChunks >= nc) break;
        if (c0 + 2 * kBatchChunks < nc) load_batch(c0 + 2 * kBatchChunks, s0, a0);
        combine(c0 + kBatchChunks, s1, a1);
    }
    if (p.final_state) store_f32<E>(p.final_state + e * E, hc);
}

// seqlen == 0: the final state (and a state_out at index -1) is the initial state.
__global__ __launch_bounds__(256) void empty_sequence_kernel(Params p) {
    const int64_t n4 = p.batch * p.nheads * (int64_t)p.headdim * p.dstate / 4;
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= n4) return;
    f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
    if (p.init_state) v = reinterpret_cast<const f32x4 *>(p.init_state)[e];
    if (p.final_state) reinterpret_cast<f32x4 *>(p.final_state)[e] = v;
    if (p.state_out) reinterpret_cast<f32x4 *>(p.state_out)[e] = v;
}

}  // namespace

hipError_t launch_state_pass(const Params &p, Elem e, hipStream_t stream) {
    // (headdim * dstate is a multiple of 256: every lane has whole 16 bytes.)
    const int64_t lanes = p.batch * p.nheads * (int64_t)p.headdim * p.dstate / (e == Elem::BF16 ? 8 : 4);
    const unsigned blocks = (unsigned)((lanes + 255) / 256);
    if (e == Elem::BF16)
        hipLaunchKernelGGL(state_pass_kernel<bf16>, dim3(blocks), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(state_pass_kernel<float>, dim3(blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_empty_sequence(const Params &p, hipStream_t stream) {
    const int64_t n4 = p.batch * p.nheads * (int64_t)p.headdim * p.dstate / 4;
    const unsigned blocks = (unsigned)((n4 + 255) / 256);
    hipLaunchKernelGGL(empty_sequence_kernel, dim3(blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ssd
