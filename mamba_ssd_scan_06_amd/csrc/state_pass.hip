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
// One lane per four consecutive state elements (b, h, p, n..n+3): 16-byte
// coalesced loads, sequential over chunks.  The chunk states of a batch of
// chunks are loaded before any result is stored so that the loads are in
// flight together.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

constexpr int kBatchChunks = 8;

template <typename T>
__device__ inline void store4(T *dst, const f32x4 &v);
template <>
__device__ inline void store4<float>(float *dst, const f32x4 &v) {
    *reinterpret_cast<f32x4 *>(dst) = v;
}
template <>
__device__ inline void store4<bf16>(bf16 *dst, const f32x4 &v) {
    *reinterpret_cast<bf16x4 *>(dst) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}

template <typename T>
__device__ inline f32x4 load4(const T *src);
template <>
__device__ inline f32x4 load4<float>(const float *src) {
    return *reinterpret_cast<const f32x4 *>(src);
}
template <>
__device__ inline f32x4 load4<bf16>(const bf16 *src) {
    const bf16x4 v = *reinterpret_cast<const bf16x4 *>(src);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

template <typename T>
__global__ __launch_bounds__(256) void state_pass_kernel(Params p) {
    const int64_t pn4 = (int64_t)p.headdim * p.dstate / 4;
    const int64_t per_b = (int64_t)p.nheads * pn4;
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= p.batch * per_b) return;
    const int64_t b = e / per_b;
    const int64_t rem = e - b * per_b;
    const int64_t h = rem / pn4;
    const int64_t q = rem - h * pn4;
    const int H = p.nheads, nc = p.nchunks, Q = p.chunk;

    f32x4 hc = f32x4{0.f, 0.f, 0.f, 0.f};
    if (p.init_state) hc = reinterpret_cast<const f32x4 *>(p.init_state)[e];
    const float *cs_last = p.cs + (b * H + h) * (int64_t)nc * Q + (Q - 1);
    const int64_t first = (b * nc * H + h) * pn4 + q;  // chunk 0's element, in units of 4
    const int64_t stride = (int64_t)H * pn4;           // one chunk further
    const T *st = reinterpret_cast<const T *>(p.states) + 4 * first;
    T *prev = reinterpret_cast<T *>(p.prev) + 4 * first;
    int cj = -2;  // chunk whose entering state the state-at-index step reads
    if (p.hj && p.state_out_idx) {
        const int j = p.state_out_idx[b];
        cj = j < 0 ? -1 : (int)(min((int64_t)j, p.seqlen - 1) / Q);
    }
    // Nothing accepted: the state-at-index step copies the initial state
    // from hj (init_state itself may be overwritten by final_state).
    if (cj == -1) reinterpret_cast<f32x4 *>(p.hj)[e] = hc;

#pragma unroll 1
    for (int c0 = 0; c0 < nc; c0 += kBatchChunks) {
        f32x4 s[kBatchChunks];
        float a[kBatchChunks];
#pragma unroll
        for (int k = 0; k < kBatchChunks; ++k) {
            if (c0 + k < nc) {
                s[k] = load4<T>(st + 4 * (c0 + k) * stride);
                a[k] = exp_neg(cs_last[(int64_t)(c0 + k) * Q]);
            }
        }
#pragma unroll
        for (int k = 0; k < kBatchChunks; ++k) {
            const int c = c0 + k;
            if (c < nc) {
                if (c > 0 || p.init_state) store4<T>(prev + 4 * c * stride, hc);
                if (c == cj) reinterpret_cast<f32x4 *>(p.hj)[e] = hc;
                hc = a[k] * hc + s[k];
            }
        }
    }
    if (p.final_state) reinterpret_cast<f32x4 *>(p.final_state)[e] = hc;
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
    const int64_t n4 = p.batch * p.nheads * (int64_t)p.headdim * p.dstate / 4;
    const unsigned blocks = (unsigned)((n4 + 255) / 256);
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
