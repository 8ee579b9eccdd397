// State passing over chunks (yellow part of the SSD block decomposition).
//
// "Transformers are SSMs" article (cloud.tencent.com.cn), section "SSD算法":
// the term linking chunks is itself a 1-semiseparable matrix, i.e. a scan
// over chunks with modified decay factors; section "深入解析分块与状态传递机制"
// runs it sequentially over the chunks' final states to obtain each chunk's
// true initial state.  With S_c the state chunk c reaches from a zero start
// and a_c = exp(cs[c][Q-1]) its decay:
//     h_{-1} = init_state (or 0),   h_c = a_c * h_{c-1} + S_c.
// The kernel overwrites S_c with h_{c-1} (the state entering chunk c) and
// writes h_{nc-1} to final_state.  For bf16 inputs it also stores h_{c-1}
// rounded to bf16 (to nearest even), the form in which the output kernel
// feeds it to the matrix cores.
//
// One lane per four consecutive state elements (b, h, p, n..n+3): 16-byte
// coalesced loads and stores, sequential over chunks.  The chunk states of a
// batch of chunks are loaded before any is overwritten so that the loads
// are in flight together.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

constexpr int kBatchChunks = 8;

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
    f32x4 *st = reinterpret_cast<f32x4 *>(p.states);

    for (int c0 = 0; c0 < nc; c0 += kBatchChunks) {
        f32x4 s[kBatchChunks];
        float a[kBatchChunks];
#pragma unroll
        for (int k = 0; k < kBatchChunks; ++k) {
            if (c0 + k < nc) {
                s[k] = st[((b * nc + c0 + k) * H + h) * pn4 + q];
                a[k] = exp_neg(cs_last[(int64_t)(c0 + k) * Q]);
            }
        }
#pragma unroll
        for (int k = 0; k < kBatchChunks; ++k) {
            if (c0 + k < nc) {
                const int64_t at = ((b * nc + c0 + k) * H + h) * pn4 + q;
                st[at] = hc;
                if (p.states16)
                    reinterpret_cast<bf16x4 *>(p.states16)[at] = bf16x4{(bf16)hc[0], (bf16)hc[1], (bf16)hc[2], (bf16)hc[3]};
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

hipError_t launch_state_pass(const Params &p, hipStream_t stream) {
    const int64_t n4 = p.batch * p.nheads * (int64_t)p.headdim * p.dstate / 4;
    const unsigned blocks = (unsigned)((n4 + 255) / 256);
    hipLaunchKernelGGL(state_pass_kernel, dim3(blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_empty_sequence(const Params &p, hipStream_t stream) {
    const int64_t n4 = p.batch * p.nheads * (int64_t)p.headdim * p.dstate / 4;
    const unsigned blocks = (unsigned)((n4 + 255) / 256);
    hipLaunchKernelGGL(empty_sequence_kernel, dim3(blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ssd
