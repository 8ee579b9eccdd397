// Chunk-local cumulative log-decay (first step of the SSD block decomposition).
//
// "Transformers are SSMs" article (cloud.tencent.com.cn), section "SSD算法":
// the scan over chunks runs on modified A factors, and inside a chunk the
// quadratic form needs the decay between any two of its tokens.  Both come
// from one chunk-local prefix sum:
//     cs[b,h,c,i] = A[h] * sum_{k=0..i} dt[b, c*Q+k, h]
// (tokens past the end of the sequence count as dt = 0).  The decay from token
// j to token i of one chunk is exp(cs_i - cs_j) and the chunk's own decay is
// exp(cs_{Q-1}).  Sums restart at every chunk, so a long sequence never
// builds an exponent beyond one chunk's.
//
// One lane per (b, h, c): lanes of a wave take 64 consecutive heads, so each
// step reads 64 consecutive dt values of one token.  The sum is carried in
// fp64 and rounded once per entry.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

__global__ __launch_bounds__(64) void chunk_cumsum_kernel(Params p) {
    const int c = blockIdx.x;
    const int h = blockIdx.y * kWave + threadIdx.x;
    const int64_t b = blockIdx.z;
    if (h >= p.nheads) return;
    const int Q = p.chunk, H = p.nheads;
    const int64_t T = p.seqlen;
    const int64_t t0 = (int64_t)c * Q;
    const int valid = (int)(T - t0 < Q ? T - t0 : Q);
    const double a = (double)p.A[h];
    const float *dtp = p.dt + (b * T + t0) * H + h;
    float *out = p.cs + ((b * H + h) * p.nchunks + c) * Q;
    double acc = 0.0;
#pragma unroll 8
    for (int i = 0; i < Q; ++i) {
        if (i < valid) acc += (double)dtp[(int64_t)i * H];
        out[i] = (float)(a * acc);
    }
}

}  // namespace

hipError_t launch_chunk_cumsum(const Params &p, hipStream_t stream) {
    dim3 grid(p.nchunks, (p.nheads + kWave - 1) / kWave, (unsigned)p.batch);
    hipLaunchKernelGGL(chunk_cumsum_kernel, grid, dim3(kWave), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ssd
