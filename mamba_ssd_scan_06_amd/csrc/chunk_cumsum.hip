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
// Two companion tables in the same [b,H,nc,Q] layout let the output kernel
// copy a head's per-token factors of one chunk with contiguous loads:
//   dtc[i] = dt_i (0 past the end of the sequence)
//   dte[i] = dt_i * exp(cs_e - cs_i), e = the last token (within the
//            sequence) of i's 32-token block; e >= i, so the factor is <= 1.
//
// One workgroup per (b, c, 16 heads): the chunk's dt values for 16 heads are
// staged in LDS (64-byte rows per token), each thread scans one segment of
// Q/16 tokens of one head in fp64, segment offsets are added, and every entry
// is rounded once to fp32 and stored as contiguous rows.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

constexpr int kHeads = 16;  // heads per workgroup
constexpr int kBlock = 32;  // token block of dte

__global__ __launch_bounds__(256) void chunk_cumsum_kernel(Params p) {
    __shared__ double sum[256][kHeads + 1];    // [token][head]: dt, then prefix sums
    __shared__ float dts[256][kHeads + 1];
    __shared__ double seg_total[kHeads][kHeads + 1];
    const int c = blockIdx.x, h0 = blockIdx.y * kHeads;
    const int64_t b = blockIdx.z;
    const int tid = threadIdx.x;
    const int Q = p.chunk, H = p.nheads;
    const int64_t L = p.seqlen;
    const int64_t t0 = (int64_t)c * Q;
    const int Qc = (int)(L - t0 < Q ? L - t0 : Q);

    for (int e = tid; e < Q * kHeads; e += 256) {
        const int i = e / kHeads, hl = e - i * kHeads;
        const float v = (i < Qc && h0 + hl < H) ? p.dt[(b * L + t0 + i) * H + h0 + hl] : 0.f;
        dts[i][hl] = v;
        sum[i][hl] = (double)v;
    }
    __syncthreads();

    const int nseg = Q < kHeads ? Q : kHeads;
    const int seg_len = Q / nseg;
    const int hl = tid % kHeads, s = tid / kHeads;
    if (s < nseg) {
        double run = 0.0;
        for (int k = 0; k < seg_len; ++k) {
            run += sum[s * seg_len + k][hl];
            sum[s * seg_len + k][hl] = run;
        }
        seg_total[s][hl] = run;
    }
    __syncthreads();
    if (s < nseg) {
        double offset = 0.0;
        for (int k = 0; k < s; ++k) offset += seg_total[k][hl];
        for (int k = 0; k < seg_len; ++k) sum[s * seg_len + k][hl] += offset;
    }
    __syncthreads();
    if (s >= nseg || h0 + hl >= H) return;

    const double a = (double)p.A[h0 + hl];
    const int64_t row = ((b * H + h0 + hl) * p.nchunks + c) * (int64_t)Q;
    for (int k = 0; k < seg_len; ++k) {
        const int i = s * seg_len + k;
        const int e = min(kBlock * (i / kBlock) + kBlock - 1, max(Qc - 1, 0));
        const float dti = dts[i][hl];
        p.cs[row + i] = (float)(a * sum[i][hl]);
        p.dtc[row + i] = dti;
        p.dte[row + i] = i < Qc ? dti * exp_neg((float)(a * (sum[e][hl] - sum[i][hl]))) : 0.f;
    }
}

}  // namespace

hipError_t launch_chunk_cumsum(const Params &p, hipStream_t stream) {
    dim3 grid(p.nchunks, (p.nheads + kHeads - 1) / kHeads, (unsigned)p.batch);
    hipLaunchKernelGGL(chunk_cumsum_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ssd
