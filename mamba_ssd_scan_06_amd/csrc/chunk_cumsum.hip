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
//   ct[i]  = cs_i * log2(e) - log2(dt_i) (+inf past the end of the sequence),
//            so that dt_j exp(cs_i - cs_j) = exp2(cs_i log2(e) - ct_j);
//   dte[i] = dt_i * exp(cs_e - cs_i), e = the last token (within the
//            sequence) of i's 32-token block; e >= i, so the factor is <= 1.
//
// One wave per (b, c, h), four heads per workgroup.  The chunk's dt values of
// the four heads are read with the token-major rows' contiguous 16 bytes per
// token and transposed through LDS; each lane then owns Q/64 (at least one)
// consecutive tokens, the prefix sum runs in fp64 (within the lane, then a
// wave-wide scan of the lane totals), every entry is rounded once to fp32,
// and each lane stores its tokens of a table row with one vector store.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

constexpr int kHeads = 4;   // heads (waves) per workgroup
constexpr int kBlock = 32;  // token block of dte
constexpr double kLog2eD = 1.4426950408889634074;

__device__ inline double shfl_up_f64(double v, int delta, int lane) {
    const int src = lane >= delta ? lane - delta : lane;
    const int lo = __builtin_amdgcn_ds_bpermute(src << 2, (int)__double2loint(v));
    const int hi = __builtin_amdgcn_ds_bpermute(src << 2, (int)__double2hiint(v));
    return __hiloint2double(hi, lo);
}

__device__ inline double shfl_f64(double v, int src) {
    const int lo = __builtin_amdgcn_ds_bpermute(src << 2, (int)__double2loint(v));
    const int hi = __builtin_amdgcn_ds_bpermute(src << 2, (int)__double2hiint(v));
    return __hiloint2double(hi, lo);
}

template <int V> struct FVec { typedef float __attribute__((ext_vector_type(V))) type; };
template <> struct FVec<1> { typedef float type; };

template <int VPT>
__global__ __launch_bounds__(64 * kHeads) void chunk_cumsum_kernel(Params p) {
    __shared__ float dts[kHeads][256];
    const int c = blockIdx.x, h0 = blockIdx.y * kHeads;
    const int64_t b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int Q = p.chunk, H = p.nheads, nc = p.nchunks;
    const int64_t L = p.seqlen;
    const int64_t t0 = (int64_t)c * Q;
    const int Qc = (int)(L - t0 < Q ? L - t0 : Q);

    // dt[b, t0 + i, h0 + k] -> dts[k][i]; consecutive threads read the four
    // heads of one token, then the next token.  The loads go through a
    // buffer descriptor over the chunk's dt rows (tokens past the sequence
    // read as zero), so that they are unconditional and all in flight at
    // once (a load under a condition gets its own branch and wait).
    {
        constexpr int U = 256 * kHeads / (64 * kHeads);  // loads per thread at Q = 256
        const auto rd = buffer_rsrc(p.dt + (b * L + t0) * H, (uint32_t)((int64_t)Qc * H * 4));
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = tid + u * 64 * kHeads, i = e / kHeads, k = e - i * kHeads;
            v[u] = e < Q * kHeads ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                                  rd, (i * H + h0 + k) * 4, 0, 0))
                                  : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = tid + u * 64 * kHeads, i = e / kHeads, k = e - i * kHeads;
            if (e < Q * kHeads) dts[k][i] = h0 + k < H ? v[u] : 0.f;
        }
    }
    __syncthreads();
    const int h = h0 + wave;
    if (h >= H) return;

    // Tokens i = VPT*lane + v (lanes past the chunk hold zeros and store nothing).
    const int i0 = VPT * lane;
    float dtv[VPT];
    double s[VPT];
    double run = 0.0;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        dtv[v] = i0 + v < Q ? dts[wave][i0 + v] : 0.f;
        run += (double)dtv[v];
        s[v] = run;
    }
    // Inclusive scan of the lane totals across the wave (Hillis-Steele).
    double tot = run;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const double o = shfl_up_f64(tot, d, lane);
        if (lane >= d) tot += o;
    }
    const double before = tot - run;
#pragma unroll
    for (int v = 0; v < VPT; ++v) s[v] += before;

    // Sum at e = end of the lane's 32-token block, clipped to the chunk's
    // last valid token.  A lane's VPT tokens lie in one block.
    const int ie = min(kBlock * (i0 / kBlock) + kBlock - 1, max(Qc - 1, 0));
    double se = 0.0;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const double o = shfl_f64(s[v], ie / VPT);
        if (ie % VPT == v) se = o;
    }

    const double a = (double)p.A[h];
    typename FVec<VPT>::type csv, ctv, dtev;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const bool in = i0 + v < Qc;
        const float cs_i = (float)(a * s[v]);
        const float ct = in ? (float)(a * s[v] * kLog2eD) - log2f(dtv[v]) : __builtin_inff();
        const float de = in ? dtv[v] * exp_neg((float)(a * (se - s[v]))) : 0.f;
        if constexpr (VPT == 1) {
            csv = cs_i;
            ctv = ct;
            dtev = de;
        } else {
            csv[v] = cs_i;
            ctv[v] = ct;
            dtev[v] = de;
        }
    }
    if (i0 < Q) {
        typedef typename FVec<VPT>::type FV;
        const int64_t row = ((b * H + h) * nc + c) * (int64_t)Q + i0;
        *reinterpret_cast<FV *>(p.cs + row) = csv;
        *reinterpret_cast<FV *>(p.ct + row) = ctv;
        *reinterpret_cast<FV *>(p.dte + row) = dtev;
    }
}

}  // namespace

hipError_t launch_chunk_cumsum(const Params &p, hipStream_t stream) {
    dim3 grid(p.nchunks, (p.nheads + kHeads - 1) / kHeads, (unsigned)p.batch);
    if (p.chunk > 256) return hipErrorNotSupported;
    if (p.chunk == 256)
        hipLaunchKernelGGL(chunk_cumsum_kernel<4>, grid, dim3(64 * kHeads), 0, stream, p);
    else if (p.chunk == 128)
        hipLaunchKernelGGL(chunk_cumsum_kernel<2>, grid, dim3(64 * kHeads), 0, stream, p);
    else
        hipLaunchKernelGGL(chunk_cumsum_kernel<1>, grid, dim3(64 * kHeads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ssd
