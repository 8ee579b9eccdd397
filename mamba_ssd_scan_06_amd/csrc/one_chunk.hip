// Fused forward of a call whose tokens fit one chunk of at most 32 tokens:
// the multi-step verify of speculative decoding ("3天把Llama训成Mamba"
// article, blog.csdn.net, section "推测解码": the verifier takes a cached
// state, runs the K draft tokens in one step, and keeps the state at the last
// accepted position and after the last token).
//
// With one chunk the block decomposition of "Transformers are SSMs"
// (cloud.tencent.com.cn, section "SSD算法") has no state passing: for tokens
// t, s < T of sequence b, head h (group g), with cs_t = A_h sum_{k<=t} dt_k,
//     e_t    = exp(cs_t),     W[t][s] = exp(cs_t - cs_s) dt_s   (s <= t)
//     h_t    = e_t h0 + sum_{s<=t} W[t][s] x_s B_s^T             (P x N)
//     y_t    = e_t (h0 C_t) + sum_{s<=t} W[t][s] (C_t . B_s) x_s + D x_t
// final_state = h_{T-1} and state_out = h_j (j = state_out_idx[b]; h0 for
// j = -1).  One workgroup per (b, h) reads h0 once, writes both states in
// fp32 and y; everything is computed in fp32 on the vector units (the state
// updates are rank-T, too thin for the matrix cores).
//
// Work split: N/4 consecutive lanes cover one state row, 16 bytes each, so
// every load and store of a wave is whole rows; per row each lane forms its
// pieces of both states and its partial products h0 C_t, which a
// reduce-scatter over the row's lanes sums.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

constexpr int kMaxTokens = 32;  // longest call the fused kernel takes
constexpr int kThreads = 256;

// MT: token capacity of this instance (8, 16 or 32), sizing LDS and the
// per-row coefficient registers.
template <typename T, int NT, int PT, int MT>
__global__ __launch_bounds__(kThreads) void one_chunk_kernel(Params p) {
    constexpr int kMaxT = MT;
    constexpr int N = NT * 16, P = PT * 16;
    constexpr int TPR = N / 4;            // lanes per state row (4 .. 64)
    constexpr int RPP = kThreads / TPR;   // rows per pass
    static_assert(P % RPP == 0, "rows per pass");
    constexpr int kLog2Tpr = TPR == 4 ? 2 : TPR == 8 ? 3 : TPR == 16 ? 4 : TPR == 32 ? 5 : 6;
    constexpr int KEEP = MT > TPR ? MT / TPR : 1;  // values a lane holds after the reduction
    __shared__ float xs[kMaxT][P];
    __shared__ __align__(16) float bsh[kMaxT][N];
    __shared__ __align__(16) float csh[kMaxT][N];
    __shared__ float wsh[kMaxT][kMaxT];  // W[t][s]
    __shared__ float msh[kMaxT][kMaxT];  // W[t][s] * (C_t . B_s)
    __shared__ float esh[kMaxT];
    __shared__ float dts[kMaxT];
    __shared__ double run_dt[kMaxT];     // sum_{k<=t} dt_k

    const int h = blockIdx.x;
    const int64_t b = blockIdx.y;
    const int H = p.nheads, G = p.ngroups;
    const int g = h / p.heads_per_group;
    const int L = (int)p.seqlen;  // 1 .. MT
    const int tid = threadIdx.x;

    // dt of the call, then its prefix sums in fp64 (one thread, <= 32 adds).
    if (tid < kMaxT) dts[tid] = tid < L ? p.dt[(b * L + tid) * H + h] : 0.f;
    // x, B, C of the call in fp32.
    const T *xg = reinterpret_cast<const T *>(p.x);
    const T *bg = reinterpret_cast<const T *>(p.B);
    const T *cg = reinterpret_cast<const T *>(p.C);
    for (int e = tid; e < kMaxT * P; e += kThreads) {
        const int t = e / P, pp = e - t * P;
        xs[t][pp] = t < L ? (float)xg[((b * L + t) * H + h) * P + pp] : 0.f;
    }
    for (int e = tid; e < kMaxT * N; e += kThreads) {
        const int t = e / N, n = e - t * N;
        bsh[t][n] = t < L ? (float)bg[((b * L + t) * G + g) * N + n] : 0.f;
        csh[t][n] = t < L ? (float)cg[((b * L + t) * G + g) * N + n] : 0.f;
    }
    __syncthreads();
    if (tid == 0) {
        double r = 0.0;
        for (int k = 0; k < kMaxT; ++k) {
            r += (double)dts[k];
            run_dt[k] = r;
        }
    }
    __syncthreads();
    // e_t = exp(cs_t) and W[t][s] = exp(cs_t - cs_s) dt_s: the exponents come
    // from fp64 partial sums, rounded once, then the hardware exp.
    const double a = (double)p.A[h];
    if (tid < kMaxT) esh[tid] = tid < L ? exp_neg((float)(a * run_dt[tid])) : 0.f;
    for (int e = tid; e < kMaxT * kMaxT; e += kThreads) {
        const int t = e / kMaxT, s = e - t * kMaxT;
        wsh[t][s] = (t < L && s <= t) ? exp_neg((float)(a * (run_dt[t] - run_dt[s]))) * dts[s] : 0.f;
    }
    __syncthreads();
    // M[t][s] = W[t][s] (C_t . B_s).
    for (int e = tid; e < kMaxT * kMaxT; e += kThreads) {
        const int t = e / kMaxT, s = e - t * kMaxT;
        float m = 0.f;
        if (t < L && s <= t) {
            float d = 0.f;
            for (int n = 0; n < N; n += 4) {
                const f32x4 cv = *reinterpret_cast<const f32x4 *>(&csh[t][n]);
                const f32x4 bv = *reinterpret_cast<const f32x4 *>(&bsh[s][n]);
                d += cv[0] * bv[0] + cv[1] * bv[1] + cv[2] * bv[2] + cv[3] * bv[3];
            }
            m = wsh[t][s] * d;
        }
        msh[t][s] = m;
    }
    __syncthreads();

    // Lanes: TPR = N/4 consecutive lanes cover one state row (16 bytes
    // each, so a wave's loads and stores are whole rows); the workgroup
    // covers RPP rows per pass.
    int j = -1;  // accepted index
    if (p.state_out) {
        j = p.state_out_idx[b];
        j = j < -1 ? -1 : (j > L - 1 ? L - 1 : j);
    }
    const int lr = tid % TPR, rg = tid / TPR;
    const int n0 = 4 * lr;
    const float eT = esh[L - 1], ej = j >= 0 ? esh[j] : 1.f;
    const float dh = p.D ? p.D[h] : 0.f;
    T *yg = reinterpret_cast<T *>(p.y);
    const int64_t hbase = (b * H + h) * (int64_t)P * N;

    // The initial-state rows of up to kInFlight passes are requested before
    // any of their results is stored: a wave's loads and stores complete in
    // order, so a load issued after a store would also wait for that store.
    constexpr int NPASS = P / RPP;
    constexpr int kInFlight = NPASS < 16 ? NPASS : 16;
    static_assert(NPASS % kInFlight == 0, "pass groups");
    f32x4 h0s[kInFlight];
    for (int g0 = 0; g0 < NPASS; g0 += kInFlight) {
#pragma unroll
        for (int u = 0; u < kInFlight; ++u)
            h0s[u] = p.init_state ? *reinterpret_cast<const f32x4 *>(p.init_state + hbase +
                                                                      (int64_t)((g0 + u) * RPP + rg) * N + n0)
                                  : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            const int pass = g0 + u;
            const int pp = pass * RPP + rg;
            const int64_t at = hbase + (int64_t)pp * N + n0;
            const f32x4 h0 = h0s[u];
            f32x4 fin = eT * h0, sout = ej * h0;
            float v[MT];  // partial h0 . C_t over this lane's four columns
#pragma unroll
            for (int s = 0; s < MT; ++s) {
                v[s] = 0.f;
                if (s < L) {
                    const float xv = xs[s][pp];
                    const f32x4 bv = *reinterpret_cast<const f32x4 *>(&bsh[s][n0]);
                    fin += (wsh[L - 1][s] * xv) * bv;
                    if (s <= j) sout += (wsh[j][s] * xv) * bv;
                    const f32x4 cv = *reinterpret_cast<const f32x4 *>(&csh[s][n0]);
                    v[s] = cv[0] * h0[0] + cv[1] * h0[1] + cv[2] * h0[2] + cv[3] * h0[3];
                }
            }
            // Both states are written once and not read again here: non-temporal
            // stores keep them from displacing lines that are still to be read.
            if (p.final_state) __builtin_nontemporal_store(fin, reinterpret_cast<f32x4 *>(p.final_state + at));
            if (p.state_out) __builtin_nontemporal_store(sout, reinterpret_cast<f32x4 *>(p.state_out + at));

            // Sum v over the TPR lanes of the row by reduce-scatter: each step
            // on lane bit d halves the values a lane holds (keeping the upper or
            // lower half of the t range by that bit), then plain sums.
            int tbase = 0;
            int len = MT;
            static_for<kLog2Tpr>([&](auto kc) __attribute__((always_inline)) {
                constexpr int d = TPR >> (decltype(kc)::value + 1);
                constexpr int half = MT >> (decltype(kc)::value + 1);
                const bool upper = (lr & d) != 0;
                if constexpr (half >= 1) {
#pragma unroll
                    for (int i = 0; i < half; ++i) {
                        const float send = upper ? v[i] : v[half + i];
                        const float keep = upper ? v[half + i] : v[i];
                        v[i] = keep + __shfl_xor(send, d, 64);
                    }
                    if (upper) tbase += half;
                } else {
                    v[0] += __shfl_xor(v[0], d, 64);
                }
            });
            (void)len;
            // The lane now holds (h0 C_t)[pp] for t = tbase .. tbase + KEEP - 1;
            // the lanes with the low bits clear write y_t[pp].
            if ((lr & (TPR / (MT < TPR ? MT : TPR) - 1)) == 0 || MT >= TPR) {
#pragma unroll
                for (int i = 0; i < KEEP; ++i) {
                    const int t = tbase + i;
                    if (t < L) {
                        float yv = esh[t] * v[i] + dh * xs[t][pp];
                        for (int s2 = 0; s2 <= t; ++s2) yv += msh[t][s2] * xs[s2][pp];
                        yg[((b * L + t) * H + h) * P + pp] = (T)yv;
                    }
                }
            }
        }
    }
}

template <typename T, int NT, int PT>
hipError_t launch_mt(const Params &p, hipStream_t stream) {
    if constexpr ((PT * 16) % (kThreads / (NT * 4)) != 0) {
        return hipErrorNotSupported;  // fewer state rows than one pass covers
    } else {
        const dim3 grid(p.nheads, (unsigned)p.batch);
        if (p.seqlen <= 8)
            hipLaunchKernelGGL((one_chunk_kernel<T, NT, PT, 8>), grid, dim3(kThreads), 0, stream, p);
        else if (p.seqlen <= 16)
            hipLaunchKernelGGL((one_chunk_kernel<T, NT, PT, 16>), grid, dim3(kThreads), 0, stream, p);
        else
            hipLaunchKernelGGL((one_chunk_kernel<T, NT, PT, 32>), grid, dim3(kThreads), 0, stream, p);
        return hipGetLastError();
    }
}

template <typename T, int NT>
hipError_t dispatch_p(const Params &p, hipStream_t stream) {
    switch (p.headdim) {
        case 16: return launch_mt<T, NT, 1>(p, stream);
        case 32: return launch_mt<T, NT, 2>(p, stream);
        case 64: return launch_mt<T, NT, 4>(p, stream);
        case 128: return launch_mt<T, NT, 8>(p, stream);
        default: return hipErrorNotSupported;
    }
}

template <typename T>
hipError_t dispatch_n(const Params &p, hipStream_t stream) {
    switch (p.dstate) {
        case 16: return dispatch_p<T, 1>(p, stream);
        case 32: return dispatch_p<T, 2>(p, stream);
        case 64: return dispatch_p<T, 4>(p, stream);
        case 128: return dispatch_p<T, 8>(p, stream);
        case 256: return dispatch_p<T, 16>(p, stream);
        default: return hipErrorNotSupported;
    }
}

}  // namespace

// A pass over the state covers 256 threads / (dstate / 4) threads per row =
// 1024 / dstate rows; headdim must be a multiple of it.
bool one_chunk_takes(const Params &p) {
    return p.seqlen >= 1 && p.seqlen <= kMaxTokens && p.nchunks == 1 && p.headdim % (1024 / p.dstate) == 0;
}

hipError_t launch_one_chunk(const Params &p, Elem e, hipStream_t stream) {
    if (!one_chunk_takes(p)) return hipErrorNotSupported;
    return e == Elem::BF16 ? dispatch_n<bf16>(p, stream) : dispatch_n<float>(p, stream);
}

}  // namespace ssd
