// Chunk outputs: diagonal blocks (orange) plus the contribution of each
// chunk's initial state (blue) plus the D skip, in one kernel.
//
// "Transformers are SSMs" article (cloud.tencent.com.cn), section "SSD算法":
// each diagonal block is a small semiseparable matrix evaluated in the
// attention-like quadratic form; the blue blocks are batched matrix
// products with the true initial state of the chunk.  Section
// "深入解析分块与状态传递机制" describes the same split: a local output assuming
// a zero initial state, then the contribution of the real initial state.
// For token i of chunk c, head h (group g), channel p:
//     y_i[p] = sum_{j<=i} exp(cs_i - cs_j) dt_j (C_i . B_j) x_j[p]      (orange)
//            + exp(cs_i) sum_n h_{c-1}[p][n] C_i[n]                     (blue)
//            + D_h x_i[p]
//
// Work split: one workgroup per (b, c, h, block of 64 tokens i); wave w
// owns 16 tokens.  Everything is computed transposed (rows p, columns i), so
// that the first product's output tile G^T[j][i] = B_j . C_i, once masked
// and scaled, is exactly the second product's B operand: a lane holds
// G^T[4*grp + r][il] for r = 0..3, and two such tiles (tokens j0..j0+15 and
// j0+16..j0+31) make the 8 contraction slots of one fragment.  The x operand
// is read from LDS with the same token-to-slot assignment.  The decay mask is
// applied before the exponential is taken (exp only of cs_i - cs_j with
// j <= i), and causal tiles above the diagonal are skipped.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

constexpr int kIBlk = 64;  // tokens i per workgroup
constexpr int kJB = 32;    // tokens j per staging step

template <typename T, int NT, int PT>
__global__ __launch_bounds__(256) void chunk_output_kernel(Params p) {
    constexpr int N = NT * 16, P = PT * 16;
    constexpr int KS = (N + 31) / 32;          // contraction steps over n
    constexpr int NP = KS * 32;                // n padded to whole steps
    constexpr int PAD = 16 / (int)sizeof(T);
    constexpr int RSB = NP + PAD;              // B block row stride   [j][n]
    constexpr int RSX = kJB + PAD;             // x^T block row stride [p][j]
    constexpr int RSH = NP + PAD;              // h_prev row stride    [p][n]
    typedef typename Vec8<T>::type V8;
    typedef typename Vec4<T>::type V4;

    __shared__ float cs_l[256];
    __shared__ float dt_l[256];
    __shared__ __align__(16) T b_lds[kJB * RSB];
    __shared__ __align__(16) T x_lds[P * RSX];
    __shared__ __align__(16) T h_lds[P * RSH];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int il = lane & 15, grp = lane >> 4;
    const int Q = p.chunk, H = p.nheads, G = p.ngroups, nc = p.nchunks;
    const int64_t L = p.seqlen;
    const int iblocks = (Q + kIBlk - 1) / kIBlk;
    const int c = blockIdx.x / iblocks, ib = blockIdx.x - c * iblocks;
    const int h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int g = h / p.heads_per_group;
    const int64_t t0 = (int64_t)c * Q;
    const int Qc = (int)(L - t0 < Q ? L - t0 : Q);
    const int i0 = ib * kIBlk;
    if (i0 >= Qc) return;
    const int iend = i0 + kIBlk < Qc ? i0 + kIBlk : Qc;

    const float *csrow = p.cs + ((b * H + h) * nc + c) * (int64_t)Q;
    for (int i = tid; i < 256; i += 256) {
        cs_l[i] = i < Q ? csrow[i] : 0.f;
        dt_l[i] = i < Qc ? p.dt[(b * L + t0 + i) * H + h] : 0.f;
    }
    const bool has_prev = c > 0 || p.init_state != nullptr;
    if (has_prev) {
        const float *hp = p.states + ((b * nc + c) * H + h) * (int64_t)P * N;
        for (int q = tid; q < P * (NP / 8); q += 256) {
            const int pp = q / (NP / 8), n0 = 8 * (q - pp * (NP / 8));
            V8 v;
            if (n0 < N) {
                const f32x4 a = *reinterpret_cast<const f32x4 *>(hp + (int64_t)pp * N + n0);
                const f32x4 bq = *reinterpret_cast<const f32x4 *>(hp + (int64_t)pp * N + n0 + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = from_f32<T>(a[e]);
                    v[e + 4] = from_f32<T>(bq[e]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = from_f32<T>(0.f);
            }
            *reinterpret_cast<V8 *>(&h_lds[pp * RSH + n0]) = v;
        }
    }
    __syncthreads();

    const int iw0 = i0 + 16 * wave;            // first token of this wave
    const bool active = iw0 < iend;
    const int i = iw0 + il;                    // this lane's token (column)
    const bool valid_i = active && i < iend;
    const T *xg = reinterpret_cast<const T *>(p.x);
    const T *bg = reinterpret_cast<const T *>(p.B);
    const T *cg = reinterpret_cast<const T *>(p.C);

    // C_i fragments, one per contraction step over n.
    Frag<T> cf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int n0 = 32 * ks + 8 * grp;
        if (valid_i && n0 < N)
            load8(cf[ks], cg + ((b * L + t0 + i) * G + g) * N + n0);
        else
            cf[ks].zero();
    }

    f32x4 acc[PT];
#pragma unroll
    for (int q = 0; q < PT; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Blue: exp(cs_i) * (h_prev C_i^T), rows p, column i.
    if (active && has_prev) {
#pragma unroll
        for (int q = 0; q < PT; ++q) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                Frag<T> a;
                load8(a, &h_lds[(16 * q + il) * RSH + 32 * ks + 8 * grp]);
                mma(a, cf[ks], acc[q]);
            }
        }
        const float ei = valid_i ? exp_neg(cs_l[i]) : 0.f;
#pragma unroll
        for (int q = 0; q < PT; ++q) acc[q] = acc[q] * ei;
    }

    // Orange: causal quadratic form, 32 tokens j per step.
    const float cs_i = valid_i ? cs_l[i] : 0.f;
    for (int jb = 0; jb < iend; jb += kJB) {
        __syncthreads();  // previous step's LDS reads are done
        for (int q = tid; q < kJB * (NP / 8); q += 256) {
            const int jj = q / (NP / 8), n0 = 8 * (q - jj * (NP / 8));
            const int j = jb + jj;
            V8 v;
            if (j < Qc && n0 < N) {
                v = *reinterpret_cast<const V8 *>(bg + ((b * L + t0 + j) * G + g) * N + n0);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = from_f32<T>(0.f);
            }
            *reinterpret_cast<V8 *>(&b_lds[jj * RSB + n0]) = v;
        }
        for (int q = tid; q < 8 * (P / 8); q += 256) {
            const int jq = q / (P / 8), p8 = q - jq * (P / 8);
            V8 v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int j = jb + 4 * jq + k;
                if (j < Qc) {
                    v[k] = *reinterpret_cast<const V8 *>(xg + ((b * L + t0 + j) * H + h) * P + 8 * p8);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[k][e] = from_f32<T>(0.f);
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e)
                *reinterpret_cast<V4 *>(&x_lds[(8 * p8 + e) * RSX + 4 * jq]) = V4{v[0][e], v[1][e], v[2][e], v[3][e]};
        }
        __syncthreads();
        if (!active || jb > iw0 + 15) continue;

        // G^T[j][i] for j in jb..jb+15 (g0) and jb+16..jb+31 (g1).
        f32x4 g0 = f32x4{0.f, 0.f, 0.f, 0.f}, g1 = g0;
        const bool need1 = jb + 16 <= iw0 + 15;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            Frag<T> a;
            load8(a, &b_lds[il * RSB + 32 * ks + 8 * grp]);
            mma(a, cf[ks], g0);
        }
        if (need1) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                Frag<T> a;
                load8(a, &b_lds[(16 + il) * RSB + 32 * ks + 8 * grp]);
                mma(a, cf[ks], g1);
            }
        }
        // Mask (j <= i) before exp, scale by the decay and dt_j, round once.
        Frag<T> lf;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j0 = jb + 4 * grp + r, j1 = j0 + 16;
            const float v0 = (valid_i && j0 <= i) ? g0[r] * exp_neg(cs_i - cs_l[j0]) * dt_l[j0] : 0.f;
            const float v1 = (valid_i && j1 <= i) ? g1[r] * exp_neg(cs_i - cs_l[j1]) * dt_l[j1] : 0.f;
            lf.set(r, v0);
            lf.set(4 + r, v1);
        }
#pragma unroll
        for (int q = 0; q < PT; ++q) {
            Frag<T> ax;
            const T *row = &x_lds[(16 * q + il) * RSX];
            load4x2(ax, row + 4 * grp, row + 16 + 4 * grp);
            mma(ax, lf, acc[q]);
        }
    }

    // Epilogue: + D x, round to the output type; lane holds p = 16q + 4grp + r of token i.
    if (!valid_i) return;
    const float dh = p.D ? p.D[h] : 0.f;
    const int64_t row = ((b * L + t0 + i) * H + h) * (int64_t)P;
    T *yg = reinterpret_cast<T *>(p.y);
#pragma unroll
    for (int q = 0; q < PT; ++q) {
        const int p0 = 16 * q + 4 * grp;
        const V4 xv = *reinterpret_cast<const V4 *>(xg + row + p0);
        V4 out;
#pragma unroll
        for (int r = 0; r < 4; ++r) out[r] = from_f32<T>(acc[q][r] + dh * to_f32(xv[r]));
        *reinterpret_cast<V4 *>(yg + row + p0) = out;
    }
}

template <typename T, int NT, int PT>
hipError_t launch_typed(const Params &p, hipStream_t stream) {
    if constexpr (sizeof(T) == 4 && NT * PT > 64) {
        return hipErrorInvalidValue;  // fp32 state tile beyond the LDS budget (rejected by the host checks)
    } else {
    const int iblocks = (p.chunk + kIBlk - 1) / kIBlk;
    dim3 grid(p.nchunks * iblocks, p.nheads, (unsigned)p.batch);
    hipLaunchKernelGGL((chunk_output_kernel<T, NT, PT>), grid, dim3(256), 0, stream, p);
    return hipGetLastError();
    }
}

template <typename T, int NT>
hipError_t dispatch_p(const Params &p, hipStream_t stream) {
    switch (p.headdim) {
        case 16: return launch_typed<T, NT, 1>(p, stream);
        case 32: return launch_typed<T, NT, 2>(p, stream);
        case 64: return launch_typed<T, NT, 4>(p, stream);
        case 128: return launch_typed<T, NT, 8>(p, stream);
        default: return hipErrorInvalidValue;
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
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_chunk_output(const Params &p, Elem e, hipStream_t stream) {
    return e == Elem::BF16 ? dispatch_n<bf16>(p, stream) : dispatch_n<float>(p, stream);
}

}  // namespace ssd
