// Chunk states (green part of the SSD block decomposition) and the state at
// a per-sequence accepted index (multi-step verify).
//
// "Transformers are SSMs" article (cloud.tencent.com.cn), section "SSD算法":
// the T/Q green blocks are computed by batched matrix multiplication;
// section "深入解析分块与状态传递机制": each chunk's final state assuming a zero
// initial state.  For chunk c, head h (group g):
//     S_c[p][n] = sum_{j in chunk} w_j * x_j[p] * B_j[n],
//     w_j = exp(cs_last - cs_j) * dt_j,
// a P x N result contracted over the chunk's tokens.  On the matrix cores it
// is computed transposed, S_c^T = B_c^T (w * X_c), so that every lane ends
// with four consecutive n of one p and stores them as one 16-byte write.
//
// The same kernel, with the contraction cut at token j = state_out_idx[b]
// and the decayed state entering that chunk added, gives the state after
// token j ("3天把Llama训成Mamba" article, blog.csdn.net, section "推测解码":
// the verifier keeps the state at the last accepted position):
//     h_j = exp(cs_j) * h_{c-1} + sum_{s <= j in chunk c} exp(cs_j - cs_s) dt_s x_s B_s^T.
//
// Layout of one step: 32 tokens of B and of w*x are staged in LDS transposed
// ([n][token] and [p][token]) so that each lane's fragment is 8 consecutive
// tokens (one 16-byte LDS read); w*x is formed in fp32 and rounded once to
// the input type.  Two LDS buffers alternate, so one barrier per step.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

constexpr int kKB = 32;  // tokens per contraction step

template <typename T, int NT, int PT>
__global__ __launch_bounds__(256) void chunk_state_kernel(Params p, bool at_index) {
    constexpr int RS = kKB + 16 / (int)sizeof(T);  // LDS row stride (elements)
    constexpr int N = NT * 16, P = PT * 16;
    constexpr int WN = NT >= 4 ? 4 : NT;            // waves along n
    constexpr int WP = 4 / WN;                      // waves along p
    constexpr int NTW = NT / WN;                    // n tiles per wave
    constexpr int PTW = PT >= WP ? PT / WP : 1;     // p tiles per wave
    typedef typename Vec8<T>::type V8;
    typedef typename Vec4<T>::type V4;

    __shared__ __align__(16) T bt_lds[2][N * RS];
    __shared__ __align__(16) T xw_lds[2][P * RS];
    __shared__ float w_lds[256];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int H = p.nheads, Q = p.chunk, nc = p.nchunks, G = p.ngroups;
    const int64_t L = p.seqlen;
    const int g = h / p.heads_per_group;

    int c, last;
    if (at_index) {
        int j = p.state_out_idx[b];
        j = j < -1 ? -1 : (j > L - 1 ? (int)(L - 1) : j);
        if (j < 0) {  // nothing accepted: the state is the initial one
            float *dst = p.state_out + (b * H + h) * (int64_t)P * N;
            const float *src = p.init_state ? p.init_state + (b * H + h) * (int64_t)P * N : nullptr;
            for (int e = tid * 4; e < P * N; e += 256 * 4)
                *reinterpret_cast<f32x4 *>(dst + e) =
                    src ? *reinterpret_cast<const f32x4 *>(src + e) : f32x4{0.f, 0.f, 0.f, 0.f};
            return;
        }
        c = j / Q;
        last = j - c * Q;
    } else {
        c = blockIdx.x;
        const int64_t rem = L - (int64_t)c * Q;
        last = (int)(rem < Q ? rem : Q) - 1;
    }
    const int64_t t0 = (int64_t)c * Q;
    const int ntok = last + 1;
    const float *csrow = p.cs + ((b * H + h) * nc + c) * (int64_t)Q;
    const float cs_last = csrow[last];

    const int wlen = Q > kKB ? Q : kKB;
    for (int i = tid; i < wlen; i += 256) {
        float w = 0.f;
        if (i < ntok) w = exp_neg(cs_last - csrow[i]) * p.dt[(b * L + t0 + i) * H + h];
        w_lds[i] = w;
    }
    __syncthreads();

    const T *xg = reinterpret_cast<const T *>(p.x);
    const T *bg = reinterpret_cast<const T *>(p.B);
    const int wn = wave % WN, wp = wave / WN;
    const bool wave_active = wp * PTW < PT;
    const int il = lane & 15, grp = lane >> 4;

    f32x4 acc[NTW][PTW];
#pragma unroll
    for (int a = 0; a < NTW; ++a)
#pragma unroll
        for (int q = 0; q < PTW; ++q) acc[a][q] = f32x4{0.f, 0.f, 0.f, 0.f};

    int buf = 0;
    for (int jb = 0; jb < ntok; jb += kKB, buf ^= 1) {
        // Stage: task = (4 tokens, 8 columns); B tasks first, then x tasks.
        constexpr int nb_tasks = 8 * (N / 8), nx_tasks = 8 * (P / 8);
        for (int task = tid; task < nb_tasks + nx_tasks; task += 256) {
            const bool is_b = task < nb_tasks;
            const int tt = is_b ? task : task - nb_tasks;
            const int ncol8 = (is_b ? N : P) / 8;
            const int jq = tt / ncol8, c8 = tt - jq * ncol8;
            V8 v[4];
            float wj[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int j = jb + 4 * jq + k;
                if (j < ntok) {
                    const int64_t t = t0 + j;
                    v[k] = is_b ? *reinterpret_cast<const V8 *>(bg + ((b * L + t) * G + g) * N + 8 * c8)
                                : *reinterpret_cast<const V8 *>(xg + ((b * L + t) * H + h) * P + 8 * c8);
                    wj[k] = w_lds[j];
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[k][e] = from_f32<T>(0.f);
                    wj[k] = 0.f;
                }
            }
            T *dst = is_b ? &bt_lds[buf][(8 * c8) * RS + 4 * jq] : &xw_lds[buf][(8 * c8) * RS + 4 * jq];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                V4 col;
                if (is_b) {
                    col = V4{v[0][e], v[1][e], v[2][e], v[3][e]};
                } else {
                    col = V4{from_f32<T>(wj[0] * to_f32(v[0][e])), from_f32<T>(wj[1] * to_f32(v[1][e])),
                             from_f32<T>(wj[2] * to_f32(v[2][e])), from_f32<T>(wj[3] * to_f32(v[3][e]))};
                }
                *reinterpret_cast<V4 *>(dst + e * RS) = col;
            }
        }
        __syncthreads();
        if (wave_active) {
            Frag<T> fa[NTW], fb[PTW];
#pragma unroll
            for (int a = 0; a < NTW; ++a)
                load8(fa[a], &bt_lds[buf][((wn + WN * a) * 16 + il) * RS + 8 * grp]);
#pragma unroll
            for (int q = 0; q < PTW; ++q)
                load8(fb[q], &xw_lds[buf][((wp * PTW + q) * 16 + il) * RS + 8 * grp]);
#pragma unroll
            for (int a = 0; a < NTW; ++a)
#pragma unroll
                for (int q = 0; q < PTW; ++q) mma(fa[a], fb[q], acc[a][q]);
        }
    }
    if (!wave_active) return;

    // acc[a][q][r] = S^T[n = 16*(wn + WN*a) + 4*grp + r][p = 16*(wp*PTW + q) + il]
    const int64_t state_base = ((b * nc + c) * H + h) * (int64_t)P * N;
    const float e_last = at_index ? exp_neg(cs_last) : 0.f;
#pragma unroll
    for (int a = 0; a < NTW; ++a) {
#pragma unroll
        for (int q = 0; q < PTW; ++q) {
            const int n = 16 * (wn + WN * a) + 4 * grp;
            const int pp = 16 * (wp * PTW + q) + il;
            f32x4 v = acc[a][q];
            if (at_index) {
                const f32x4 hp = *reinterpret_cast<const f32x4 *>(p.states + state_base + (int64_t)pp * N + n);
                v = v + e_last * hp;
                *reinterpret_cast<f32x4 *>(p.state_out + ((b * H + h) * (int64_t)P + pp) * N + n) = v;
            } else {
                *reinterpret_cast<f32x4 *>(p.states + state_base + (int64_t)pp * N + n) = v;
            }
        }
    }
}

template <typename T, int NT, int PT>
hipError_t launch_typed(const Params &p, bool at_index, hipStream_t stream) {
    dim3 grid(at_index ? 1 : p.nchunks, p.nheads, (unsigned)p.batch);
    hipLaunchKernelGGL((chunk_state_kernel<T, NT, PT>), grid, dim3(256), 0, stream, p, at_index);
    return hipGetLastError();
}

template <typename T, int NT>
hipError_t dispatch_p(const Params &p, bool at_index, hipStream_t stream) {
    switch (p.headdim) {
        case 16: return launch_typed<T, NT, 1>(p, at_index, stream);
        case 32: return launch_typed<T, NT, 2>(p, at_index, stream);
        case 64: return launch_typed<T, NT, 4>(p, at_index, stream);
        case 128: return launch_typed<T, NT, 8>(p, at_index, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t dispatch_n(const Params &p, bool at_index, hipStream_t stream) {
    switch (p.dstate) {
        case 16: return dispatch_p<T, 1>(p, at_index, stream);
        case 32: return dispatch_p<T, 2>(p, at_index, stream);
        case 64: return dispatch_p<T, 4>(p, at_index, stream);
        case 128: return dispatch_p<T, 8>(p, at_index, stream);
        case 256: return dispatch_p<T, 16>(p, at_index, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_chunk_state(const Params &p, Elem e, hipStream_t stream) {
    return e == Elem::BF16 ? dispatch_n<bf16>(p, false, stream) : dispatch_n<float>(p, false, stream);
}

hipError_t launch_state_at_index(const Params &p, Elem e, hipStream_t stream) {
    return e == Elem::BF16 ? dispatch_n<bf16>(p, true, stream) : dispatch_n<float>(p, true, stream);
}

}  // namespace ssd
