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
// Staging: 32 tokens of B and of w*x at a time are copied into LDS in their
// natural token-major layout (whole 16-byte pieces of rows; w*x is formed in
// fp32 and rounded once to the input type on the way).  Both operands have
// the token as contraction index, so their fragments are read with the
// transposing LDS read (see load_tr).  Two LDS buffers alternate and the
// global loads of a step are issued two steps ahead, so one barrier per step.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

constexpr int kKB = 32;   // tokens per contraction step
constexpr int kXcds = 8;  // XCDs of an MI355X

template <typename T, int NT, int PT>
__global__ __launch_bounds__(256) void chunk_state_kernel(Params p, bool at_index) {
    constexpr int N = NT * 16, P = PT * 16;
    constexpr int PADE = 32 / (int)sizeof(T);       // 32-byte row padding
    constexpr int LDB = N + PADE, LDX = P + PADE;   // LDS row strides (elements)
    constexpr int WN = NT >= 4 ? 4 : NT;            // waves along n
    constexpr int WP = 4 / WN;                      // waves along p
    constexpr int NTW = NT / WN;                    // n tiles per wave
    constexpr int PTW = PT >= WP ? PT / WP : 1;     // p tiles per wave
    constexpr int EV = 16 / (int)sizeof(T);         // elements per 16-byte piece
    constexpr int NBP = kKB * N / EV, NXP = kKB * P / EV;  // pieces of one step
    constexpr int PPT = (NBP + NXP + 255) / 256;    // pieces per thread
    typedef typename Vec8<T>::type V8;
    typedef typename Vec4<T>::type V4;
    typedef typename std::conditional<sizeof(T) == 2, V8, V4>::type VP;  // one 16-byte piece

    __shared__ __align__(16) T b_lds[2][kKB * LDB];
    __shared__ __align__(16) T x_lds[2][kKB * LDX];
    __shared__ float w_lds[256];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform across the wave
    const int H = p.nheads, Q = p.chunk, nc = p.nchunks, G = p.ngroups;
    const int64_t L = p.seqlen;

    // Workgroup -> (b, c, h).  Chunk states: heads sharing one (b, c) -- one
    // block of B -- run one after another on the same XCD (consecutive
    // workgroups are dealt round-robin over the 8 XCDs, each with its own L2).
    int h;
    int64_t b;
    int c, last;
    if (at_index) {
        h = blockIdx.y;
        b = blockIdx.z;
    } else {
        const int64_t per_xcd = gridDim.x / kXcds;
        const int64_t logical = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
        if (logical >= p.batch * nc * H) return;
        h = (int)(logical % H);
        c = (int)((logical / H) % nc);
        b = logical / ((int64_t)H * nc);
    }
    const int g = h / p.heads_per_group;

    if (at_index) {
        int j = p.state_out_idx[b];
        j = j < -1 ? -1 : (j > L - 1 ? (int)(L - 1) : j);
        if (j < 0) {  // nothing accepted: the state is the initial one, kept in hj by the state pass
            float *dst = p.state_out + (b * H + h) * (int64_t)P * N;
            const float *src = p.hj + (b * H + h) * (int64_t)P * N;
            for (int e = tid * 4; e < P * N; e += 256 * 4)
                *reinterpret_cast<f32x4 *>(dst + e) =
                    src ? *reinterpret_cast<const f32x4 *>(src + e) : f32x4{0.f, 0.f, 0.f, 0.f};
            return;
        }
        c = j / Q;
        last = j - c * Q;
    } else {
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

    const T *xg = reinterpret_cast<const T *>(p.x);
    const T *bg = reinterpret_cast<const T *>(p.B);
    const int wn = wave % WN, wp = wave / WN;
    const bool wave_active = wp * PTW < PT;

    f32x4 acc[NTW][PTW];
#pragma unroll
    for (int a = 0; a < NTW; ++a)
#pragma unroll
        for (int q = 0; q < PTW; ++q) acc[a][q] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One step = 32 token rows of B (NBP pieces) and of x (NXP pieces).  Rows
    // past the last counted token are read from that token instead (in
    // bounds, finite); their weight w is exactly zero.
    const T *bchunk = bg + ((b * L + t0) * G + g) * N;   // row j at bchunk + j*G*N
    const T *xchunk = xg + ((b * L + t0) * H + h) * P;   // row j at xchunk + j*H*P
    const int bstride = G * N, xstride = H * P;
    auto piece = [&](int u, int &row, int &col, bool &is_b) {
        const int q = tid + 256 * u;
        is_b = q < NBP;
        const int qq = is_b ? q : q - NBP;
        const int per_row = (is_b ? N : P) / EV;
        row = qq / per_row;
        col = EV * (qq - row * per_row);
    };
    auto load_step = [&](VP (&r)[PPT], int jb) {
#pragma unroll
        for (int u = 0; u < PPT; ++u) {
            if (tid + 256 * u >= NBP + NXP) continue;
            int row, col;
            bool is_b;
            piece(u, row, col, is_b);
            const int j = min(jb + row, ntok - 1);
            r[u] = is_b ? *reinterpret_cast<const VP *>(bchunk + j * bstride + col)
                        : *reinterpret_cast<const VP *>(xchunk + j * xstride + col);
        }
    };
    auto store_step = [&](const VP (&r)[PPT], int jb, int buf) {
#pragma unroll
        for (int u = 0; u < PPT; ++u) {
            if (tid + 256 * u >= NBP + NXP) continue;
            int row, col;
            bool is_b;
            piece(u, row, col, is_b);
            if (is_b) {
                *reinterpret_cast<VP *>(&b_lds[buf][row * LDB + col]) = r[u];
            } else {
                const float w = w_lds[jb + row];
                VP v;
#pragma unroll
                for (int e = 0; e < EV; ++e) v[e] = from_f32<T>(w * to_f32(r[u][e]));
                *reinterpret_cast<VP *>(&x_lds[buf][row * LDX + col]) = v;
            }
        }
    };
    auto compute = [&](int buf) {
        if (!wave_active) return;
        Frag<T> fa[NTW], fb[PTW];
#pragma unroll
        for (int a = 0; a < NTW; ++a) load_tr(fa[a], b_lds[buf], LDB, 0, 16, 16 * (wn + WN * a));
#pragma unroll
        for (int q = 0; q < PTW; ++q) load_tr(fb[q], x_lds[buf], LDX, 0, 16, 16 * (wp * PTW + q));
#pragma unroll
        for (int a = 0; a < NTW; ++a)
#pragma unroll
            for (int q = 0; q < PTW; ++q) mma(fa[a], fb[q], acc[a][q]);
    };

    VP ra[PPT], rb[PPT];
    load_step(ra, 0);
    if (kKB < ntok) load_step(rb, kKB);
    __syncthreads();  // w_lds ready
    for (int jb = 0; jb < ntok; jb += 2 * kKB) {
        store_step(ra, jb, 0);
        __syncthreads();
        if (jb + 2 * kKB < ntok) load_step(ra, jb + 2 * kKB);
        compute(0);
        if (jb + kKB >= ntok) break;
        store_step(rb, jb + kKB, 1);
        __syncthreads();
        if (jb + 3 * kKB < ntok) load_step(rb, jb + 3 * kKB);
        compute(1);
    }
    if (!wave_active) return;

    // acc[a][q][r] = S^T[n = 16*(wn + WN*a) + 4*grp + r][p = 16*(wp*PTW + q) + il]
    const int il = lane & 15, grp = lane >> 4;
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
                const int64_t at = ((b * H + h) * (int64_t)P + pp) * N + n;
                const f32x4 hp = *reinterpret_cast<const f32x4 *>(p.hj + at);
                v = v + e_last * hp;
                *reinterpret_cast<f32x4 *>(p.state_out + at) = v;
            } else {
                T *sd = reinterpret_cast<T *>(p.states) + state_base + (int64_t)pp * N + n;
                if constexpr (sizeof(T) == 2)
                    *reinterpret_cast<bf16x4 *>(sd) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
                else
                    *reinterpret_cast<f32x4 *>(sd) = v;
            }
        }
    }
}

template <typename T, int NT, int PT>
hipError_t launch_typed(const Params &p, bool at_index, hipStream_t stream) {
    dim3 grid(1, p.nheads, (unsigned)p.batch);
    if (!at_index) {
        const int64_t total = p.batch * p.nchunks * (int64_t)p.nheads;
        grid = dim3((unsigned)((total + kXcds - 1) / kXcds * kXcds));
    }
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
