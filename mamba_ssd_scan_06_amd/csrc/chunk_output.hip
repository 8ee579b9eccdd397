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
// Work split.  One workgroup covers one (b, c, h) chunk, or a slice of its
// 16-token column tiles ("i-tiles") when a wave would otherwise hold too many
// accumulators.  i-tiles are dealt to the workgroup's waves in a snake order
// (0..W-1, then W-1..0, ...) so that the causal work per wave is balanced.
// Workgroups are numbered so that the heads sharing one (b, c) -- and so one
// block of B and C -- run one after another on the same XCD (the hardware
// deals consecutive workgroups round-robin over the 8 XCDs, each with its own
// L2).
//
// Per wave, everything is computed transposed (rows p, columns i): the first
// product's output tile G^T[j][i] = B_j . C_i, masked and scaled, is exactly
// the B operand of the second product (a lane holds G^T[4*grp + r][il] of two
// 16-token j tiles = the 8 contraction slots of one fragment), and the x
// operand is read from its natural token-major LDS copy with the transposing
// LDS read, which yields the same token-to-slot assignment.  C_i fragments
// stay in registers for the whole chunk; tokens j stream through LDS 32 at a
// time (two buffers, global loads issued two steps ahead).  The decay mask is
// applied before the exponential (exp only of cs_i - cs_j with j <= i); tiles
// above the diagonal are skipped.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

constexpr int kJB = 32;     // tokens j per staging step
constexpr int kWaves = 4;   // waves per workgroup
constexpr int kXcds = 8;    // XCDs of an MI355X

template <typename T, int NT, int PT, int MAXIT>
__global__ __launch_bounds__(256) void chunk_output_kernel(Params p, int isplit) {
    constexpr int N = NT * 16, P = PT * 16;
    constexpr int KS = (N + 31) / 32;          // contraction steps over n
    constexpr int NP = KS * 32;                // n padded to whole steps
    constexpr int EV = 16 / (int)sizeof(T);    // elements per 16-byte piece
    constexpr int RSB = NP + EV;               // B block row stride   [j][n] (16-byte pad)
    constexpr int LDX = P + 2 * EV;            // x block row stride   [j][p] (32-byte pad)
    constexpr int RSH = NP + EV;               // h_prev row stride    [p][n]
    constexpr int NBP = kJB * NP / EV;         // 16-byte pieces of one B block
    constexpr int NXP = kJB * P / EV;          // ... of one x block
    constexpr int PPT = (NBP + NXP + 255) / 256;
    typedef typename Vec8<T>::type V8;
    typedef typename Vec4<T>::type V4;
    typedef typename std::conditional<sizeof(T) == 2, V8, V4>::type VP;  // one 16-byte piece

    __shared__ float cs_l[256];
    __shared__ float dt_l[256];
    __shared__ __align__(16) T b_lds[2][kJB * RSB];
    __shared__ __align__(16) T x_lds[2][kJB * LDX];
    __shared__ __align__(16) T h_lds[P * RSH];

    const int Q = p.chunk, H = p.nheads, G = p.ngroups, nc = p.nchunks;
    const int64_t L = p.seqlen;

    // Workgroup -> (b, c, h, slice): consecutive logical ids on one XCD.
    const int64_t total = p.batch * nc * H * isplit;
    const int64_t per_xcd = gridDim.x / kXcds;
    const int64_t logical = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (logical >= total) return;
    const int slice = (int)(logical % isplit);
    const int h = (int)((logical / isplit) % H);
    const int c = (int)((logical / ((int64_t)isplit * H)) % nc);
    const int64_t b = logical / ((int64_t)isplit * H * nc);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform across the wave
    const int il = lane & 15, grp = lane >> 4;
    const int g = h / p.heads_per_group;
    const int64_t t0 = (int64_t)c * Q;
    const int Qc = (int)(L - t0 < Q ? L - t0 : Q);
    const int nit = (Qc + 15) / 16;                 // valid i-tiles in this chunk
    const int W = kWaves * isplit;                  // waves sharing the chunk
    const int gw = slice * kWaves + wave;           // this wave among them

    // This wave's i-tiles (snake order) and the workgroup's causal extent.
    int tile[MAXIT];
    int jend = 0;                                   // tokens j any wave here needs
#pragma unroll
    for (int k = 0; k < MAXIT; ++k) {
        tile[k] = k * W + ((k & 1) ? W - 1 - gw : gw);
        for (int ww = 0; ww < kWaves; ++ww) {
            const int gww = slice * kWaves + ww;
            const int t = k * W + ((k & 1) ? W - 1 - gww : gww);
            if (t < nit) jend = max(jend, min(16 * t + 16, Qc));
        }
    }
    if (jend == 0) return;

    const float *csrow = p.cs + ((b * H + h) * nc + c) * (int64_t)Q;
    for (int i = tid; i < 256; i += 256) {
        cs_l[i] = i < Q ? csrow[i] : 0.f;
        dt_l[i] = i < Qc ? p.dt[(b * L + t0 + i) * H + h] : 0.f;
    }
    const bool has_prev = c > 0 || p.init_state != nullptr;
    if (has_prev) {
        const T *hp = reinterpret_cast<const T *>(p.prev) + ((b * nc + c) * H + h) * (int64_t)P * N;
        for (int q = tid; q < P * (NP / 8); q += 256) {
            const int pp = q / (NP / 8), n0 = 8 * (q - pp * (NP / 8));
            V8 v;
            if (n0 < N) {
                v = *reinterpret_cast<const V8 *>(hp + (int64_t)pp * N + n0);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = from_f32<T>(0.f);
            }
            *reinterpret_cast<V8 *>(&h_lds[pp * RSH + n0]) = v;
        }
    }

    const T *xg = reinterpret_cast<const T *>(p.x);
    const T *bg = reinterpret_cast<const T *>(p.B);
    const T *cg = reinterpret_cast<const T *>(p.C);

    // C_i fragments of this wave's tiles, one per contraction step over n.
    Frag<T> cf[MAXIT][KS];
#pragma unroll
    for (int k = 0; k < MAXIT; ++k) {
        const int i = 16 * tile[k] + il;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int n0 = 32 * ks + 8 * grp;
            if (i < Qc && n0 < N)
                load8(cf[k][ks], cg + ((b * L + t0 + i) * G + g) * N + n0);
            else
                cf[k][ks].zero();
        }
    }

    // One 32-token step: B rows (natural [j][n]) and x rows (natural [j][p]),
    // whole 16-byte pieces.  Rows past the chunk are read from its last token
    // instead (always in bounds and finite); every product they enter is
    // multiplied by an exact zero (dt = 0 past the end, or the causal mask).
    const T *bchunk = bg + ((b * L + t0) * G + g) * N;   // row j at bchunk + j*G*N
    const T *xchunk = xg + ((b * L + t0) * H + h) * P;   // row j at xchunk + j*H*P
    const int bstride = G * N, xstride = H * P;
    auto piece = [&](int u, int &row, int &col, bool &is_b) {
        const int q = tid + 256 * u;
        is_b = q < NBP;
        const int qq = is_b ? q : q - NBP;
        const int per_row = (is_b ? NP : P) / EV;
        row = qq / per_row;
        col = EV * (qq - row * per_row);
    };
    auto load_step = [&](VP (&r)[PPT], int js) {
#pragma unroll
        for (int u = 0; u < PPT; ++u) {
            if (tid + 256 * u >= NBP + NXP) continue;
            int row, col;
            bool is_b;
            piece(u, row, col, is_b);
            const int j = min(js + row, Qc - 1);
            if constexpr (NP != N) {  // dstate 16: the contraction step is half padding
                if (is_b && col >= N) {
#pragma unroll
                    for (int e = 0; e < EV; ++e) r[u][e] = from_f32<T>(0.f);
                    continue;
                }
            }
            r[u] = is_b ? *reinterpret_cast<const VP *>(bchunk + j * bstride + col)
                        : *reinterpret_cast<const VP *>(xchunk + j * xstride + col);
        }
    };
    auto store_step = [&](const VP (&r)[PPT], int buf) {
#pragma unroll
        for (int u = 0; u < PPT; ++u) {
            if (tid + 256 * u >= NBP + NXP) continue;
            int row, col;
            bool is_b;
            piece(u, row, col, is_b);
            T *dst = is_b ? &b_lds[buf][row * RSB + col] : &x_lds[buf][row * LDX + col];
            *reinterpret_cast<VP *>(dst) = r[u];
        }
    };

    f32x4 acc[MAXIT][PT];
#pragma unroll
    for (int k = 0; k < MAXIT; ++k)
#pragma unroll
        for (int q = 0; q < PT; ++q) acc[k][q] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Orange for one 32-token step js (tokens j = js .. js+31 in LDS buffer buf).
    // A lane's 8 slots stand for j = js + 4*grp + (s & 3) + 16*(s >> 2).
    // Tiles strictly after the step use exp(cs_i - cs_j) =
    // exp(cs_i - cs_ref) * exp(cs_ref - cs_j) with cs_ref at the step's last
    // token, both factors <= 1; tiles the step overlaps take the exponential
    // of the masked difference directly.  All selects are branch-free.
    auto compute = [&](int buf, int js) {
        Frag<T> bf0[KS], bf1[KS], xf[PT];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            load8(bf0[ks], &b_lds[buf][il * RSB + 32 * ks + 8 * grp]);
            load8(bf1[ks], &b_lds[buf][(16 + il) * RSB + 32 * ks + 8 * grp]);
        }
#pragma unroll
        for (int q = 0; q < PT; ++q) load_tr(xf[q], x_lds[buf], LDX, 0, 16, 16 * q);
        const float cs_ref = cs_l[min(js + kJB, Qc) - 1];
        float csj[8], dtj[8], ej[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int j = js + 4 * grp + (s & 3) + 16 * (s >> 2);   // < 256
            csj[s] = cs_l[j];
            dtj[s] = dt_l[j];                                         // 0 past the chunk
            ej[s] = exp_neg(fminf(cs_ref - csj[s], 0.f)) * dtj[s];
        }
#pragma unroll
        for (int k = 0; k < MAXIT; ++k) {
            const int ti = tile[k];
            if (ti >= nit || js > 16 * ti + 15) continue;
            const int i = 16 * ti + il;
            const float cs_i = cs_l[min(i, 255)];
            const bool after = 16 * ti >= js + kJB;   // whole tile after the step
            const bool need1 = js + 16 <= 16 * ti + 15;
            f32x4 g0 = f32x4{0.f, 0.f, 0.f, 0.f}, g1 = g0;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) mma(bf0[ks], cf[k][ks], g0);
            if (need1) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) mma(bf1[ks], cf[k][ks], g1);
            }
            Frag<T> lf;
            if (after) {
                const float ei = exp_neg(fminf(cs_i - cs_ref, 0.f));
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    lf.set(r, g0[r] * (ei * ej[r]));
                    lf.set(4 + r, g1[r] * (ei * ej[4 + r]));
                }
            } else {
                // Mask (j <= i) before exp, scale by the decay and dt_j, round once.
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const int j = js + 4 * grp + (s & 3) + 16 * (s >> 2);
                    const float e = exp_neg(fminf(cs_i - csj[s], 0.f)) * dtj[s];
                    const float gv = s < 4 ? g0[s] : g1[s - 4];
                    lf.set(s, j <= i ? gv * e : 0.f);
                }
            }
#pragma unroll
            for (int q = 0; q < PT; ++q) mma(xf[q], lf, acc[k][q]);
        }
    };

    // Everything loaded so far (cs, dt, h_prev, C fragments) is complete
    // before the staging pipeline starts, so that inside the pipeline only
    // the step loads are outstanding and each wait covers exactly one step.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // cs_l, dt_l, h_lds ready
    VP rbuf[2][PPT];
    load_step(rbuf[0], 0);
    load_step(rbuf[1], kJB);  // rows are clamped: always in bounds, even past jend

    // Blue: exp(cs_i) * (h_prev C_i^T), rows p, column i.
    if (has_prev) {
#pragma unroll
        for (int k = 0; k < MAXIT; ++k) {
            if (tile[k] >= nit) continue;
#pragma unroll
            for (int q = 0; q < PT; ++q) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    Frag<T> a;
                    load8(a, &h_lds[(16 * q + il) * RSH + 32 * ks + 8 * grp]);
                    mma(a, cf[k][ks], acc[k][q]);
                }
            }
            const int i = 16 * tile[k] + il;
            const float ei = i < Qc ? exp_neg(cs_l[i]) : 0.f;
#pragma unroll
            for (int q = 0; q < PT; ++q) acc[k][q] = acc[k][q] * ei;
        }
    }

    // Orange: two LDS buffers, global loads issued two steps ahead.
    // The step loop is unrolled (a chunk has at most 256 / 32 steps) and its
    // loads are issued unconditionally (clamped rows), so that every wait
    // before a step's LDS store covers exactly that step's loads while the
    // next step's stay in flight.
#pragma unroll
    for (int st = 0; st < 256 / kJB; ++st) {
        const int js = st * kJB;
        if (js >= jend) break;
        store_step(rbuf[st & 1], st & 1);
        __syncthreads();
        load_step(rbuf[st & 1], js + 2 * kJB);
        compute(st & 1, js);
    }

    // Epilogue: + D x, round to the output type; lane holds p = 16q + 4grp + r of token i.
    const float dh = p.D ? p.D[h] : 0.f;
    T *yg = reinterpret_cast<T *>(p.y);
#pragma unroll
    for (int k = 0; k < MAXIT; ++k) {
        const int i = 16 * tile[k] + il;
        if (tile[k] >= nit || i >= Qc) continue;
        const int64_t row = ((b * L + t0 + i) * H + h) * (int64_t)P;
#pragma unroll
        for (int q = 0; q < PT; ++q) {
            const int p0 = 16 * q + 4 * grp;
            const V4 xv = *reinterpret_cast<const V4 *>(xg + row + p0);
            V4 out;
#pragma unroll
            for (int r = 0; r < 4; ++r) out[r] = from_f32<T>(acc[k][q][r] + dh * to_f32(xv[r]));
            *reinterpret_cast<V4 *>(yg + row + p0) = out;
        }
    }
}


// ---------------------------------------------------------------------------
// bf16 variant with a direct-to-LDS copy pipeline.
//
// Same computation and work split as chunk_output_kernel.  The 32-token steps
// of B and x are copied global -> LDS with global_load_lds_dwordx4 into a ring
// of NSTAGE buffers, NSTAGE-1 steps ahead, so several steps of loads are in
// flight without holding registers.  Tiles are stored unpadded with an XOR
// swizzle of their 16-byte pieces (the copying lane picks the global piece
// that belongs to its LDS slot): B rows are read 16 bytes per lane, 16 rows
// at a time, and x rows through the transposing read, 4 rows x 32 bytes per
// 16 lanes; the swizzles spread both patterns over all LDS banks.
// ---------------------------------------------------------------------------

template <int NT, int PT, int MAXIT, int NSTAGE>
__global__ __launch_bounds__(256) void chunk_output_dma_kernel(Params p, int isplit) {
    using T = bf16;
    constexpr int N = NT * 16, P = PT * 16;
    constexpr int KS = (N + 31) / 32;          // contraction steps over n
    constexpr int NP = KS * 32;                // n padded to whole steps
    constexpr int WB = NP / 8, WX = P / 8;     // 16-byte pieces per B / x row
    constexpr int IB = kJB * WB / 64, IX = kJB * WX / 64;   // 1 KB copies per step
    constexpr int IPW = (IB + IX + kWaves - 1) / kWaves;    // copies per wave per step
    constexpr int RSH = NP + 8;                // h_prev row stride [p][n]
    typedef typename Vec8<T>::type V8;
    typedef typename Vec4<T>::type V4;
    static_assert(IB * 64 == kJB * WB && IX * 64 == kJB * WX, "whole 1 KB copies");

    __shared__ float cs_l[256];
    __shared__ float dt_l[256];
    __shared__ __align__(16) T b_st[NSTAGE][kJB * NP];
    __shared__ __align__(16) T x_st[NSTAGE][kJB * P];
    __shared__ __align__(16) T h_lds[P * RSH];
    __shared__ __align__(16) T junk[512];       // target of padding copies (never read)

    const int Q = p.chunk, H = p.nheads, G = p.ngroups, nc = p.nchunks;
    const int64_t L = p.seqlen;

    const int64_t total = p.batch * nc * H * isplit;
    const int64_t per_xcd = gridDim.x / kXcds;
    const int64_t logical = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (logical >= total) return;
    const int slice = (int)(logical % isplit);
    const int h = (int)((logical / isplit) % H);
    const int c = (int)((logical / ((int64_t)isplit * H)) % nc);
    const int64_t b = logical / ((int64_t)isplit * H * nc);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform across the wave
    const int il = lane & 15, grp = lane >> 4;
    const int g = h / p.heads_per_group;
    const int64_t t0 = (int64_t)c * Q;
    const int Qc = (int)(L - t0 < Q ? L - t0 : Q);
    const int nit = (Qc + 15) / 16;
    const int W = kWaves * isplit;
    const int gw = slice * kWaves + wave;

    int tile[MAXIT];
    int jend = 0;
#pragma unroll
    for (int k = 0; k < MAXIT; ++k) {
        tile[k] = k * W + ((k & 1) ? W - 1 - gw : gw);
        for (int ww = 0; ww < kWaves; ++ww) {
            const int gww = slice * kWaves + ww;
            const int t = k * W + ((k & 1) ? W - 1 - gww : gww);
            if (t < nit) jend = max(jend, min(16 * t + 16, Qc));
        }
    }
    if (jend == 0) return;

    // ---- per-chunk loads through registers: cs, dt, h_prev (-> bf16), C_i.
    const float *csrow = p.cs + ((b * H + h) * nc + c) * (int64_t)Q;
    for (int i = tid; i < 256; i += 256) {
        cs_l[i] = i < Q ? csrow[i] : 0.f;
        dt_l[i] = i < Qc ? p.dt[(b * L + t0 + i) * H + h] : 0.f;
    }
    const bool has_prev = c > 0 || p.init_state != nullptr;
    if (has_prev) {
        const T *hp = reinterpret_cast<const T *>(p.prev) + ((b * nc + c) * H + h) * (int64_t)P * N;
        for (int q = tid; q < P * (NP / 8); q += 256) {
            const int pp = q / (NP / 8), n0 = 8 * (q - pp * (NP / 8));
            V8 v;
            if (n0 < N) {
                v = *reinterpret_cast<const V8 *>(hp + (int64_t)pp * N + n0);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = (T)0.f;
            }
            *reinterpret_cast<V8 *>(&h_lds[pp * RSH + n0]) = v;
        }
    }
    const T *xg = reinterpret_cast<const T *>(p.x);
    const T *bg = reinterpret_cast<const T *>(p.B);
    const T *cg = reinterpret_cast<const T *>(p.C);
    Frag<T> cf[MAXIT][KS];
#pragma unroll
    for (int k = 0; k < MAXIT; ++k) {
        const int i = 16 * tile[k] + il;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int n0 = 32 * ks + 8 * grp;
            if (i < Qc && n0 < N)
                load8(cf[k][ks], cg + ((b * L + t0 + i) * G + g) * N + n0);
            else
                cf[k][ks].zero();
        }
    }
    // The copy pipeline below counts only its own loads.
    wait_vmcnt<0>();

    // ---- copy issue for one step: rows past the chunk read its last token
    // (in bounds, finite; every product they enter is multiplied by an exact
    // zero).  dstate 16 pads each B row to 32 columns with a second copy of
    // the row (C is zero there).
    const T *bchunk = bg + ((b * L + t0) * G + g) * N;
    const T *xchunk = xg + ((b * L + t0) * H + h) * P;
    const int bstride = G * N, xstride = H * P;
    auto issue = [&](int js, int stage) {
#pragma unroll
        for (int u = 0; u < IPW; ++u) {
            const int ins = wave + kWaves * u;
            if (ins < IB) {
                const int U = 64 * ins + lane;
                const int row = U / WB, pos = U - row * WB;
                int gc = pos ^ swz_rows16<WB>(row);
                if constexpr (NP != N) gc %= N / 8;
                const int j = min(js + row, Qc - 1);
                copy16_to_lds(bchunk + j * bstride + 8 * gc, &b_st[stage][ins * 512]);
            } else if (ins < IB + IX) {
                const int U = 64 * (ins - IB) + lane;
                const int row = U / WX, pos = U - row * WX;
                const int gc = pos ^ swz_tr<WX>(row);
                const int j = min(js + row, Qc - 1);
                copy16_to_lds(xchunk + j * xstride + 8 * gc, &x_st[stage][(ins - IB) * 512]);
            } else {
                copy16_to_lds(bchunk, junk);
            }
        }
    };

    // ---- per-lane LDS offsets of the fragments (elements within a stage).
    int boff[2][KS];
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
        const int r = 16 * jt + il;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) boff[jt][ks] = r * NP + 8 * ((4 * ks + grp) ^ swz_rows16<WB>(r));
    }
    int xoff[2][PT];
    {
        const int s = lane & 15;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int r = 16 * kk + 4 * grp + (s >> 2);
#pragma unroll
            for (int q = 0; q < PT; ++q) {
                const int col = 16 * q + 4 * (s & 3);
                xoff[kk][q] = r * P + 8 * ((col >> 3) ^ swz_tr<WX>(r)) + (col & 7);
            }
        }
    }

    f32x4 acc[MAXIT][PT];
#pragma unroll
    for (int k = 0; k < MAXIT; ++k)
#pragma unroll
        for (int q = 0; q < PT; ++q) acc[k][q] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int stage, int js) {
        const T *bs = b_st[stage];
        const T *xs = x_st[stage];
        Frag<T> bf0[KS], bf1[KS], xf[PT];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            load8(bf0[ks], bs + boff[0][ks]);
            load8(bf1[ks], bs + boff[1][ks]);
        }
#pragma unroll
        for (int q = 0; q < PT; ++q) {
            const i16x4 a = ds_read_tr16(xs + xoff[0][q]);
            const i16x4 bq = ds_read_tr16(xs + xoff[1][q]);
            typedef short i16x8 __attribute__((ext_vector_type(8)));
            xf[q].v = __builtin_bit_cast(bf16x8, i16x8{a[0], a[1], a[2], a[3], bq[0], bq[1], bq[2], bq[3]});
        }
        const float cs_ref = cs_l[min(js + kJB, Qc) - 1];
        float csj[8], dtj[8], ej[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int j = js + 4 * grp + (s & 3) + 16 * (s >> 2);
            csj[s] = cs_l[j];
            dtj[s] = dt_l[j];
            ej[s] = exp_neg(fminf(cs_ref - csj[s], 0.f)) * dtj[s];
        }
#pragma unroll
        for (int k = 0; k < MAXIT; ++k) {
            const int ti = tile[k];
            if (ti >= nit || js > 16 * ti + 15) continue;
            const int i = 16 * ti + il;
            const float cs_i = cs_l[min(i, 255)];
            const bool after = 16 * ti >= js + kJB;
            const bool need1 = js + 16 <= 16 * ti + 15;
            f32x4 g0 = f32x4{0.f, 0.f, 0.f, 0.f}, g1 = g0;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) mma(bf0[ks], cf[k][ks], g0);
            if (need1) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) mma(bf1[ks], cf[k][ks], g1);
            }
            Frag<T> lf;
            if (after) {
                const float ei = exp_neg(fminf(cs_i - cs_ref, 0.f));
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    lf.set(r, g0[r] * (ei * ej[r]));
                    lf.set(4 + r, g1[r] * (ei * ej[4 + r]));
                }
            } else {
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const int j = js + 4 * grp + (s & 3) + 16 * (s >> 2);
                    const float e = exp_neg(fminf(cs_i - csj[s], 0.f)) * dtj[s];
                    const float gv = s < 4 ? g0[s] : g1[s - 4];
                    lf.set(s, j <= i ? gv * e : 0.f);
                }
            }
#pragma unroll
            for (int q = 0; q < PT; ++q) mma(xf[q], lf, acc[k][q]);
        }
    };

    // ---- pipeline prologue, then the blue term while the copies land.
#pragma unroll
    for (int s = 0; s < NSTAGE - 1; ++s) issue(s * kJB, s);
    lds_barrier();  // cs_l, dt_l, h_lds visible; the copies keep flying

    if (has_prev) {
#pragma unroll
        for (int k = 0; k < MAXIT; ++k) {
            if (tile[k] >= nit) continue;
#pragma unroll
            for (int q = 0; q < PT; ++q) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    Frag<T> a;
                    load8(a, &h_lds[(16 * q + il) * RSH + 32 * ks + 8 * grp]);
                    mma(a, cf[k][ks], acc[k][q]);
                }
            }
            const int i = 16 * tile[k] + il;
            const float ei = i < Qc ? exp_neg(cs_l[i]) : 0.f;
#pragma unroll
            for (int q = 0; q < PT; ++q) acc[k][q] = acc[k][q] * ei;
        }
    }

    // ---- orange: wait for step st, then refill the buffer step st-1 used.
    const int nsteps = (jend + kJB - 1) / kJB;
    for (int st = 0; st < nsteps; ++st) {
        wait_vmcnt<IPW * (NSTAGE - 2)>();
        barrier_only();
        issue((st + NSTAGE - 1) * kJB, (st + NSTAGE - 1) % NSTAGE);
        compute(st % NSTAGE, st * kJB);
    }
    wait_vmcnt<0>();  // no copy may outlive the workgroup's use of LDS

    // Epilogue: + D x, round to bf16; lane holds p = 16q + 4grp + r of token i.
    // All x values are loaded before any y is stored (x and y may not be
    // assumed disjoint by the compiler, which would otherwise serialise them).
    const float dh = p.D ? p.D[h] : 0.f;
    T *yg = reinterpret_cast<T *>(p.y);
    V4 xv[MAXIT][PT];
#pragma unroll
    for (int k = 0; k < MAXIT; ++k) {
        const int i = min(16 * tile[k] + il, Qc - 1);
        const int64_t row = ((b * L + t0 + i) * H + h) * (int64_t)P;
#pragma unroll
        for (int q = 0; q < PT; ++q) xv[k][q] = *reinterpret_cast<const V4 *>(xg + row + 16 * q + 4 * grp);
    }
#pragma unroll
    for (int k = 0; k < MAXIT; ++k) {
        const int i = 16 * tile[k] + il;
        if (tile[k] >= nit || i >= Qc) continue;
        const int64_t row = ((b * L + t0 + i) * H + h) * (int64_t)P;
#pragma unroll
        for (int q = 0; q < PT; ++q) {
            V4 out;
#pragma unroll
            for (int r = 0; r < 4; ++r) out[r] = (T)(acc[k][q][r] + dh * (float)xv[k][q][r]);
            *reinterpret_cast<V4 *>(yg + row + 16 * q + 4 * grp) = out;
        }
    }
}

// Accumulator tiles per wave: bf16 keeps up to 4 i-tiles per wave (a whole
// 256-token chunk per workgroup); fp32 fragments are twice as wide, so fp32
// keeps one and spreads a chunk over several workgroups.
template <typename T>
constexpr int max_tiles_per_wave() { return sizeof(T) == 2 ? 4 : 1; }

template <typename T, int NT, int PT, int MAXIT>
hipError_t launch_typed(const Params &p, hipStream_t stream) {
    const int nit = (p.chunk + 15) / 16;
    const int isplit = (nit + kWaves * MAXIT - 1) / (kWaves * MAXIT);
    const int64_t total = p.batch * p.nchunks * (int64_t)p.nheads * isplit;
    const int64_t per_xcd = (total + kXcds - 1) / kXcds;
    const dim3 grid((unsigned)(per_xcd * kXcds));
    if constexpr (sizeof(T) == 2) {
        constexpr int kStages = (NT * 16 + 31) / 32 * 32 + PT * 16 <= 192 ? 4 : 3;
        hipLaunchKernelGGL((chunk_output_dma_kernel<NT, PT, MAXIT, kStages>), grid, dim3(256), 0, stream, p, isplit);
    } else {
        hipLaunchKernelGGL((chunk_output_kernel<T, NT, PT, MAXIT>), grid, dim3(256), 0, stream, p, isplit);
    }
    return hipGetLastError();
}

template <typename T, int NT, int PT>
hipError_t dispatch_tiles(const Params &p, hipStream_t stream) {
    constexpr int cap = max_tiles_per_wave<T>();
    const int nit = (p.chunk + 15) / 16;
    const int need = (nit + kWaves - 1) / kWaves;  // tiles per wave with one workgroup per chunk
    if (need <= 1 || cap == 1) return launch_typed<T, NT, PT, 1>(p, stream);
    if constexpr (cap >= 2) {
        if (need <= 2) return launch_typed<T, NT, PT, 2>(p, stream);
    }
    if constexpr (cap >= 4) return launch_typed<T, NT, PT, 4>(p, stream);
    return hipErrorInvalidValue;
}

template <typename T, int NT>
hipError_t dispatch_p(const Params &p, hipStream_t stream) {
    switch (p.headdim) {
        case 16: return dispatch_tiles<T, NT, 1>(p, stream);
        case 32: return dispatch_tiles<T, NT, 2>(p, stream);
        case 64: return dispatch_tiles<T, NT, 4>(p, stream);
        case 128:
            if constexpr (sizeof(T) == 4 && NT * 8 > 64) {
                return hipErrorInvalidValue;  // fp32 state tile beyond the LDS budget (rejected by the host checks)
            } else {
                return dispatch_tiles<T, NT, 8>(p, stream);
            }
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
