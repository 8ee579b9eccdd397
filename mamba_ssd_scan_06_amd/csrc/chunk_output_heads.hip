// Chunk outputs, head-batched (bf16): the orange (diagonal block), blue
// (state-to-output) and D-skip terms of the SSD block decomposition for all
// heads of one B/C group in one workgroup.
//
// "Transformers are SSMs" article (cloud.tencent.com.cn), section "SSD算法":
// each diagonal block is a small semiseparable matrix that may be evaluated
// in any way, in particular in the attention-like quadratic form; the blue
// blocks are batched products with each chunk's true initial state.  For
// token i of chunk c, head h of group g, channel p:
//     y_i[p] = sum_{j<=i} exp(cs_i - cs_j) dt_j (C_i . B_j) x_j[p]      (orange)
//            + exp(cs_i) sum_n h_{c-1}[p][n] C_i[n]                     (blue)
//            + D_h x_i[p]
// The factor C_i . B_j does not depend on the head, only the decay and x do.
// Heads of one group (all heads when there is one group, the grouped-value
// heads of section "研究贡献") therefore share it: a workgroup owns
// (b, c, g, a slice of the group's heads), computes the causal tiles of
// G^T[j][i] = B_j . C_i once into registers (phase A), and then runs over its
// heads, each head only masking/scaling G^T and multiplying by x (phase B).
//
// Work split.  The chunk's 16-token column tiles ("i-tiles") are dealt to
// W = tiles/2 waves, wave w owning tiles w and tiles-1-w, so that every wave
// holds the same number of causal (i-tile, 32-token j block) pairs
// (tiles/2 + 1).  Per pair a wave keeps two 16x16 tiles of G^T, rounded to
// bf16 (nearest even) to fit the register budget; the decay-scaled value is
// rounded to bf16 once more as the second product's operand.
//
// Data movement (gfx950 direct global -> LDS copies, no register staging):
//  - phase A streams B through a ring of 32-token steps, several in flight;
//  - phase B double-buffers whole heads: while head k computes, head k+1's x
//    rows, bf16 initial state and per-token tables (cs, dt, dt_decay) land
//    in the other buffer.
// Tiles are stored unpadded with XOR swizzles so that the 16-byte-per-lane
// reads (B, h) and the transposing reads (x) are spread over all LDS banks.
//
// Decay factors: for a j block wholly before the i-tile,
//     exp(cs_i - cs_j) dt_j = exp(cs_i - cs_e) * dte_j,   e = last token of the block,
// with dte_j = dt_j exp(cs_e - cs_j) precomputed by the cumsum kernel (both
// factors <= 1); for the block holding the tile's diagonal the masked
// difference is exponentiated directly (mask before exp).
#include "device_common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

constexpr int kXcds = 8;
constexpr int kStep = 32;  // tokens per j block

template <int NT, int PT, int NIT>
struct HeadsCfg {
    static constexpr int N = NT * 16, P = PT * 16;
    static constexpr int KS = (N + 31) / 32, NP = KS * 32;
    static constexpr int WB = NP / 8, WX = P / 8;              // 16-byte pieces per B / h row, per x row
    static constexpr int W = NIT >= 2 ? NIT / 2 : 1;            // waves
    static constexpr int THREADS = 64 * W;
    static constexpr int MAXIT = NIT >= 2 ? 2 : 1;              // i-tiles per wave
    static constexpr int NPAIR = NIT >= 2 ? NIT / 2 + 1 : 1;    // (i-tile, j block) pairs per wave
    static constexpr int QP = NIT * 16 < kStep ? kStep : NIT * 16;  // token rows held per head
    static constexpr int XE = QP * P;                           // x elements per head buffer
    static constexpr int HE = P * NP;                           // initial-state elements per head buffer
    static constexpr int RSLOT = kStep * NP;                    // elements per B ring slot
    static constexpr int RING = XE >= 4 * RSLOT ? 4 : 2;        // B ring slots (phase A, in x buffer 1)
    static constexpr int X1E = XE > RING * RSLOT ? XE : RING * RSLOT;
    static constexpr int IXH = QP * WX / 64;                    // 1 KB copies per head: x rows
    static constexpr int IHH = P * WB / 64;                     //   initial-state rows
    static constexpr int IHEAD = IXH + IHH + 3;                 //   + cs, dt, dt_decay tables
    static constexpr int IHEAD_W = (IHEAD + W - 1) / W;
    static constexpr int IB = kStep * WB / 64;                  // 1 KB copies per B step
    static constexpr int IB_W = (IB + W - 1) / W;
    static constexpr size_t LDS_BYTES = (size_t)(XE + X1E + 2 * HE + 512) * 2 + 2 * 3 * 256 * 4;
};

template <int NT, int PT, int NIT>
__global__ __launch_bounds__(64 * (NIT >= 2 ? NIT / 2 : 1)) void chunk_output_heads_kernel(Params p, int hps,
                                                                                           int nslices) {
    using Cf = HeadsCfg<NT, PT, NIT>;
    using T = bf16;
    constexpr int N = Cf::N, P = Cf::P, KS = Cf::KS, NP = Cf::NP, WB = Cf::WB, WX = Cf::WX, W = Cf::W;
    constexpr int MAXIT = Cf::MAXIT, NPAIR = Cf::NPAIR, RING = Cf::RING;
    typedef typename Vec4<T>::type V4;

    __shared__ __align__(16) T xs[Cf::XE + Cf::X1E];  // head buffers 0 and 1; the B ring in buffer 1 during phase A
    T *const xs1 = xs + Cf::XE;
    __shared__ __align__(16) T hs[2][Cf::HE];
    __shared__ __align__(16) float tab[2][3][256];  // cs, dt, dt_decay of the buffered head
    __shared__ __align__(16) T junk[512];           // target of padding copies (never read)

    const int Q = p.chunk, H = p.nheads, G = p.ngroups, nc = p.nchunks, HPG = p.heads_per_group;
    const int64_t L = p.seqlen;

    // Workgroup -> (b, c, g, slice); slices of one (b, c) run back to back on one XCD.
    const int64_t total = p.batch * nc * G * nslices;
    const int64_t per_xcd = gridDim.x / kXcds;
    const int64_t logical = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (logical >= total) return;
    const int slice = (int)(logical % nslices);
    const int g = (int)((logical / nslices) % G);
    const int c = (int)((logical / ((int64_t)nslices * G)) % nc);
    const int64_t b = logical / ((int64_t)nslices * G * nc);
    const int hbeg = g * HPG + slice * hps;
    const int hcnt = min(hps, HPG - slice * hps);
    if (hcnt <= 0) return;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform across the wave
    const int il = lane & 15, grp = lane >> 4, sl = lane & 15;
    const int64_t t0 = (int64_t)c * Q;
    const int Qc = (int)(L - t0 < Q ? L - t0 : Q);
    const int nit = (Qc + 15) / 16;
    const bool has_prev = c > 0 || p.init_state != nullptr;

    int tile[MAXIT];
    tile[0] = wave;
    if constexpr (MAXIT == 2) tile[1] = NIT - 1 - wave;
    const int n0 = tile[0] / 2 + 1;  // pairs of tile 0; pairs n0.. belong to tile 1
    // pair u -> (slot k, j block m); wave-uniform
    auto pair_k = [&](int u) { return (MAXIT == 1 || u < n0) ? 0 : 1; };
    auto pair_m = [&](int u) { return u < n0 ? u : u - n0; };

    const T *xg = reinterpret_cast<const T *>(p.x);
    const T *bg = reinterpret_cast<const T *>(p.B);
    const T *cg = reinterpret_cast<const T *>(p.C);
    const T *h16 = reinterpret_cast<const T *>(p.prev);

    // ---- C_i fragments of the wave's tiles (register loads, once).
    Frag<T> cf[MAXIT][KS];
#pragma unroll
    for (int k = 0; k < MAXIT; ++k) {
        const int i = 16 * tile[k] + il;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int n0c = 32 * ks + 8 * grp;
            if (i < Qc && n0c < N)
                load8(cf[k][ks], cg + ((b * L + t0 + i) * G + g) * N + n0c);
            else
                cf[k][ks].zero();
        }
    }
    wait_vmcnt<0>();  // the copy pipelines below count only their own loads

    // ---- copies of one head into buffer `set`.  Token rows past the chunk
    // read its last token (in bounds, finite; their products meet an exact
    // zero); dstate 16 fills each 32-column state row with two copies.
    auto issue_head = [&](int hh, int set) {
        const int h = hbeg + hh;
        const T *xsrc = xg + ((b * L + t0) * H + h) * P;
        const T *hsrc = h16 + (((b * nc + c) * H + h) * (int64_t)P) * N;
        const int64_t trow = ((b * H + h) * nc + c) * (int64_t)Q;
        T *xdst = xs + set * Cf::XE;
#pragma unroll
        for (int u = 0; u < Cf::IHEAD_W; ++u) {
            const int ins = wave + W * u;
            if (ins < Cf::IXH) {
                const int U = 64 * ins + lane;
                const int row = U / WX, pos = U - row * WX;
                const int j = min(row, Qc - 1);
                copy16_to_lds(xsrc + (int64_t)j * H * P + 8 * (pos ^ swz_tr<WX>(row)), xdst + ins * 512);
            } else if (ins < Cf::IXH + Cf::IHH) {
                if (has_prev) {
                    const int U = 64 * (ins - Cf::IXH) + lane;
                    const int row = U / WB, pos = U - row * WB;
                    int gc = pos ^ swz_rows16<WB>(row);
                    if constexpr (NP != N) gc %= N / 8;
                    copy16_to_lds(hsrc + row * N + 8 * gc, &hs[set][(ins - Cf::IXH) * 512]);
                } else {
                    copy16_to_lds(xsrc, junk);
                }
            } else if (ins < Cf::IHEAD) {
                const int t = ins - Cf::IXH - Cf::IHH;
                const float *src = t == 0 ? p.cs : (t == 1 ? p.dtc : p.dte);
                copy16_to_lds(src + trow + 4 * min(lane, Q / 4 - 1), &tab[set][t][0]);
            } else {
                copy16_to_lds(xsrc, junk);
            }
        }
    };

    // ---- phase A: causal tiles of G^T = B C^T, B streamed through the ring.
    bf16x8 gt[NPAIR];  // slots 0-3: j tile 2m, slots 4-7: j tile 2m+1 (rows 4*grp + r)
#pragma unroll
    for (int u = 0; u < NPAIR; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) gt[u][e] = (bf16)0.f;

    const T *bsrc = bg + ((b * L + t0) * G + g) * N;
    auto issue_b = [&](int step, int slot) {
#pragma unroll
        for (int u = 0; u < Cf::IB_W; ++u) {
            const int ins = wave + W * u;
            if (ins < Cf::IB) {
                const int U = 64 * ins + lane;
                const int row = U / WB, pos = U - row * WB;
                int gc = pos ^ swz_rows16<WB>(row);
                if constexpr (NP != N) gc %= N / 8;
                const int j = min(kStep * step + row, Qc - 1);
                copy16_to_lds(bsrc + (int64_t)j * G * N + 8 * gc, xs1 + slot * Cf::RSLOT + ins * 512);
            } else {
                copy16_to_lds(bsrc, junk);
            }
        }
    };
    // Per-lane LDS offsets (elements).  Every swizzle here depends only on the
    // row modulo a period that divides 16 (rows16) or 8 (tr), so a fragment's
    // address is a per-lane constant plus a wave-uniform row offset.
    //  - 16-byte-per-lane reads (B ring, h): row 16*a + il, piece 4*ks + grp.
    int roff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) roff[ks] = il * NP + 8 * ((4 * ks + grp) ^ swz_rows16<WB>(il));
    //  - transposing reads of x: rows 32*m + 16*half + rl, columns 16*q + 4*(sl%4).
    const int rl = 4 * grp + (sl >> 2);
    int xoff[PT];
#pragma unroll
    for (int q = 0; q < PT; ++q) xoff[q] = rl * P + 16 * (q ^ (swz_tr<WX>(rl) >> 1)) + 4 * (sl & 3);
    //  - D x reads: row i = 16*t + il, columns 16*q + 4*grp .. +3.
    int dxoff[PT];
#pragma unroll
    for (int q = 0; q < PT; ++q)
        dxoff[q] = il * P + 8 * ((2 * q + (grp >> 1)) ^ swz_tr<WX>(il)) + 4 * (grp & 1);

    issue_head(0, 0);
    const int nstep = (Qc + kStep - 1) / kStep;
#pragma unroll
    for (int s = 0; s < RING - 1; ++s) issue_b(s, s);
    for (int s = 0; s < nstep; ++s) {
        wait_vmcnt<Cf::IB_W * (RING - 2)>();
        barrier_only();
        issue_b(s + RING - 1, (s + RING - 1) % RING);
        const T *ring = xs1 + (s % RING) * Cf::RSLOT;
        Frag<T> bfr[2][KS];
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) load8(bfr[half][ks], ring + 16 * half * NP + roff[ks]);
#pragma unroll
        for (int u = 0; u < NPAIR; ++u) {
            if (pair_m(u) != s) continue;
            auto body = [&](auto kc) {
                constexpr int K = decltype(kc)::value;
                const int t = tile[K];
                if (t >= nit) return;
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    if (2 * s + half > t) continue;  // above the diagonal
                    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) mma(bfr[half][ks], cf[K][ks], acc);
#pragma unroll
                    for (int r = 0; r < 4; ++r) gt[u][4 * half + r] = (bf16)acc[r];
                }
            };
            if (pair_k(u) == 0) body(std::integral_constant<int, 0>{});
            else if constexpr (MAXIT == 2) body(std::integral_constant<int, 1>{});
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // ---- phase B: heads.  Each wave waits for its own copies of head hh+1
    // before it stores head hh's outputs (vmcnt counts stores too, so a wait
    // placed after the stores would also wait for them to be written), and
    // the barrier at the top of the next iteration then covers every wave's
    // copies.
    T *yg = reinterpret_cast<T *>(p.y);
    wait_vmcnt<0>();  // head 0's copies (and any ring leftovers) have landed
    for (int hh = 0; hh < hcnt; ++hh) {
        const int set = hh & 1;
        barrier_only();  // head hh is in buffer `set` for every wave; the other buffer is no longer read
        if (hh + 1 < hcnt) issue_head(hh + 1, set ^ 1);

        const int h = hbeg + hh;
        const T *xsb = xs + set * Cf::XE;
        const T *hsb = hs[set];
        const float *csv = tab[set][0], *dtv = tab[set][1], *dtev = tab[set][2];

        f32x4 acc[MAXIT][PT];
#pragma unroll
        for (int k = 0; k < MAXIT; ++k)
#pragma unroll
            for (int q = 0; q < PT; ++q) acc[k][q] = f32x4{0.f, 0.f, 0.f, 0.f};

        // Blue: exp(cs_i) * (h_prev C_i^T), rows p, column i.
        if (has_prev) {
#pragma unroll
            for (int q = 0; q < PT; ++q) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    Frag<T> hf;
                    load8(hf, hsb + 16 * q * NP + roff[ks]);
#pragma unroll
                    for (int k = 0; k < MAXIT; ++k) mma(hf, cf[k][ks], acc[k][q]);
                }
            }
#pragma unroll
            for (int k = 0; k < MAXIT; ++k) {
                const int i = 16 * tile[k] + il;
                const float ei = i < Qc ? exp_neg(csv[i]) : 0.f;
#pragma unroll
                for (int q = 0; q < PT; ++q) acc[k][q] = acc[k][q] * ei;
            }
        }

        // Orange: per (tile, j block) pair, mask/scale G^T and multiply by x.
#pragma unroll
        for (int u = 0; u < NPAIR; ++u) {
            auto body = [&](auto kc) {
                constexpr int K = decltype(kc)::value;
                const int t = tile[K];
                if (t >= nit) return;
                const int m = pair_m(u);
                const int i = 16 * t + il;
                const float cs_i = csv[i];
                Frag<T> lf;
                if (kStep * m + kStep - 1 < 16 * t) {
                    // whole block before the tile: exp(cs_i - cs_e) * dte_j
                    const float ai = exp_neg(fminf(cs_i - csv[kStep * m + kStep - 1], 0.f));
                    const f32x4 d0 = *reinterpret_cast<const f32x4 *>(dtev + kStep * m + 4 * grp);
                    const f32x4 d1 = *reinterpret_cast<const f32x4 *>(dtev + kStep * m + 16 + 4 * grp);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        lf.set(r, (float)gt[u][r] * (ai * d0[r]));
                        lf.set(4 + r, (float)gt[u][4 + r] * (ai * d1[r]));
                    }
                } else {
                    // block holding the diagonal: mask (j <= i) before exp
                    const f32x4 c0 = *reinterpret_cast<const f32x4 *>(csv + kStep * m + 4 * grp);
                    const f32x4 c1 = *reinterpret_cast<const f32x4 *>(csv + kStep * m + 16 + 4 * grp);
                    const f32x4 t0v = *reinterpret_cast<const f32x4 *>(dtv + kStep * m + 4 * grp);
                    const f32x4 t1v = *reinterpret_cast<const f32x4 *>(dtv + kStep * m + 16 + 4 * grp);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j0 = kStep * m + 4 * grp + r, j1 = j0 + 16;
                        const float e0 = exp_neg(fminf(cs_i - c0[r], 0.f)) * t0v[r];
                        const float e1 = exp_neg(fminf(cs_i - c1[r], 0.f)) * t1v[r];
                        lf.set(r, j0 <= i ? (float)gt[u][r] * e0 : 0.f);
                        lf.set(4 + r, j1 <= i ? (float)gt[u][4 + r] * e1 : 0.f);
                    }
                }
                const T *xm = xsb + kStep * m * P;
#pragma unroll
                for (int q = 0; q < PT; ++q) {
                    const i16x4 a0 = ds_read_tr16(xm + xoff[q]);
                    const i16x4 a1 = ds_read_tr16(xm + 16 * P + xoff[q]);
                    typedef short i16x8 __attribute__((ext_vector_type(8)));
                    Frag<T> xf;
                    xf.v = __builtin_bit_cast(bf16x8, i16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]});
                    mma(xf, lf, acc[K][q]);
                }
            };
            if (pair_k(u) == 0) body(std::integral_constant<int, 0>{});
            else if constexpr (MAXIT == 2) body(std::integral_constant<int, 1>{});
            // Keep the scheduler from hoisting later pairs' LDS reads over this
            // one (their live ranges would exceed the register budget).
            __builtin_amdgcn_sched_barrier(0);
        }

        // + D x (x_i from the head's LDS rows), round to bf16, store.
        const float dh = p.D ? p.D[h] : 0.f;
        wait_vmcnt<0>();  // head hh+1's copies have landed (earlier stores are long done)
#pragma unroll
        for (int k = 0; k < MAXIT; ++k) {
            const int i = 16 * tile[k] + il;
            if (tile[k] >= nit || i >= Qc) continue;
            const int64_t row = ((b * L + t0 + i) * H + h) * (int64_t)P;
#pragma unroll
            for (int q = 0; q < PT; ++q) {
                const V4 xv = *reinterpret_cast<const V4 *>(xsb + 16 * tile[k] * P + dxoff[q]);
                V4 out;
#pragma unroll
                for (int r = 0; r < 4; ++r) out[r] = (T)(acc[k][q][r] + dh * (float)xv[r]);
                *reinterpret_cast<V4 *>(yg + row + 16 * q + 4 * grp) = out;
            }
        }
    }
    wait_vmcnt<0>();  // no copy outlives the workgroup
}

template <int NT, int PT, int NIT>
hipError_t launch_nit(const Params &p, hipStream_t stream) {
    using Cf = HeadsCfg<NT, PT, NIT>;
    if constexpr (Cf::LDS_BYTES > 160 * 1024) {
        return hipErrorNotSupported;
    } else {
        const int64_t base = p.batch * p.nchunks * (int64_t)p.ngroups;
        int nslices = (int)std::min<int64_t>(p.heads_per_group, std::max<int64_t>(1, (256 + base - 1) / base));
        const int hps = (p.heads_per_group + nslices - 1) / nslices;
        nslices = (p.heads_per_group + hps - 1) / hps;
        const int64_t total = base * nslices;
        const int64_t per_xcd = (total + kXcds - 1) / kXcds;
        hipLaunchKernelGGL((chunk_output_heads_kernel<NT, PT, NIT>), dim3((unsigned)(per_xcd * kXcds)),
                           dim3(Cf::THREADS), 0, stream, p, hps, nslices);
        return hipGetLastError();
    }
}

template <int NT, int PT>
hipError_t dispatch_q(const Params &p, hipStream_t stream) {
    switch (p.chunk) {
        case 8:
        case 16: return launch_nit<NT, PT, 1>(p, stream);
        case 32: return launch_nit<NT, PT, 2>(p, stream);
        case 64: return launch_nit<NT, PT, 4>(p, stream);
        case 128: return launch_nit<NT, PT, 8>(p, stream);
        case 256: return launch_nit<NT, PT, 16>(p, stream);
        default: return hipErrorNotSupported;
    }
}

template <int NT>
hipError_t dispatch_p(const Params &p, hipStream_t stream) {
    switch (p.headdim) {
        case 16: return dispatch_q<NT, 1>(p, stream);
        case 32: return dispatch_q<NT, 2>(p, stream);
        case 64: return dispatch_q<NT, 4>(p, stream);
        case 128: return dispatch_q<NT, 8>(p, stream);
        default: return hipErrorNotSupported;
    }
}

}  // namespace

hipError_t launch_chunk_output_heads(const Params &p, hipStream_t stream) {
    switch (p.dstate) {
        case 16: return dispatch_p<1>(p, stream);
        case 32: return dispatch_p<2>(p, stream);
        case 64: return dispatch_p<4>(p, stream);
        case 128: return dispatch_p<8>(p, stream);
        case 256: return dispatch_p<16>(p, stream);
        default: return hipErrorNotSupported;
    }
}

}  // namespace ssd
