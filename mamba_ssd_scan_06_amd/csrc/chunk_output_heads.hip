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
// heads, each head only scaling G^T and multiplying by x (phase B).
//
// Channels.  The rows p of the state are independent, so a workgroup may
// own P of a head's channels (x, y and the state rows of that slice); the
// head's G^T is then formed once per channel slice.  dstate 256 with
// 256-token chunks runs 32-channel slices in the one-tile-per-wave layout:
// two buffers of a 32-channel head fit in LDS next to the B ring, and 16
// waves share the compute unit instead of the 8 of the two-tile layout.
//
// Work split.  The chunk's 16-token column tiles ("i-tiles") are dealt to
// W = tiles/2 waves, wave w owning tiles w and tiles-1-w, so every wave holds
// the same number of causal (i-tile, 32-token j block) pairs.  Tile t meets
// the j blocks m < t/2 wholly before it ("off-diagonal") and block t/2, which
// holds its diagonal.  A wave walks the j blocks once per head: each block's
// x^T fragments are read from LDS once and feed the pairs of both its tiles.
// The G^T values of a pair are kept in registers rounded to bf16 (nearest
// even); the decay-scaled value is rounded to bf16 once more as the second
// product's operand.
//
// Decay factors (per head, from the cumsum tables):
//  - off-diagonal block m, e = its last token:
//        exp(cs_i - cs_j) dt_j = exp2(cs2_i - cs2_e) * dte_j,
//    with cs2 = cs * log2(e) and dte_j = dt_j exp(cs_e - cs_j) (both factors <= 1);
//  - diagonal block: exp(cs_i - cs_j) dt_j = exp2(cs2_i - ct_j),
//    ct_j = cs2_j - log2(dt_j) (+inf where dt = 0); the causal mask j <= i is
//    applied to the block's G^T values once, in phase A.
//
// Data movement:
//  - phase A reads B fragments straight from global memory (L2);
//  - phase B (gfx950 direct global -> LDS copies, no register staging) keeps whole heads in three buffers (two where LDS is short):
//    while head k computes, the copies of head k+2 (x rows, bf16 initial
//    state, per-token tables cs, ct, dte) are in flight and head k+1's have
//    landed.  Each wave waits for its own copies of head k+1 before it stores
//    head k's outputs (vmcnt counts stores too, so a wait after the stores
//    would also wait for them to be written); the barrier that opens the
//    next head then covers every wave's copies.
// Tiles are stored unpadded with XOR swizzles of their 16-byte pieces so that
// the 16-byte-per-lane reads of h and the transposing reads of x (four rows
// of 32 bytes per 16 lanes) use all LDS banks.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

constexpr int kXcds = 8;
constexpr int kStep = 32;  // tokens per j block

// Piece swizzle of an x row of W 16-byte pieces for the transposing reads
// (per 16 lanes: four rows, one 32-byte column pair each).
template <int W>
__device__ __forceinline__ int xsw(int r) {
    return swz_tr<W>(r);
}

// WIDE: one i-tile per wave (NIT waves, at most 128 VGPRs, so four waves
// share a SIMD); otherwise two tiles per wave (NIT/2 waves).
template <int NT, int PT, int NIT, bool WIDE>
struct HeadsCfg {
    static constexpr int N = NT * 16, P = PT * 16;
    static constexpr int KS = (N + 31) / 32, NP = KS * 32;
    static constexpr int WB = NP / 8, WX = P / 8;              // 16-byte pieces per h row, per x row
    static constexpr int W = WIDE ? NIT : (NIT >= 2 ? NIT / 2 : 1);  // waves
    static constexpr int THREADS = 64 * W;
    static constexpr int MAXIT = !WIDE && NIT >= 2 ? 2 : 1;     // i-tiles per wave
    static constexpr int NBLK = NIT >= 2 ? NIT / 2 : 1;         // j blocks a wave visits at most
    static constexpr int S0 = WIDE ? (NIT >= 2 ? NIT / 2 - 1 : 0)       // off-diagonal blocks of tile 0, at most
                                   : (NIT >= 4 ? (W - 1) / 2 : 0);
    static constexpr int S1 = !WIDE && NIT >= 2 ? W - 1 : 0;    //   of tile 1, at most
    static constexpr int U1 = !WIDE && NIT >= 4 ? W / 2 : 0;    //   of tile 1, at least
    static constexpr int QP = NIT * 16 < kStep ? kStep : NIT * 16;  // token rows held per head
    static constexpr int XE = QP * P;                           // x elements per head buffer
    static constexpr int HE = P * NP;                           // initial-state elements per head buffer
    static constexpr int IXH = QP * WX / 64;                    // 1 KB copies per head: x rows
    static constexpr int IHH = P * WB / 64;                     //   initial-state rows
    static constexpr int UX = (IXH + W - 1) / W;                // copies per wave per head: x
    static constexpr int UH = (IHH + W - 1) / W;                //   initial state
    static constexpr int UT = (3 + W - 1) / W;                  //   tables
    // Phase A of the one-tile layout streams B through a ring of RING
    // 32-token slots (IB 1 KB copies per slot).
    static constexpr int RSLOT = kStep * NP, RING = 4;
    static constexpr int IB = kStep * WB / 64;
    static constexpr int IB_W = (IB + W - 1) / W;
    static constexpr size_t lds_bytes(int nbuf) {
        return (size_t)nbuf * ((XE + HE) * 2 + 3 * 256 * 4) + 512 * 2 + (WIDE ? (size_t)RING * RSLOT * 2 : 0);
    }
    // Head buffers: three (copies run two heads ahead) when they fit in LDS
    // and one head's copies per wave fit the vmcnt counter.
    // (The one-tile-per-wave layout hides latency with four waves per SIMD
    // and keeps two buffers: fewer per-buffer address registers.)
    static constexpr int NBUF = !WIDE && lds_bytes(3) <= 160 * 1024 && UX + UH + UT < 64 ? 3 : 2;
    static constexpr size_t LDS_BYTES = lds_bytes(NBUF);
};

template <int NT, int PT, int NIT, bool WIDE>
__global__ __launch_bounds__(WIDE ? 64 * NIT : 64 * (NIT >= 2 ? NIT / 2 : 1)) void chunk_output_heads_kernel(Params p, int hps,
                                                                                                  int nslices,
                                                                                                  int csplit) {
    using Cf = HeadsCfg<NT, PT, NIT, WIDE>;
    using T = bf16;
    constexpr int N = Cf::N, P = Cf::P, KS = Cf::KS, NP = Cf::NP, WB = Cf::WB, WX = Cf::WX, W = Cf::W;
    constexpr int MAXIT = Cf::MAXIT, NBLK = Cf::NBLK, S0 = Cf::S0, S1 = Cf::S1, U1 = Cf::U1;
    constexpr int NBUF = Cf::NBUF, XE = Cf::XE, HE = Cf::HE;
    typedef typename Vec4<T>::type V4;

    // Head buffers, one LDS object each: accesses to different objects carry
    // different alias scopes, so reading one buffer while copies into another
    // are in flight needs no wait for those copies.
    __shared__ __align__(16) T xb0[XE], xb1[XE], xb2[NBUF == 3 ? XE : 8];
    __shared__ __align__(16) T hb0[HE], hb1[HE], hb2[NBUF == 3 ? HE : 8];
    __shared__ __align__(16) float tb0[3 * 256], tb1[3 * 256], tb2[NBUF == 3 ? 3 * 256 : 4];  // cs, ct, dte
    __shared__ __align__(16) T junk[512];  // target of padding copies (never read)
    // B ring of phase A (one-tile layout), one LDS object per slot.
    __shared__ __align__(16) T rg0[WIDE ? Cf::RSLOT : 8], rg1[WIDE ? Cf::RSLOT : 8], rg2[WIDE ? Cf::RSLOT : 8],
        rg3[WIDE ? Cf::RSLOT : 8];
    auto ring = [&](auto sc) __attribute__((always_inline)) -> T * {
        constexpr int k = decltype(sc)::value % Cf::RING;
        if constexpr (k == 0) return rg0;
        else if constexpr (k == 1) return rg1;
        else if constexpr (k == 2) return rg2;
        else return rg3;
    };
    auto xbuf = [&](auto bc) __attribute__((always_inline)) -> T * {
        if constexpr (decltype(bc)::value == 0) return xb0;
        else if constexpr (decltype(bc)::value == 1) return xb1;
        else return xb2;
    };
    auto hbuf = [&](auto bc) __attribute__((always_inline)) -> T * {
        if constexpr (decltype(bc)::value == 0) return hb0;
        else if constexpr (decltype(bc)::value == 1) return hb1;
        else return hb2;
    };
    auto tbuf = [&](auto bc) __attribute__((always_inline)) -> float * {
        if constexpr (decltype(bc)::value == 0) return tb0;
        else if constexpr (decltype(bc)::value == 1) return tb1;
        else return tb2;
    };

    const int Q = p.chunk, H = p.nheads, G = p.ngroups, nc = p.nchunks, HPG = p.heads_per_group;
    const int64_t L = p.seqlen;
    // Channels: a workgroup owns P of the head's PF = csplit P channels
    // (rows p of the state are independent), channel slice cs.
    const int PF = P * csplit;

    // Workgroup -> (b, c, g, slice, channel slice); the slices of one (b, c)
    // run back to back on one XCD.
    const int64_t total = p.batch * nc * G * nslices * csplit;
    const int64_t per_xcd = gridDim.x / kXcds;
    const int64_t logical0 = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (logical0 >= total) return;
    const int cs = (int)(logical0 % csplit);
    const int64_t logical = logical0 / csplit;
    const int slice = (int)(logical % nslices);
    const int g = (int)((logical / nslices) % G);
    const int c = (int)((logical / ((int64_t)nslices * G)) % nc);
    const int64_t b = logical / ((int64_t)nslices * G * nc);
    const int hbeg = g * HPG + slice * hps;
    const int hcnt = min(hps, HPG - slice * hps);
    if (hcnt <= 0) return;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform across the wave
    const int il = lane & 15, grp = lane >> 4;
    const int64_t t0 = (int64_t)c * Q;
    const int Qc = (int)(L - t0 < Q ? L - t0 : Q);
    const int nit = (Qc + 15) / 16;
    const bool has_prev = c > 0 || p.init_state != nullptr;

    // The wave's tiles, their diagonal blocks, and whether they hold tokens.
    int tile[MAXIT], md[MAXIT];
    bool live[MAXIT];
    if constexpr (WIDE) {
        tile[0] = wide_tile<NIT>(wave);
    } else {
        tile[0] = wave;
        if constexpr (MAXIT == 2) tile[1] = NIT - 1 - wave;
    }
#pragma unroll
    for (int k = 0; k < MAXIT; ++k) {
        md[k] = tile[k] >> 1;
        live[k] = tile[k] < nit;
    }

    const T *xg = reinterpret_cast<const T *>(p.x);
    const T *bg = reinterpret_cast<const T *>(p.B);
    const T *cg = reinterpret_cast<const T *>(p.C);
    const T *hg = reinterpret_cast<const T *>(p.prev);

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

    // ---- copies of one head into buffer `bc`.  Token rows past the chunk
    // read its last token (in bounds, finite; their products meet an exact
    // zero); dstate 16 fills each 32-column state row with two copies.  A
    // wave knows how many copies one head adds (padding copies go to `junk`;
    // with three or more waves only waves 0-2 copy the three table rows), so
    // it can wait for all but the last head's copies.
    // Per-lane source offsets (elements) of the copies; the same for every
    // head, whose base address is uniform.
    uint32_t offx[Cf::UX], offh[Cf::UH];
#pragma unroll
    for (int u = 0; u < Cf::UX; ++u) {
        const int U = 64 * (wave + W * u) + lane;
        const int row = U / WX, pos = U - row * WX;
        offx[u] = (uint32_t)min(row, Qc - 1) * (uint32_t)(H * PF) + 8 * (pos ^ xsw<WX>(row));
    }
#pragma unroll
    for (int u = 0; u < Cf::UH; ++u) {
        const int U = 64 * (wave + W * u) + lane;
        const int row = U / WB, pos = U - row * WB;
        int gc = pos ^ swz_rows16<WB>(row);
        if constexpr (NP != N) gc %= N / 8;
        offh[u] = (uint32_t)(row * N + 8 * gc);
    }
    const uint32_t offt = 4 * min(lane, Q / 4 - 1);

    auto issue_head = [&](int hh, auto bc) __attribute__((always_inline)) {
        const int h = hbeg + hh;
        // Opaque copies of the lane offsets: otherwise base + lane offset is
        // reassociated and hoisted out of the head loop as 64-bit values.
        uint32_t ox[Cf::UX], oh[Cf::UH];
#pragma unroll
        for (int u = 0; u < Cf::UX; ++u) {
            ox[u] = offx[u];
            asm volatile("" : "+v"(ox[u]));
        }
#pragma unroll
        for (int u = 0; u < Cf::UH; ++u) {
            oh[u] = offh[u];
            asm volatile("" : "+v"(oh[u]));
        }
        const T *xsrc = xg + ((b * L + t0) * H + h) * PF + cs * P;
        T *xdst = xbuf(bc);
#pragma unroll
        for (int u = 0; u < Cf::UX; ++u) {
            const int ins = wave + W * u;
            if (Cf::IXH % W == 0 || ins < Cf::IXH) copy16_to_lds(xsrc + ox[u], xdst + ins * 512);
            else copy16_to_lds(xsrc, junk);
        }
        if (has_prev) {
            const T *hsrc = hg + (((b * nc + c) * H + h) * (int64_t)PF + cs * P) * N;
            T *hdst = hbuf(bc);
#pragma unroll
            for (int u = 0; u < Cf::UH; ++u) {
                const int ins = wave + W * u;
                if (Cf::IHH % W == 0 || ins < Cf::IHH) copy16_to_lds(hsrc + oh[u], hdst + ins * 512);
                else copy16_to_lds(hsrc, junk);
            }
        }
        // Per-token tables of this (b, h, c): one 1 KB row each (Q <= 256).
        const int64_t trow = ((b * H + h) * nc + c) * (int64_t)Q;
        uint32_t offt_h = offt;
        asm volatile("" : "+v"(offt_h));
        float *tdst = tbuf(bc);
#pragma unroll
        for (int u = 0; u < Cf::UT; ++u) {
            const int t = wave + W * u;
            if (t < 3) copy16_to_lds(((t == 0 ? p.cs : (t == 1 ? p.ct : p.dte)) + trow) + offt_h, tdst + 256 * t);
            else if (W < 3) copy16_to_lds(p.cs + trow, junk);  // waves that copy several tables copy equally many
        }
    };

    // 16-byte-per-lane reads of h and of the B ring: row 16*a + il, piece
    // 4*ks + grp (swizzle period 16, so a per-lane constant).
    int roff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) roff[ks] = il * NP + 8 * ((4 * ks + grp) ^ swz_rows16<WB>(il));

    // ---- phase A: causal tiles of G^T = B C^T.  B fragments come straight
    // from global memory (each 32-token step of B is read by every wave, from
    // L2 after the first), one step ahead of the products.
    // go0/go1: off-diagonal blocks of tiles 0/1 (index = block), gd: diagonal
    // blocks.  Lane (il, grp) holds G^T[j][i] for i = 16t + il and
    // j = 32m + 4grp + r (slots 0-3) and j + 16 (slots 4-7).
    bf16x8 go0[S0 > 0 ? S0 : 1], go1[S1 > 0 ? S1 : 1], gd[MAXIT];
    const bf16x8 zero8 = {};
#pragma unroll
    for (int s = 0; s < (S0 > 0 ? S0 : 1); ++s) go0[s] = zero8;
#pragma unroll
    for (int s = 0; s < (S1 > 0 ? S1 : 1); ++s) go1[s] = zero8;
#pragma unroll
    for (int k = 0; k < MAXIT; ++k) gd[k] = zero8;

    const T *bsrc = bg + ((b * L + t0) * G + g) * N;
    auto load_b = [&](int s, Frag<T> (&bf)[2][KS]) __attribute__((always_inline)) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int j = min(kStep * s + 16 * half + il, Qc - 1);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int n0c = 32 * ks + 8 * grp;
                if (n0c < N) load8(bf[half][ks], bsrc + (int64_t)j * G * N + n0c);
                else bf[half][ks].zero();
            }
        }
    };
    // One step of phase A: the pair (tile K, block S).
    auto pair_a = [&](auto kc, auto sc, const Frag<T> (&bfr)[2][KS]) __attribute__((always_inline)) {
        constexpr int K = decltype(kc)::value, S = decltype(sc)::value;
        if (!live[K] || S > md[K]) return;
        const int t = tile[K];
        const bool is_diag = S == md[K];
        const int i = 16 * t + il;
        bf16x8 v = zero8;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            if (2 * S + half > t) continue;  // above the diagonal
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) mma(bfr[half][ks], cf[K][ks], acc);
            // The diagonal block keeps only j <= i (the causal mask, applied
            // here once instead of per head).
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = kStep * S + 16 * half + 4 * grp + r;
                v[4 * half + r] = (bf16)(is_diag && j > i ? 0.f : acc[r]);
            }
        }
        // Value selects, not a branch between two destinations (that would
        // turn into a store through a selected pointer and keep the arrays in
        // scratch memory).
        gd[K] = is_diag ? v : gd[K];
        if constexpr (K == 0 && S < S0) go0[S] = is_diag ? go0[S] : v;
        if constexpr (K == 1 && S < S1) go1[S] = is_diag ? go1[S] : v;
    };

    const int nstep = (Qc + kStep - 1) / kStep;
    {
        if constexpr (MAXIT == 2) {
            // Two tiles: the wave visits (nearly) every step; B one step ahead.
            Frag<T> ba[2][KS], bb[2][KS];
            load_b(0, ba);
            issue_head(0, std::integral_constant<int, 0>{});
            if (NBUF == 3 && hcnt > 1) issue_head(1, std::integral_constant<int, 1>{});
            static_for<NBLK>([&](auto sc) __attribute__((always_inline)) {
                constexpr int s = decltype(sc)::value;
                if (s < nstep) {
                    auto step = [&](Frag<T> (&cur)[2][KS], Frag<T> (&nxt)[2][KS]) __attribute__((always_inline)) {
                        if (s + 1 < nstep) load_b(s + 1, nxt);
                        pair_a(std::integral_constant<int, 0>{}, sc, cur);
                        pair_a(std::integral_constant<int, 1>{}, sc, cur);
                    };
                    if constexpr (s % 2 == 0) step(ba, bb);
                    else step(bb, ba);
                }
            });
        } else if constexpr (!WIDE) {
            // One tile of at most 16 tokens (one j block): B from global memory.
            issue_head(0, std::integral_constant<int, 0>{});
            if (NBUF == 3 && hcnt > 1) issue_head(1, std::integral_constant<int, 1>{});
            if (live[0]) {
                Frag<T> bf[2][KS];
                load_b(0, bf);
                pair_a(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, bf);
            }
        } else {
            // One tile: B streams through the LDS ring, RING-1 steps ahead;
            // each wave multiplies only the blocks up to its diagonal.  Every
            // wave issues IB_W copies per step (padding copies go to junk),
            // so one count waits for a step.
            const T *bsrc = bg + ((b * L + t0) * G + g) * N;
            auto issue_b = [&](int step, auto slot) __attribute__((always_inline)) {
                T *dst = ring(slot);
#pragma unroll
                for (int u = 0; u < Cf::IB_W; ++u) {
                    const int ins = wave + W * u;
                    if (ins < Cf::IB) {
                        const int U = 64 * ins + lane;
                        const int row = U / WB, pos = U - row * WB;
                        int gc = pos ^ swz_rows16<WB>(row);
                        if constexpr (NP != N) gc %= N / 8;
                        const int j = min(kStep * step + row, Qc - 1);
                        copy16_to_lds(bsrc + (int64_t)j * G * N + 8 * gc, dst + ins * 512);
                    } else {
                        copy16_to_lds(bsrc, junk);
                    }
                }
            };
            issue_head(0, std::integral_constant<int, 0>{});
            static_for<Cf::RING - 1>([&](auto sc) __attribute__((always_inline)) {
                if (decltype(sc)::value < nstep) issue_b(decltype(sc)::value, sc);
            });
            static_for<NBLK>([&](auto sc) __attribute__((always_inline)) {
                constexpr int s = decltype(sc)::value;
                if (s < nstep) {
                    // Step s has landed once at most RING-2 later steps are pending.
                    if (s + Cf::RING - 2 < nstep) wait_vmcnt<Cf::IB_W * (Cf::RING - 2)>();
                    else wait_vmcnt<0>();
                    // ... for every wave; and slot (s-1) % RING is no longer read (its
                    // reads feed products that need not be issued yet, hence
                    // the LDS wait before the barrier).
                    lds_barrier();
                    if (s + Cf::RING - 1 < nstep)
                        issue_b(s + Cf::RING - 1, std::integral_constant<int, s + Cf::RING - 1>{});
                    if (s <= md[0] && live[0]) {
                        const T *rb = ring(sc);
                        Frag<T> bf[2][KS];
#pragma unroll
                        for (int half = 0; half < 2; ++half)
#pragma unroll
                            for (int ks = 0; ks < KS; ++ks) load8(bf[half][ks], rb + 16 * half * NP + roff[ks]);
                        pair_a(std::integral_constant<int, 0>{}, sc, bf);
                    }
                }
            });
        }
    }

    // Per-lane LDS offsets (elements).  Every swizzle depends only on the row
    // modulo a period dividing 16, so a fragment's address is a per-lane
    // constant plus a wave-uniform row offset.
    //  - transposing reads of x: source lane (il = 4*kr + a) points at row
    //    16*half + 4*grp + kr, columns 16*q + 4*a .. +3.
    const int rl = 4 * grp + (il >> 2);
    int xoff[PT];
#pragma unroll
    for (int q = 0; q < PT; ++q)
        xoff[q] = rl * P + 8 * ((2 * q + ((il & 3) >> 1)) ^ xsw<WX>(rl)) + 4 * (il & 1);

    // ---- phase B: heads; head hh lives in buffer hh % NBUF.
    T *yg = reinterpret_cast<T *>(p.y);
    // Per-lane output offsets within one head's rows: token i, channels 16q + 4grp.
    uint32_t yoff[MAXIT];
#pragma unroll
    for (int k = 0; k < MAXIT; ++k) yoff[k] = (uint32_t)(16 * tile[k] + il) * (uint32_t)(H * PF) + 4 * grp;

    auto head = [&](auto bc, int hh) __attribute__((always_inline)) {
        constexpr int BI = decltype(bc)::value;
        // Head hh is in buffer BI for every wave, and no wave still reads the
        // buffer of head hh-1, which now receives head hh+NBUF-1.
        barrier_only();
        const int ahead = hh + NBUF - 1;
        // With three buffers, the first head of each loop iteration issues its
        // copies after computing: the compiler's waitcnt state at the loop
        // header no longer separates the buffers, so its LDS reads wait for
        // every copy in flight, and those should then be old ones only.
        constexpr bool late = NBUF == 3 && BI == 0;
        if (!late && ahead < hcnt) issue_head(ahead, std::integral_constant<int, (BI + NBUF - 1) % NBUF>{});

        const int h = hbeg + hh;
        const T *xsb = xbuf(bc);
        const T *hsb = hbuf(bc);
        const float *csv = tbuf(bc), *ctv = csv + 256, *dtev = csv + 512;

        float cs2i[MAXIT];
#pragma unroll
        for (int k = 0; k < MAXIT; ++k) cs2i[k] = csv[16 * tile[k] + il] * kLog2e;
        // Keep G^T packed between heads: an empty asm makes the values opaque
        // per head, so their bf16 -> fp32 unpacking is not hoisted out of the
        // head loop (twice the registers, and spills).
#pragma unroll
        for (int s = 0; s < (S0 > 0 ? S0 : 1); ++s) asm volatile("" : "+v"(go0[s]));
#pragma unroll
        for (int s = 0; s < (S1 > 0 ? S1 : 1); ++s) asm volatile("" : "+v"(go1[s]));
#pragma unroll
        for (int k = 0; k < MAXIT; ++k) asm volatile("" : "+v"(gd[k]));

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
                const float ei = exp2_hw(cs2i[k]);
#pragma unroll
                for (int q = 0; q < PT; ++q) acc[k][q] = acc[k][q] * ei;
            }
        }

        // Orange: walk the j blocks; each block's x^T fragments serve both tiles.
        static_for<NBLK>([&](auto mc) __attribute__((always_inline)) {
            constexpr int m = decltype(mc)::value;
            const bool use0 = live[0] && m <= md[0];
            const bool use1 = MAXIT == 2 && live[MAXIT - 1] && m <= md[MAXIT - 1];
            if (!use0 && !use1) return;
            const T *xm = xsb + kStep * m * P;
            auto read_x = [&](int q) __attribute__((always_inline)) {
                const i16x4 a0 = ds_read_tr16(xm + xoff[q]);
                const i16x4 a1 = ds_read_tr16(xm + 16 * P + xoff[q]);
                typedef short i16x8 __attribute__((ext_vector_type(8)));
                Frag<T> xq;
                xq.v = __builtin_bit_cast(bf16x8, i16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]});
                return xq;
            };
            // Two tiles per wave: the block's x^T fragments are read once and
            // serve both; one tile per wave: each is read just before its
            // product (fewer live registers).
            Frag<T> xf[MAXIT == 2 ? PT : 1];
            if constexpr (MAXIT == 2) {
#pragma unroll
                for (int q = 0; q < PT; ++q) xf[q] = read_x(q);
            }
            auto products = [&](auto kc, const Frag<T> &lf) __attribute__((always_inline)) {
                constexpr int K = decltype(kc)::value;
                if constexpr (MAXIT == 2) {
#pragma unroll
                    for (int q = 0; q < PT; ++q) mma(xf[q], lf, acc[K][q]);
                } else {
#pragma unroll
                    for (int q = 0; q < PT; ++q) mma(read_x(q), lf, acc[K][q]);
                }
            };
            auto off_diag = [&](auto kc, const bf16x8 &gv) __attribute__((always_inline)) {
                constexpr int K = decltype(kc)::value;
                const float ai = exp2_hw(cs2i[K] - csv[kStep * m + kStep - 1] * kLog2e);
                const f32x4 d0 = *reinterpret_cast<const f32x4 *>(dtev + kStep * m + 4 * grp);
                const f32x4 d1 = *reinterpret_cast<const f32x4 *>(dtev + kStep * m + 16 + 4 * grp);
                Frag<T> lf;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    lf.set(r, (float)gv[r] * (ai * d0[r]));
                    lf.set(4 + r, (float)gv[4 + r] * (ai * d1[r]));
                }
                products(kc, lf);
            };
            auto diag = [&](auto kc) __attribute__((always_inline)) {
                constexpr int K = decltype(kc)::value;
                const f32x4 c0 = *reinterpret_cast<const f32x4 *>(ctv + kStep * m + 4 * grp);
                const f32x4 c1 = *reinterpret_cast<const f32x4 *>(ctv + kStep * m + 16 + 4 * grp);
                Frag<T> lf;
                // gd is zero above the diagonal; there the exponent may be
                // large, so it is capped to keep 0 * 2^x finite (below the
                // diagonal it is at most log2(dt_j)).
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float e0 = exp2_hw(fminf(cs2i[K] - c0[r], 64.f));
                    const float e1 = exp2_hw(fminf(cs2i[K] - c1[r], 64.f));
                    lf.set(r, (float)gd[K][r] * e0);
                    lf.set(4 + r, (float)gd[K][4 + r] * e1);
                }
                products(kc, lf);
            };
            if (use0) {
                if constexpr (m < S0) {
                    if (m < md[0]) off_diag(std::integral_constant<int, 0>{}, go0[m]);
                    else diag(std::integral_constant<int, 0>{});
                } else {
                    diag(std::integral_constant<int, 0>{});
                }
            }
            if constexpr (MAXIT == 2) {
                if (use1) {
                    if constexpr (m < U1) {
                        off_diag(std::integral_constant<int, 1>{}, go1[m]);
                    } else if constexpr (m < S1) {
                        if (m < md[1]) off_diag(std::integral_constant<int, 1>{}, go1[m]);
                        else diag(std::integral_constant<int, 1>{});
                    } else {
                        diag(std::integral_constant<int, 1>{});
                    }
                }
            }
        });

        // + D x (x_i from the head's LDS rows), round to bf16, store.  The
        // row/column offsets are recomputed here from an opaque copy of the
        // lane index (hoisted out of the head loop they would hold registers).
        int ilo = il, grpo = grp;
        asm volatile("" : "+v"(ilo), "+v"(grpo));
        if (late && ahead < hcnt) issue_head(ahead, std::integral_constant<int, (BI + NBUF - 1) % NBUF>{});

        // D through the constant address space: a scalar load, which vmcnt
        // does not count (a vector load here would have to wait for the copies).
        const float dh = p.D ? ((const __attribute__((address_space(4))) float *)(uintptr_t)p.D)[h] : 0.f;
        T *yh = yg + ((b * L + t0) * H + h) * PF + cs * P;
        // Head hh+1's copies have landed: its loads precede the last head's
        // in issue order and loads complete in order (pending older stores
        // only make the wait stricter).
        if (NBUF == 3 && ahead < hcnt) {
            constexpr int CX = NBUF == 3 ? Cf::UX : 0, CH = NBUF == 3 ? Cf::UH : 0, CT = NBUF == 3 ? Cf::UT : 0;
            const bool tab_wave = W < 3 || wave < 3;  // waves that copy the tables
            if (has_prev) {
                if (tab_wave) wait_vmcnt<CX + CH + CT>();
                else wait_vmcnt<CX + CH>();
            } else {
                if (tab_wave) wait_vmcnt<CX + CT>();
                else wait_vmcnt<CX>();
            }
        } else {
            wait_vmcnt<0>();
        }
#pragma unroll
        for (int k = 0; k < MAXIT; ++k) {
            const int i = 16 * tile[k] + il;
            if (!live[k] || i >= Qc) continue;
#pragma unroll
            for (int q = 0; q < PT; ++q) {
                // x_i[16q + 4grp .. +3]: row i = 16*t + il of the head's x buffer.
                const int dxoff = ilo * P + 8 * ((2 * q + (grpo >> 1)) ^ xsw<WX>(ilo)) + 4 * (grpo & 1);
                const V4 xv = *reinterpret_cast<const V4 *>(xsb + 16 * tile[k] * P + dxoff);
                V4 out;
#pragma unroll
                for (int r = 0; r < 4; ++r) out[r] = (T)(acc[k][q][r] + dh * (float)xv[r]);
                *reinterpret_cast<V4 *>(yh + yoff[k] + 16 * q) = out;
            }
        }
    };

    wait_vmcnt<0>();  // the first heads' copies have landed
    for (int h0 = 0; h0 < hcnt; h0 += NBUF) {
        static_for<NBUF>([&](auto bc) __attribute__((always_inline)) {
            const int hh = h0 + decltype(bc)::value;
            if (hh < hcnt) head(bc, hh);
        });
    }
    wait_vmcnt<0>();  // no copy outlives the workgroup
}

template <int NT, int PT, int NIT, bool WIDE>
hipError_t launch_nit(const Params &p, hipStream_t stream) {
    using Cf = HeadsCfg<NT, PT, NIT, WIDE>;
    if constexpr (Cf::LDS_BYTES > 160 * 1024) {
        return hipErrorNotSupported;
    } else {
        const int csplit = p.headdim / Cf::P;  // channel slices per head
        const int64_t base = p.batch * p.nchunks * (int64_t)p.ngroups * csplit;
        int nslices = (int)std::min<int64_t>(p.heads_per_group, std::max<int64_t>(1, (256 + base - 1) / base));
        const int hps = (p.heads_per_group + nslices - 1) / nslices;
        nslices = (p.heads_per_group + hps - 1) / hps;
        const int64_t total = base * nslices;
        const int64_t per_xcd = (total + kXcds - 1) / kXcds;
        hipLaunchKernelGGL((chunk_output_heads_kernel<NT, PT, NIT, WIDE>), dim3((unsigned)(per_xcd * kXcds)),
                           dim3(Cf::THREADS), 0, stream, p, hps, nslices, csplit);
        return hipGetLastError();
    }
}

// Shapes whose one-tile-per-wave variant fits 128 VGPRs.
template <int NT, int PT>
constexpr bool kWideOk = NT <= 8 && PT <= 4;
// dstate 256 with 256-token chunks runs 32-channel workgroups in the
// one-tile-per-wave layout (a head's buffers then fit LDS next to the B ring,
// and 16 waves share a compute unit instead of 8).
#ifndef SSD_OUT_SPLIT256
#define SSD_OUT_SPLIT256 1
#endif

template <int NT, int PT>
hipError_t dispatch_q(const Params &p, hipStream_t stream) {
    switch (p.chunk) {
        case 8:
        case 16: return launch_nit<NT, PT, 1, false>(p, stream);
        case 32: return launch_nit<NT, PT, 2, false>(p, stream);
        case 64: return launch_nit<NT, PT, 4, false>(p, stream);
        case 128: return launch_nit<NT, PT, 8, kWideOk<NT, PT>>(p, stream);
        case 256:
            if constexpr (SSD_OUT_SPLIT256 && NT == 16 && PT >= 2) return launch_nit<NT, 2, 16, true>(p, stream);
            else return launch_nit<NT, PT, 16, kWideOk<NT, PT>>(p, stream);
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
