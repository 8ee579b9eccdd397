// Single-pass SSD forward (bf16): one workgroup at a time per item (sequence
// b, head h, or a 64-channel half of a head of headdim 128) walks the
// sequence in blocks of 128 tokens and keeps the running state in registers,
// so all four parts of the block decomposition of "Transformers are SSMs"
// (cloud.tencent.com.cn, section "SSD算法") run in one kernel: the chunk
// states and the states entering each block never reach memory, x is read
// once and y written once.  The state passing is the sequential scan over
// chunks of section "深入解析分块与状态传递机制", carried by the workgroup.
// The chunk-local cumulative decay is computed here too (from dt and A), so
// the call is this one kernel.
//
// The kernel's block length (128 tokens) is its own and does not depend on
// the chunk_size of the call: every block length gives the same result up
// to rounding, since the block decomposition is an exact re-association.
//
// Block c (tokens t0 .. t0+Qc-1), head h of group g; cs the block-local
// inclusive cumulative log-decay A_h sum dt, cs2 = cs log2(e),
// ct_j = cs2_j - log2(dt_j), e(m) the last token of 32-token block m,
// dte_j = dt_j exp(cs_e(m) - cs_j) for j in m and wl_j = dt_j exp(cs_last -
// cs_j) (all computed per block by one wave, in fp64 and rounded once):
//   G      = C B^T (causal 16x32 tiles, fp32 accumulate)
//   orange y_i  = sum_{j<=i} exp(cs_i - cs_j) dt_j G_ij x_j
//   blue   y_i += exp(cs_i) C_i . h_{c-1}
//   green  h_c  = exp(cs_last) h_{c-1} + sum_j wl_j B_j^T x_j
//          y_i += D_h x_i.
// Decay factors.  Every factor applied is at most max(1, dt):
//   orange, block m below the tile's diagonal block md: G_ij times
//     exp2(cs2_i - cs2_e(m)) dte_j, rounded once to bf16, on raw x;
//   orange, diagonal block md: G_ij times the exact exp2(cs2_i - ct_j)
//     (selected to 0 above the diagonal), plus D at j = i, rounded
//     once, on raw x; exact however strong the decay inside the block;
//   blue: exp2(cs2_i) times C_i . h_{c-1};
//   state: the state scaled once per block by exp(cs_last), plus the
//     products of the B fragments weighted by wl (formed from the
//     transposed B read and rounded once) with raw x.
// The state after an accepted index j (multi-step verify, "3天把Llama训成
// Mamba", blog.csdn.net, section "推测解码") is computed in the block holding
// j, from the state entering it, with the exact factors exp2(cs2_j - ct_s):
//   h_j = exp(cs_j) h_{c-1} + sum_{s<=j} exp(cs_j - cs_s) dt_s x_s B_s^T.
//
// Channels: the rows p of the state are independent recurrences, so a head
// of headdim 128 runs as two items of 64 channels, which share dt, B and C
// and own their columns of x and y and their rows of the state.
//
// Work split inside a workgroup: 8 waves, each owning one 16-row tile of
// the block (tiles dealt so that the two waves of a SIMD meet 3 off-diagonal
// 32-token blocks together) and the state tiles of one n tile.  Per block a
// wave computes blue, then walks the 32-token blocks m once: each block's x
// fragments (transposing LDS read) feed both its orange product (m <= md)
// and its state update.  LDS holds the block's B rows and x rows
// (token-major, read with the transposing LDS read), h_{c-1} in bf16 and the
// per-token tables (two copies: wave 0 writes the next block's while this
// block's are read).  Under 80 KB at dstate 128, so two workgroups share a
// compute unit and one's block switch overlaps the other's products.  The
// next block's x and B rows are loaded into registers at the start of a
// block, its dt values and C rows after the block's last use of C; at the
// switch every wave writes the next block's LDS and one barrier publishes
// it.  Global accesses go through buffer descriptors over each block's rows
// (rows past the sequence read as zero, their stores are dropped).
//
// Schedule: a grid of two workgroups per compute unit; workgroup w runs on
// XCD w mod 8 (the hardware deals workgroups to the XCDs in turn), and each
// XCD takes a contiguous range of items, so heads sharing B and C rows share
// that XCD's L2.  With at least as many items as workgroups, each takes
// whole items and the leftovers are split in two halves of their blocks;
// with fewer, every item is split in up to four ranges.  A range that does
// not start at block 0 first runs the state recurrence alone (no C, no y)
// over the blocks before it, from the initial state: recomputing is cheaper
// than waiting for another workgroup, and no workgroup ever waits for
// another one.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

constexpr int kXcds = 8;
constexpr int kStep = 32;           // tokens per j block (one MFMA k step)
constexpr int kMaxRanges = 4;       // ranges per item when items are fewer than workgroups
constexpr int kAuxNt = 2;           // cache-policy operand of the buffer builtins: nt (non-temporal)
constexpr double kLog2eD = 1.4426950408889634074;

// Compute units of the current device (cached per device).
int compute_units() {
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Geometry for dstate 16 NT, item channels 16 PT and blocks of QB tokens:
// QB / 16 waves, one 16-row tile each.
template <int NT, int PT, int QB>
struct FusedCfg {
    static constexpr int N = NT * 16, P = PT * 16, Q = QB;
    static constexpr int W = Q / 16, THREADS = 64 * W;  // waves, threads
    static constexpr int NBLK = Q / kStep;              // 32-token blocks per block
    static constexpr int TPL = Q / 64;                  // tokens per lane in the table wave
    static constexpr int KS = N / 32;                   // 32-wide k steps over n
    static constexpr int WB = N / 8, WX = P / 8;        // 16-byte pieces per B row, per x row
    // Waves along n and p over the 16x16 tiles of the state: all of n
    // first, so that each B fragment of the state update, scaled by the
    // per-token decay, is read (and scaled) by one wave only.
    static constexpr int WPN = NT >= W ? W : NT, WPP = W / WPN;
    static constexpr int NTW = NT / WPN, PTW = PT / WPP;
    static constexpr int UXR = Q * WX / THREADS;        // 16-byte x pieces per thread
    static constexpr int UBR = Q * WB / THREADS;        // 16-byte B pieces per thread
    // Per-block tables in LDS (floats): cs2, ct, dte and wl per token, then
    // cs2 at the end of each 32-token block.
    static constexpr int TB_CS2 = 0, TB_CT = Q, TB_DTE = 2 * Q, TB_WL = 3 * Q, TB_CE = 4 * Q;
    static constexpr int TB_SIZE = 4 * Q + NBLK;
    // LDS rows are padded by 32 bytes, so that every fragment address is one
    // per-lane base plus an immediate offset, and consecutive rows start on
    // different banks.  (A 16-byte pad measured twice the bank conflicts.)
    static constexpr int SB = N * 2 + 32, SX = P * 2 + 32, SH = N * 2 + 32;  // bytes per LDS row of B, x, h
    static constexpr size_t LDS_BYTES = (size_t)Q * SB + (size_t)Q * SX + (size_t)P * SH + 2 * TB_SIZE * 4;
    // Two workgroups per compute unit when two fit its 160 KB of LDS.
    static constexpr int WGS_PER_CU = LDS_BYTES <= 80 * 1024 ? 2 : 1;
    static constexpr bool OK = NTW >= 1 && PTW >= 1 && NT % WPN == 0 && PT % WPP == 0 && UXR >= 1 && UBR >= 1 &&
                               (Q * WX) % THREADS == 0 && (Q * WB) % THREADS == 0 && LDS_BYTES <= 160 * 1024 &&
                               W * WGS_PER_CU == 16;
};

// Raw buffer descriptor over [base, base + bytes): loads beyond it read 0
// and stores beyond it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double shfl_f64(double v, int src) {
    const int lo = __builtin_amdgcn_ds_bpermute(src << 2, (int)__double2loint(v));
    const int hi = __builtin_amdgcn_ds_bpermute(src << 2, (int)__double2hiint(v));
    return __hiloint2double(hi, lo);
}

// bf16 fragment times per-slot fp32 factors, rounded once to bf16.
__device__ __forceinline__ void scale_frag(Frag<bf16> &f, const f32x4 &w0, const f32x4 &w1) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        f.v[s] = (bf16)((float)f.v[s] * w0[s]);
        f.v[4 + s] = (bf16)((float)f.v[4 + s] * w1[s]);
    }
}

template <int NT, int PT, int QB>
__global__ __launch_bounds__(4 * QB) __attribute__((amdgpu_waves_per_eu(4)))  // QB / 16 waves
void chunk_scan_fused_kernel(Params p) {
    using Cf = FusedCfg<NT, PT, QB>;
    using T = bf16;
    constexpr int N = Cf::N, P = Cf::P, Q = Cf::Q, KS = Cf::KS, WB = Cf::WB, WX = Cf::WX;
    constexpr int W = Cf::W, THREADS = Cf::THREADS, NBLK = Cf::NBLK, TPL = Cf::TPL;
    static_assert(THREADS == 4 * QB, "launch bounds");
    constexpr int TB_CS2 = Cf::TB_CS2, TB_CT = Cf::TB_CT, TB_DTE = Cf::TB_DTE, TB_WL = Cf::TB_WL, TB_CE = Cf::TB_CE;
    constexpr int NTW = Cf::NTW, PTW = Cf::PTW, UXR = Cf::UXR, UBR = Cf::UBR;
    constexpr int SB = Cf::SB, SX = Cf::SX, SH = Cf::SH;
    constexpr int RX = THREADS / WX, RB = THREADS / WB;  // rows between a thread's x / B pieces
    typedef typename Vec8<T>::type V8;
    typedef typename Vec4<T>::type V4;
    typedef short i16x8 __attribute__((ext_vector_type(8)));

    __shared__ __align__(16) char bl[Q * SB];  // B rows (token-major)
    __shared__ __align__(16) char xs[Q * SX];  // x rows (token-major)
    __shared__ __align__(16) char hb[P * SH];  // h_{c-1} in bf16, rows p
    // Tables of a block; two objects, so that one block's are read while
    // wave 0 writes the next block's.
    __shared__ __align__(16) float tb0[Cf::TB_SIZE], tb1[Cf::TB_SIZE];

    const int H = p.nheads, G = p.ngroups, HPG = p.heads_per_group;
    const int PF = p.headdim, PS = PF / P;  // channels of a head, items per head
    const int64_t L = p.seqlen;
    const int nb = (int)((L + Q - 1) / Q);

    // ---- work of this workgroup.  A unit is an item (b, h, channel half s),
    // item (b*H + h)*PS + s, with its blocks [c0, c1); blocks [0, c0) are
    // run first for the state alone.  (Items fit 31 bits: the launcher
    // checks.)
    const int I = (int)(p.batch * H * PS);
    const int Wg = gridDim.x;
    const int NX = (Wg % kXcds == 0 && I >= kXcds) ? kXcds : 1;
    const int xcd = (int)blockIdx.x % NX, wl = (int)blockIdx.x / NX, Wx = Wg / NX;
    const int Ibase = I / NX, Iext = I % NX;
    const int Ix = Ibase + (xcd < Iext ? 1 : 0);
    const int ibeg = xcd * Ibase + min(xcd, Iext);  // first item of this XCD
    struct Unit {
        int item, c0, c1;
    };
    int nunits = 0, F = 0, R = 0, S = 1;
    bool split = false;
    if (Ix >= Wx) {
        F = Ix / Wx;
        R = Ix - F * Wx;
        split = R > 0 && 2 * R <= Wx && nb >= 2 && !p.no_split;
        nunits = F + (split ? (wl < 2 * R ? 1 : 0) : (wl < R ? 1 : 0));
    } else if (Ix > 0) {
        S = p.no_split ? 1 : min(kMaxRanges, min(Wx / Ix, nb));
        nunits = wl < Ix * S ? 1 : 0;
    }
    auto unit = [&](int k) -> Unit {
        if (Ix < Wx) {
            const int r = wl / Ix;
            return Unit{ibeg + (wl - r * Ix), r * nb / S, (r + 1) * nb / S};
        }
        if (k < F) return Unit{ibeg + wl + Wx * k, 0, nb};
        if (!split) return Unit{ibeg + F * Wx + wl, 0, nb};
        if (wl < R) return Unit{ibeg + F * Wx + wl, 0, nb / 2};
        return Unit{ibeg + F * Wx + (wl - R), nb / 2, nb};
    };
    if (nunits == 0) return;
    // A step is one block of one unit; units run in order, each from block 0.
    // (b, h, g of the item are worked out once per unit.)
    struct Step {
        int k, c, c0, c1;
        int item, b, bh;  // bh = b*H + h
        int h, g, s;
    };
    auto step_of = [&](int k) -> Step {
        const Unit u = unit(k);
        const uint32_t it = (uint32_t)u.item, bh = it / (uint32_t)PS, hh = bh % (uint32_t)H;
        return Step{k, 0, u.c0, u.c1, u.item, (int)(bh / (uint32_t)H), (int)bh, (int)hh, (int)hh / HPG,
                    (int)(it - bh * (uint32_t)PS)};
    };
    auto next_step = [&](const Step &st) -> Step {
        if (st.c + 1 < st.c1) {
            Step n = st;
            n.c = st.c + 1;
            return n;
        }
        return step_of(st.k + 1);
    };
    int nsteps = 0;
    for (int k = 0; k < nunits; ++k) nsteps += unit(k).c1;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int il = lane & 15, grp = lane >> 4;
    const int tile = wide_tile<W>(wave), md = tile >> 1;
    // With 16 waves in one workgroup per compute unit, waves meet md
    // off-diagonal blocks each and a block lasts as long as the waves with
    // the most: their issue priority grows with md, so that the others fill
    // the gaps.  (With two workgroups per compute unit the other
    // workgroup's waves fill them; there all waves keep one priority.)
    if constexpr (W == 16) {
        const int prio = md * 4 / NBLK;
        if (prio >= 3)
            __builtin_amdgcn_s_setprio(3);
        else if (prio == 2)
            __builtin_amdgcn_s_setprio(2);
        else if (prio == 1)
            __builtin_amdgcn_s_setprio(1);
    }
    const int nw = wave % Cf::WPN, pw = wave / Cf::WPN;  // the wave's state tiles

    const uint32_t HP2 = (uint32_t)H * PF * 2, GN2 = (uint32_t)G * N * 2;  // bytes per token row
    auto block_len = [&](int c) -> int { return (int)min((int64_t)Q, L - (int64_t)c * Q); };
    // Token rows of a step's block: x and y of its item, B and C of its
    // group, dt of its head.  With on = false the descriptor covers no bytes:
    // its loads read 0 and its stores are dropped, so that every step issues
    // the same sequence of memory instructions (and the compiler's waits
    // for loads in flight count exactly, without waiting for more).
    auto x_rows = [&](const Step &st, bool on) {
        return rsrc((const T *)p.x + (((int64_t)st.b * L + (int64_t)st.c * Q) * H + st.h) * PF + st.s * P,
                    on ? block_len(st.c) * HP2 : 0u);
    };
    auto y_rows = [&](const Step &st, bool on) {
        return rsrc((const T *)p.y + (((int64_t)st.b * L + (int64_t)st.c * Q) * H + st.h) * PF + st.s * P,
                    on ? block_len(st.c) * HP2 : 0u);
    };
    auto b_rows = [&](const Step &st, bool on) {
        return rsrc((const T *)p.B + (((int64_t)st.b * L + (int64_t)st.c * Q) * G + st.g) * N,
                    on ? block_len(st.c) * GN2 : 0u);
    };
    auto c_rows = [&](const Step &st, bool on) {
        return rsrc((const T *)p.C + (((int64_t)st.b * L + (int64_t)st.c * Q) * G + st.g) * N,
                    on ? block_len(st.c) * GN2 : 0u);
    };
    auto dt_rows = [&](const Step &st, bool on) {
        return rsrc(p.dt + ((int64_t)st.b * L + (int64_t)st.c * Q) * H + st.h,
                    on ? block_len(st.c) * (uint32_t)H * 4 : 0u);
    };

    // ---- per-thread offsets of the global loads and of the LDS writes,
    // recomputed where used from an opaque thread index (kept across the
    // loop they would need registers): the thread's 16-byte pieces of x and
    // B rows and its C fragments (row 16 tile + il, columns 8grp + 32ks).
    auto otid = [&]() __attribute__((always_inline)) {
        int t = tid;
        asm volatile("" : "+v"(t));
        return t;
    };

    V8 xr[UXR], br[UBR];
    Frag<T> cf[KS];   // C rows of the wave's tile (G and blue)
    auto load_x = [&](const Step &st, bool on) __attribute__((always_inline)) {
        const auto r = x_rows(st, on);
        const int t = otid();
        const uint32_t vx = (uint32_t)(t / WX) * HP2 + (t % WX) * 16;
#pragma unroll
        for (int u = 0; u < UXR; ++u)
            xr[u] = __builtin_bit_cast(V8, __builtin_amdgcn_raw_buffer_load_b128(r, vx, u * RX * HP2, 0));
    };
    auto load_b = [&](const Step &st, bool on) __attribute__((always_inline)) {
        const auto r = b_rows(st, on);
        const int t = otid();
        const uint32_t vb = (uint32_t)(t / WB) * GN2 + (t % WB) * 16;
#pragma unroll
        for (int u = 0; u < UBR; ++u)
            br[u] = __builtin_bit_cast(V8, __builtin_amdgcn_raw_buffer_load_b128(r, vb, u * RB * GN2, 0));
    };
    auto load_c = [&](const Step &st, bool on) __attribute__((always_inline)) {
        const auto r = c_rows(st, on);
        const int t = otid() & 63;
        const uint32_t vc = (uint32_t)(16 * tile + (t & 15)) * GN2 + (t >> 4) * 16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            cf[ks].v = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, vc, 64 * ks, 0));
    };
    // dt of a step's tokens TPL lane .. TPL lane + TPL - 1 (0 past the
    // sequence), which wave 0 turns into tables.  Every wave issues the
    // loads (so that the value is not a branch result), but only wave 0's
    // descriptor covers any bytes.  Issued first at a switch, so that
    // waiting for them never waits for the others.
    float dtr[TPL];
    auto load_dt = [&](const Step &st, bool on) __attribute__((always_inline)) {
        const auto r = dt_rows(st, on && wave == 0);
        int ln = lane;  // opaque: recomputed here
        asm volatile("" : "+v"(ln));
        const uint32_t o = (uint32_t)(TPL * ln) * H * 4;
#pragma unroll
        for (int v = 0; v < TPL; ++v)
            dtr[v] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, o + v * H * 4, 0, 0));
    };
    // Wave 0: the tables of a step from its dt values (dtr).  Prefix sums
    // in fp64 (within the lane, then a wave-wide scan of the lane totals on
    // the DPP row shifts and broadcasts), each table entry rounded once.
    auto make_tables = [&](const Step &st, float *tb) __attribute__((always_inline)) {
        const int Qc = block_len(st.c);
        const double a = (double)((const __attribute__((address_space(4))) float *)(uintptr_t)p.A)[st.h];
        // Opaque lane index: everything derived from it is computed here
        // and not kept (or spilled) across the loop.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int i0 = TPL * ln;
        double sv[TPL];
        double run = 0.0;
#pragma unroll
        for (int v = 0; v < TPL; ++v) {
            run += (double)dtr[v];
            sv[v] = run;
        }
        double tot = run;
        auto dpp_add = [&](auto ctrl, auto rmask) __attribute__((always_inline)) {
            constexpr int C = decltype(ctrl)::value, M = decltype(rmask)::value;
            const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(tot), C, M, 0xf, true);
            const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(tot), C, M, 0xf, true);
            tot += __hiloint2double(hi, lo);
        };
        dpp_add(std::integral_constant<int, 0x111>{}, std::integral_constant<int, 0xf>{});  // row_shr:1
        dpp_add(std::integral_constant<int, 0x112>{}, std::integral_constant<int, 0xf>{});  // row_shr:2
        dpp_add(std::integral_constant<int, 0x114>{}, std::integral_constant<int, 0xf>{});  // row_shr:4
        dpp_add(std::integral_constant<int, 0x118>{}, std::integral_constant<int, 0xf>{});  // row_shr:8
        dpp_add(std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xa>{});  // row_bcast:15
        dpp_add(std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xc>{});  // row_bcast:31
        const double before = tot - run;
#pragma unroll
        for (int v = 0; v < TPL; ++v) sv[v] += before;
        // Sums at the ends of the 32-token blocks, e(m) = min(32m + 31, Qc - 1)
        // (uniform lanes and slots, read from their registers).
        double se[NBLK];
#pragma unroll
        for (int m = 0; m < NBLK; ++m) {
            const int e = min(kStep * m + kStep - 1, Qc - 1);
            double v = sv[0];
#pragma unroll
            for (int k = 1; k < TPL; ++k) v = e % TPL == k ? sv[k] : v;
            se[m] = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), e / TPL),
                                     __builtin_amdgcn_readlane(__double2loint(v), e / TPL));
        }
        const int mb = i0 / kStep;  // the lane's 32-token block
        double sl = se[0];
#pragma unroll
        for (int m = 1; m < NBLK; ++m) sl = mb == m ? se[m] : sl;
        // se[NBLK - 1] is the sum at the block's last token Qc - 1.
        typedef float FV __attribute__((ext_vector_type(TPL)));
        FV c, ct, de, wv;
#pragma unroll
        for (int v = 0; v < TPL; ++v) {
            const bool in = i0 + v < Qc;
            c[v] = (float)(a * sv[v] * kLog2eD);
            ct[v] = in ? c[v] - log2f(dtr[v]) : __builtin_inff();
            de[v] = in ? dtr[v] * exp_neg((float)(a * (sl - sv[v]))) : 0.f;
            wv[v] = in ? dtr[v] * exp_neg((float)(a * (se[NBLK - 1] - sv[v]))) : 0.f;
        }
        *reinterpret_cast<FV *>(tb + TB_CS2 + i0) = c;
        *reinterpret_cast<FV *>(tb + TB_CT + i0) = ct;
        *reinterpret_cast<FV *>(tb + TB_DTE + i0) = de;
        *reinterpret_cast<FV *>(tb + TB_WL + i0) = wv;
        // cs2 at the end e(m) of each 32-token block m (lane m < NBLK).
        if (ln < NBLK) {
            double sm = se[0];
#pragma unroll
            for (int m = 1; m < NBLK; ++m) sm = ln == m ? se[m] : sm;
            tb[TB_CE + ln] = (float)(a * sm * kLog2eD);
        }
    };

    // ---- per-lane LDS bases of the fragment reads (bytes); every read adds
    // an immediate offset.
    // Transposing reads (k = tokens): source lane il = 4kr + a points at
    // token row 4grp + kr (and +16), columns 16t + 4a .. +3; lane il then
    // holds column 16t + il of token rows 4grp + r (slots 0-3) and
    // 16 + 4grp + r (slots 4-7).
    const int rl = 4 * grp + (il >> 2);
    const int xT = rl * SX + 8 * (il & 3);                      // x fragments (+32 per p tile)
    const int bT = rl * SB + 8 * (il & 3) + 32 * nw * NTW;      // B^T fragments of the wave's state n tiles
    const int xS = xT + 32 * pw * PTW;                          // x fragments of the wave's state p tiles
    // 16-byte row reads: B (G: rows 16half + il, piece 4ks + grp) and h
    // (blue: rows p = 16q + il, piece 4ks + grp).
    const int bR = il * SB + 16 * grp;
    const int hR = il * SH + 16 * grp;
    auto lds16 = [&](const char *ptr) __attribute__((always_inline)) {
        Frag<T> f;
        f.v = *reinterpret_cast<const bf16x8 *>(ptr);
        return f;
    };
    // Transposing read of two 16-token halves, `half` bytes apart.
    auto read_tr = [&](const char *ptr, int half) __attribute__((always_inline)) {
        const i16x4 a0 = ds_read_tr16(reinterpret_cast<const T *>(ptr));
        const i16x4 a1 = ds_read_tr16(reinterpret_cast<const T *>(ptr + half));
        Frag<T> f;
        f.v = __builtin_bit_cast(bf16x8, i16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]});
        return f;
    };
    // The per-token factors of the lane's k slots in 32-token block m:
    // tokens 32m + 4grp + r and 32m + 16 + 4grp + r.
    auto slot_pair = [&](const float *row, int m, f32x4 &w0, f32x4 &w1) __attribute__((always_inline)) {
        int g4 = 4 * grp;  // opaque: recomputed here rather than kept (or spilled) across the loop
        asm volatile("" : "+v"(g4));
        w0 = *reinterpret_cast<const f32x4 *>(row + kStep * m + g4);
        w1 = *reinterpret_cast<const f32x4 *>(row + kStep * m + 16 + g4);
    };

    // ---- running state, tiles of S^T: hs[a][q][r] = h[p = 16(pw PTW + q) + il][n = 16(nw NTW + a) + 4grp + r]
    f32x4 hs[NTW][PTW];
    // Element offsets of the lane's state values within h[P][N], from an
    // opaque lane index (used rarely; not worth registers across the loop).
    auto state_offsets = [&](uint32_t (&so)[NTW][PTW]) __attribute__((always_inline)) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int a = 0; a < NTW; ++a)
#pragma unroll
            for (int q = 0; q < PTW; ++q)
                so[a][q] = (uint32_t)((16 * (pw * PTW + q) + (ln & 15)) * N + 16 * (nw * NTW + a) + 4 * (ln >> 4));
    };
    // Accepted index of the item's sequence, clamped to [-1, L-1] (-1 when
    // no state is asked for at an index).
    auto j_of = [&](const Step &st) -> int64_t {
        if (!p.state_out) return -2;
        const int j = ((const __attribute__((address_space(4))) int *)(uintptr_t)p.state_out_idx)[st.b];
        return j < 0 ? -1 : min((int64_t)j, L - 1);
    };
    // The item's rows of a head's state, as a buffer: item * P * N = (bh * PF
    // + s * P) * N.  With on = false (or no tensor) it covers no bytes.
    auto state_rows = [&](const float *base, const Step &st, bool on) {
        return rsrc(base + (int64_t)st.item * P * N, on && base != nullptr ? (uint32_t)(P * N * 4) : 0u);
    };
    // State loads and stores are rare (an item's first and last steps, and
    // the step holding its accepted index) and issued only where needed.
    // A unit starts from h_{-1}, the initial state (or 0), loaded at the
    // switch into it and waited for there: a load still in flight into the
    // state on one path would make the compiler wait for every load in
    // flight wherever the state is next used, on every path.
    auto load_init = [&](const Step &st) __attribute__((always_inline)) {
        if (p.init_state) {
            const auto r = state_rows(p.init_state, st, true);
            uint32_t so[NTW][PTW];
            state_offsets(so);
#pragma unroll
            for (int a = 0; a < NTW; ++a)
#pragma unroll
                for (int q = 0; q < PTW; ++q)
                    hs[a][q] =
                        __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 4 * so[a][q], 0, 0));
            wait_vmcnt<0>();
        } else {
#pragma unroll
            for (int a = 0; a < NTW; ++a)
#pragma unroll
                for (int q = 0; q < PTW; ++q) hs[a][q] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };
    auto store_state = [&](float *base, const Step &st, const f32x4 (&v)[NTW][PTW])
        __attribute__((always_inline)) {
        const auto r = state_rows(base, st, true);
        uint32_t so[NTW][PTW];
        state_offsets(so);
#pragma unroll
        for (int a = 0; a < NTW; ++a)
#pragma unroll
            for (int q = 0; q < PTW; ++q)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v[a][q]), r, 4 * so[a][q], 0, 0);
    };
    auto dh_of = [&](const Step &st) {
        return p.D ? ((const __attribute__((address_space(4))) float *)(uintptr_t)p.D)[st.h] : 0.f;
    };

    // ---- per-block factors (uniform).
    float ce[NBLK];   // cs2 at the end of each 32-token block
    int Qc = 0, nblk = 0;
    bool live = false, full = false;

    // Switch to a step: its x and B rows have landed, its tables are in tb
    // (and every wave has finished the previous step's LDS reads).
    auto enter = [&](const Step &st, const float *tb) __attribute__((always_inline)) {
        Qc = block_len(st.c);
        nblk = (Qc + kStep - 1) / kStep;
        full = st.c >= st.c0;
        live = full && 16 * tile < Qc;
        const int t = otid();
        const int lx = (t / WX) * SX + 16 * (t % WX), lb = (t / WB) * SB + 16 * (t % WB);
#pragma unroll
        for (int u = 0; u < UBR; ++u) *reinterpret_cast<V8 *>(bl + lb + u * RB * SB) = br[u];
#pragma unroll
        for (int u = 0; u < UXR; ++u) *reinterpret_cast<V8 *>(xs + lx + u * RX * SX) = xr[u];
        if (full && (st.c > 0 || p.init_state)) {  // blue reads h_{c-1} in bf16
#pragma unroll
            for (int a = 0; a < NTW; ++a)
#pragma unroll
                for (int q = 0; q < PTW; ++q) {
                    const int pp = 16 * (pw * PTW + q) + il, n = 16 * (nw * NTW + a) + 4 * grp;
                    *reinterpret_cast<V4 *>(hb + pp * SH + 2 * n) =
                        V4{(T)hs[a][q][0], (T)hs[a][q][1], (T)hs[a][q][2], (T)hs[a][q][3]};
                }
        }
#pragma unroll
        for (int m = 0; m < NBLK; ++m)
            ce[m] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(tb[TB_CE + m])));
    };

    // Blue for the wave's rows: exp(cs_i) C_i . h_{c-1} (rows p, column i).
    auto blue = [&](const float cs2i, f32x4 (&acc)[PT]) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < PT; ++q)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) mma(lds16(hb + hR + 16 * q * SH + 64 * ks), cf[ks], acc[q]);
        const float ei = exp2_hw(cs2i);
#pragma unroll
        for (int q = 0; q < PT; ++q) acc[q] = acc[q] * ei;
    };
    // G^T of 32-token block m, half `half`, for the wave's rows: lane (il,
    // grp) holds G^T[j][i], i = 16 tile + il, j = 32m + 16half + 4grp + r.
    auto g_half = [&](int m, int half) __attribute__((always_inline)) {
        f32x4 a4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) mma(lds16(bl + bR + (kStep * m + 16 * half) * SB + 64 * ks), cf[ks], a4);
        return a4;
    };
    // Orange factors of block m below the diagonal block md: G times
    // exp2(cs2_i - cs2_e(m)) dte_j, rounded to bf16 once (applied to raw x).
    auto orange_below = [&](int m, const float *tb, float cs2i) __attribute__((always_inline)) {
        const float ai = exp2_hw(cs2i - ce[m]);
        f32x4 w0, w1;
        slot_pair(tb + TB_DTE, m, w0, w1);
        Frag<T> gf;
        const f32x4 g0 = g_half(m, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) gf.set(r, g0[r] * (ai * w0[r]));
        const f32x4 g1 = g_half(m, 1);
#pragma unroll
        for (int r = 0; r < 4; ++r) gf.set(4 + r, g1[r] * (ai * w1[r]));
        return gf;
    };
    // Orange factors of the diagonal block md: G times the exact factors
    // exp2(cs2_i - ct_j) (the exponent is at most log2(dt_j) for j <= i;
    // above the diagonal the product is replaced by 0), plus D at j = i (the
    // skip term), rounded to bf16 once (applied to raw x).  j - i = 16 half +
    // r - di, with di from an opaque copy so that the comparisons are made
    // here and not kept across the loop.
    auto orange_diag = [&](const float *tb, float cs2i, float dh, int mdo, int todd) __attribute__((always_inline)) {
        int di = 16 * todd + il - 4 * grp;
        asm volatile("" : "+v"(di));
        f32x4 ct0, ct1;
        slot_pair(tb + TB_CT, mdo, ct0, ct1);
        Frag<T> lf;
        const f32x4 g0 = g_half(mdo, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            // above the diagonal the factor may overflow; the select drops it
            const float v = r > di ? 0.f : g0[r] * exp2_hw(cs2i - ct0[r]);
            lf.set(r, r == di ? v + dh : v);
        }
        if (todd) {
            const f32x4 g1 = g_half(mdo, 1);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float v = 16 + r > di ? 0.f : g1[r] * exp2_hw(cs2i - ct1[r]);
                lf.set(4 + r, 16 + r == di ? v + dh : v);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) lf.set(4 + r, 0.f);  // rows above the diagonal
        }
        return lf;
    };
    // y, rounded; rows past the sequence fall outside the buffer (and with
    // on = false every store is dropped).  y is written once and not read
    // here: non-temporal stores keep it from displacing the B and C rows the
    // other heads still read.  Lane (il, grp) holds channels 16q + 4grp .. +3
    // of row il; the four lanes of a row swap values (through the LDS
    // permute) so that lane g holds the 16-byte pieces g and 4 + g (channels
    // 8g .. +7 and 32 + 8g .. +7) of row il.  With 64 channels, lanes il and
    // il ^ 8 then swap one piece (a DPP row rotation) so that each of the two
    // stores writes 8 whole 128-byte rows: partial lines would cost the
    // memory a read-modify-write.
    auto store_y = [&](const Step &st, bool on, const f32x4 (&acc)[PT]) __attribute__((always_inline)) {
        const auto r = y_rows(st, on);
        int ln = lane;  // opaque: the shuffle sources are recomputed here
        asm volatile("" : "+v"(ln));
        const int g = ln >> 4, s0 = ((ln & 15) + 32 * (g & 1)) << 2, s1 = s0 + 64;
        u32x2 o[PT];
#pragma unroll
        for (int q = 0; q < PT; ++q)
            o[q] = __builtin_bit_cast(u32x2, V4{(T)acc[q][0], (T)acc[q][1], (T)acc[q][2], (T)acc[q][3]});
        u32x4 d[PT / 2];  // d[k]: piece 4k + g of row il
#pragma unroll
        for (int k = 0; k < PT / 2; ++k) {
            u32x4 w[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {  // channels 16(2k + j) + 4grp' .., grp' = 2(g & 1) and 2(g & 1) + 1
                const u32x2 v = o[2 * k + j];
                w[j] = u32x4{(unsigned)__builtin_amdgcn_ds_bpermute(s0, (int)v[0]),
                             (unsigned)__builtin_amdgcn_ds_bpermute(s0, (int)v[1]),
                             (unsigned)__builtin_amdgcn_ds_bpermute(s1, (int)v[0]),
                             (unsigned)__builtin_amdgcn_ds_bpermute(s1, (int)v[1])};
            }
            d[k] = (g >> 1) ? w[1] : w[0];
        }
        if constexpr (PT == 4) {
            const bool lo = (ln & 8) == 0;
            const u32x4 x = lo ? d[1] : d[0];
            u32x4 rcv;
#pragma unroll
            for (int e = 0; e < 4; ++e)  // row_ror:8 within each row of 16 lanes: lane il ^ 8
                rcv[e] = (unsigned)__builtin_amdgcn_update_dpp(0, (int)x[e], 0x128, 0xf, 0xf, false);
            // lane (il, g) writes piece g + 4 (il >> 3) of rows (il & 7) and (il & 7) + 8
            const uint32_t vy = (uint32_t)(16 * tile + (ln & 7)) * HP2 + 16 * (g + 4 * ((ln >> 3) & 1));
            __builtin_amdgcn_raw_buffer_store_b128(lo ? d[0] : rcv, r, vy, 0, kAuxNt);
            __builtin_amdgcn_raw_buffer_store_b128(lo ? rcv : d[1], r, vy + 8 * HP2, 0, kAuxNt);
        } else {
            const uint32_t vyr = (uint32_t)(16 * tile + (ln & 15)) * HP2 + 16 * g;
#pragma unroll
            for (int k = 0; k < PT / 2; ++k) __builtin_amdgcn_raw_buffer_store_b128(d[k], r, vyr + 64 * k, 0, kAuxNt);
        }
    };

    // The state after an accepted index j in this step (position jl, 32-token
    // block mj), from the state entering the step (hs, before the step's
    // update): h_j = exp(cs_j) h_{c-1} + sum over tokens s <= j of B_s^T x_s
    // with the exact factors exp2(cs2_j - ct_s), into hv.  Runs at most once
    // per item.
    auto state_at_index = [&](const float *tb, int jl, f32x4 (&hv)[NTW][PTW]) __attribute__((always_inline)) {
        const int mj = jl / kStep;
        const float ej = exp2_hw(tb[TB_CS2 + jl]);
#pragma unroll
        for (int a = 0; a < NTW; ++a)
#pragma unroll
            for (int q = 0; q < PTW; ++q) hv[a][q] = hs[a][q] * ej;
        const float cs2j = tb[TB_CS2 + jl];
        for (int m = 0; m <= mj; ++m) {
            Frag<T> fa[NTW];
#pragma unroll
            for (int a = 0; a < NTW; ++a) fa[a] = read_tr(bl + bT + kStep * m * SB + 32 * a, 16 * SB);
            int j4 = jl - 4 * grp;  // slot r of half 0 is token 32m + 4grp + r
            asm volatile("" : "+v"(j4));
            f32x4 c0, c1, w0, w1;
            slot_pair(tb + TB_CT, m, c0, c1);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                w0[r] = kStep * m + r > j4 ? 0.f : exp2_hw(cs2j - c0[r]);
                w1[r] = kStep * m + 16 + r > j4 ? 0.f : exp2_hw(cs2j - c1[r]);
            }
#pragma unroll
            for (int a = 0; a < NTW; ++a) scale_frag(fa[a], w0, w1);
#pragma unroll
            for (int q = 0; q < PTW; ++q) {
                const Frag<T> fb = read_tr(xs + xS + kStep * m * SX + 32 * q, 16 * SX);
#pragma unroll
                for (int a = 0; a < NTW; ++a) mma(fa[a], fb, hv[a][q]);
            }
        }
    };

    // One step (tables in tb).  With the outputs (a full step): blue, then
    // one pass over the 32-token blocks m that reads each block's x
    // fragments once for both products: the orange part of the wave's rows
    // (m <= md) and the state update
    //   h_c = exp(cs_last) h_{c-1} + sum_j wl_j B_j^T x_j,
    //   wl_j = dt_j exp(cs_last - cs_j) <= dt_j  (the weighted B fragment
    //   formed from the transposed B read and rounded once),
    // then y.  The next step's C rows are fetched once the wave's last
    // C . B^T product is issued, and wave 0 makes the next step's tables at
    // the end of its work (its rows meet the fewest blocks).
    auto compute = [&](const Step &st, bool has_next, const Step &nx, const float *tb, float *tb_next)
        __attribute__((always_inline)) {
        // The next step's dt (for its tables, made at the end of this step)
        // and its x and B rows (written to LDS at the switch): issued here,
        // outside the switch, so that no wave waits at a barrier for their
        // issue, and a whole step covers their latency.
        load_dt(nx, has_next);  // first: see load_dt
        load_x(nx, has_next);
        load_b(nx, has_next);
        {
            // state_out: the state after the accepted index j if j lies in
            // this step, the initial state if j = -1 (in the item's first step).
            const int64_t j = full ? j_of(st) : -2;
            if (j >= 0 && j / Q == st.c) {
                f32x4 hv[NTW][PTW];
                state_at_index(tb, (int)(j - (int64_t)st.c * Q), hv);
                store_state(p.state_out, st, hv);
            } else if (j == -1 && st.c == 0) {
                store_state(p.state_out, st, hs);
            }
        }
        f32x4 acc[PT];
#pragma unroll
        for (int q = 0; q < PT; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        const float cs2i = tb[TB_CS2 + 16 * tile + il];
        const float dh = dh_of(st);
        if (live && (st.c > 0 || p.init_state != nullptr)) blue(cs2i, acc);
        // md and the tile's parity from opaque copies: the compiler would
        // otherwise hoist every comparison with them out of the loop as a
        // 64-bit lane mask and keep (spill) them all.
        int mdo = md, todd = tile & 1;
        asm volatile("" : "+s"(mdo), "+s"(todd));
        const float gl = exp2_hw(ce[NBLK - 1]);  // exp(cs_last)
#pragma unroll
        for (int a = 0; a < NTW; ++a)
#pragma unroll
            for (int q = 0; q < PTW; ++q) hs[a][q] = hs[a][q] * gl;
        static_for<NBLK>([&](auto mc) __attribute__((always_inline)) {
            constexpr int m = decltype(mc)::value;
            if (m >= nblk) return;
            const bool orange = live && m <= mdo;
            Frag<T> of;
            if (live && m < mdo) of = orange_below(m, tb, cs2i);
            if (live && m == mdo) of = orange_diag(tb, cs2i, dh, mdo, todd);
            Frag<T> fa[NTW];
#pragma unroll
            for (int a = 0; a < NTW; ++a) fa[a] = read_tr(bl + bT + kStep * m * SB + 32 * a, 16 * SB);
            f32x4 w0, w1;
            slot_pair(tb + TB_WL, m, w0, w1);
#pragma unroll
            for (int a = 0; a < NTW; ++a) scale_frag(fa[a], w0, w1);
            // Each x fragment of the block feeds the orange product of the
            // wave's rows and the state update of the wave's p tiles
            // pw PTW .. pw PTW + PTW - 1.
#pragma unroll
            for (int q = 0; q < PT; ++q) {
                const Frag<T> xf = read_tr(xs + xT + kStep * m * SX + 32 * q, 16 * SX);
                if (orange) mma(xf, of, acc[q]);
                if (Cf::WPP == 1 || q / PTW == pw) {
#pragma unroll
                    for (int a = 0; a < NTW; ++a) mma(fa[a], xf, hs[a][q % PTW]);
                }
            }
        });
        if (st.c + 1 == st.c1 && st.c1 == nb) store_state(p.final_state, st, hs);  // the item's last step
        load_c(nx, has_next && nx.c >= nx.c0);
        store_y(st, live, acc);
        if (has_next && wave == 0) make_tables(nx, tb_next);
    };

    // ---- prologue: the first step's inputs and tables.  The tables of
    // step s are in tb0 / tb1 for s even / odd, made by wave 0 at the end
    // of step s - 1 from the dt values fetched at its start.
    Step cur = step_of(0);
    load_dt(cur, true);
    load_x(cur, true);
    load_b(cur, true);
    load_c(cur, cur.c >= cur.c0);
    wait_vmcnt<0>();
    if (wave == 0) make_tables(cur, tb0);
    lds_barrier();  // the tables are written
    load_init(cur);
    enter(cur, tb0);
    lds_barrier();

    // ---- steps.
    for (int s = 0; s < nsteps; ++s) {
        const bool has_next = s + 1 < nsteps;
        const Step nx = has_next ? next_step(cur) : cur;
        float *tbc = (s & 1) ? tb1 : tb0, *tbn = (s & 1) ? tb0 : tb1;
        compute(cur, has_next, nx, tbc, tbn);
        // Wait for the next step's x and B rows, not for this step's y
        // stores or the next step's C rows issued after them: a wave's vector
        // memory operations complete in the order they were issued.
        wait_vmcnt<KS + PT / 2>();
        // The switch runs after the last step too (nothing was loaded for
        // it), so that every path round the loop issues the same memory
        // operations and the compiler's count of loads in flight is exact.
        lds_barrier();  // every wave has finished this step's LDS reads; next tables written
        if (has_next && nx.c == 0) load_init(nx);
        enter(nx, tbn);
        lds_barrier();
        cur = nx;
    }
}

template <int NT, int PT, int QB>
hipError_t launch_cfg(const Params &p, hipStream_t stream) {
    using Cf = FusedCfg<NT, PT, QB>;
    if constexpr (!Cf::OK) {
        return hipErrorNotSupported;
    } else {
        const int grid = Cf::WGS_PER_CU * compute_units();
        hipLaunchKernelGGL((chunk_scan_fused_kernel<NT, PT, QB>), dim3((unsigned)grid), dim3(Cf::THREADS), 0, stream,
                           p);
        return hipGetLastError();
    }
}

// The block length: 256 tokens with one 16-wave workgroup per compute unit
// where that geometry exists, else 128 tokens with two 8-wave workgroups.
template <int NT, int PT>
hipError_t launch_q(const Params &p, hipStream_t stream) {
#ifndef SSD_FUSED_Q
#define SSD_FUSED_Q 128
#endif
    if constexpr (SSD_FUSED_Q == 256 && FusedCfg<NT, PT, 256>::OK) return launch_cfg<NT, PT, 256>(p, stream);
    else return launch_cfg<NT, PT, 128>(p, stream);
}

template <int NT>
hipError_t dispatch_p(const Params &p, hipStream_t stream) {
    switch (p.headdim) {
        case 32: return launch_q<NT, 2>(p, stream);
        case 64: return launch_q<NT, 4>(p, stream);
        case 128: return launch_q<NT, 4>(p, stream);  // two 64-channel items per head
        default: return hipErrorNotSupported;
    }
}

}  // namespace

bool chunk_scan_fused_takes(const Params &p) {
    const int64_t items = p.batch * p.nheads * (p.headdim == 128 ? 2 : 1);
    // 32-bit byte offsets of one block's rows of x and y.
    const int64_t row_bytes = (int64_t)p.nheads * p.headdim * 2;
    return items >= kFusedMinItems && items < ((int64_t)1 << 30) && p.seqlen >= 1 &&
           row_bytes * 256 < ((int64_t)1 << 31) && (int64_t)p.ngroups * p.dstate * 2 * 256 < ((int64_t)1 << 31) &&
           (p.dstate == 64 || p.dstate == 128) && (p.headdim == 32 || p.headdim == 64 || p.headdim == 128);
}

hipError_t launch_chunk_scan_fused(const Params &p, hipStream_t stream) {
    if (!chunk_scan_fused_takes(p)) return hipErrorNotSupported;
    switch (p.dstate) {
        case 64: return dispatch_p<4>(p, stream);
        case 128: return dispatch_p<8>(p, stream);
        default: return hipErrorNotSupported;
    }
}

}  // namespace ssd
