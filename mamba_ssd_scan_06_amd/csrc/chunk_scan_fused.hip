// Single-pass SSD forward (bf16): one workgroup at a time per (sequence b,
// head h) walks the chunks in order and keeps the running state in registers, so all
// four parts of the block decomposition of "Transformers are SSMs"
// (cloud.tencent.com.cn, section "SSD算法") run in one kernel: the chunk
// states and the states entering each chunk never reach memory, x is read
// once and y written once.  The state passing is the sequential scan over
// chunks that section "深入解析分块与状态传递机制" describes, here carried
// by the workgroup itself.
//
// Chunk c (tokens t0 .. t0+Qc-1, head h of group g), with cs the chunk-local
// cumulative log-decay, cs2 = cs log2(e), ct = cs2 - log2(dt), e(m) the last
// token of 32-token block m and dte_j = dt_j exp(cs_e(m) - cs_j) for j in m
// (the tables of the cumsum kernel, which also gives cs2_e(m) and the
// state's Horner factors per block):
//   G      = C_c B_c^T (causal 16x32 tiles, bf16, nearest even)
//   orange y_i  = sum_{j<=i} exp(cs_i - cs_j) dt_j G_ij x_j
//   blue   y_i += exp(cs_i) C_i . h_{c-1}
//   green  h_c  = exp(cs_last) h_{c-1} + sum_j exp(cs_last - cs_j) dt_j x_j B_j^T
//          y_i += D_h x_i.
// Decay factors.  Outside the diagonal blocks every factor splits into the
// per-token dte_j, applied once to x (xd = dte x, rounded to bf16), and
// factors of at most 1 that depend on the block only:
//   orange, block m < md (md the tile's diagonal block): G_ij times
//     exp2(cs2_i - cs2_e(m)), rounded to bf16, on xd;
//   blue: exp2(cs2_i) times C_i . h_{c-1};
//   state, in Horner form: acc = h_{c-1}; acc = acc g_m + B_m^T xd_m over the
//     chunk's blocks, g_0 = exp2(cs2_e(0)), g_m = exp2(cs2_e(m) - cs2_e(m-1)),
//     which leaves h_c (e of the last block is the chunk's last token).
// The diagonal block keeps the exact factor exp2(cs2_i - ct_j) per element
// on raw x (the mask applied through the exponent), so it stays exact
// however strong the decay inside a block; the skip term D x_i enters as D
// added to its j = i coefficient before rounding.
//
// Channels: the rows p of the state are independent (each is its own
// recurrence), so a head of headdim 128 is run as two items of 64 channels
// each, which share dt, B and C and own their columns of x and y and their
// rows of the state.
//
// Work split: NIT = Q/16 waves, each owning one 16-row tile (balanced so
// that every SIMD meets the same number of causal blocks) and, for the
// state, NTW x PTW of its 16x16 tiles.  LDS holds the chunk's B rows, x and
// xd rows (token-major, read with the transposing LDS read) and h_{c-1} in
// bf16.  While chunk c computes, chunk c+1's x and B rows are loaded into
// registers and its tables copied to LDS; its C rows follow once chunk c no
// longer needs them.  At the switch every wave waits for its loads and
// writes the next chunk's LDS, and one barrier publishes them.  y is stored
// before the state part, whose products cover the stores' latency.  Global
// accesses go through buffer descriptors over each chunk's rows, with fixed
// per-lane offsets.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

constexpr int kXcds = 8;
constexpr int kStep = 32;  // tokens per j block
constexpr int kSpinLimit = 1 << 20;  // polls before a hand-off wait gives up (well over 0.1 s)
constexpr int kAuxNt = 2;  // cache-policy operand of the buffer builtins: nt (non-temporal)

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

template <int NT, int PT, int NIT>
struct FusedCfg {
    static constexpr int N = NT * 16, P = PT * 16, Q = NIT * 16;
    static constexpr int W = NIT, THREADS = 64 * NIT;          // one 16-row tile per wave
    static constexpr int KS = N / 32;                            // 32-wide k steps over n
    static constexpr int WB = N / 8, WX = P / 8;                 // 16-byte pieces per B row, per x row
    static constexpr int NBLK = Q / kStep;
    static constexpr int WPN = NT < W ? NT : W, WPP = W / WPN;  // waves along n, p (state tiles)
    static constexpr int NTW = NT / WPN, PTW = PT / WPP;         // state tiles per wave
    static constexpr int UXR = Q * WX / THREADS;                 // 16-byte x pieces per thread
    static constexpr int UBR = Q * WB / THREADS;                 // 16-byte B pieces per thread
    static constexpr size_t LDS_BYTES =
        (size_t)Q * N * 2 + 2 * (size_t)Q * P * 2 + (size_t)P * N * 2 + 2 * 4 * 256 * 4;
    static constexpr bool OK = NIT >= 8 && NT >= 2 && NT % WPN == 0 && PT % WPP == 0 && PTW >= 1 &&
                               (Q * WX) % THREADS == 0 && UXR >= 1 && (Q * WB) % THREADS == 0 &&
                               LDS_BYTES <= 160 * 1024;
};

// Raw buffer descriptor over [base, base + bytes): loads beyond it read 0
// and stores beyond it are dropped, which takes care of rows past the end of
// the sequence.  Word 3 selects 32-bit data, the gfx9 value for untyped access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int NT, int PT, int NIT>
__global__ __launch_bounds__(64 * NIT) void chunk_scan_fused_kernel(Params p) {
    using Cf = FusedCfg<NT, PT, NIT>;
    using T = bf16;
    constexpr int N = Cf::N, P = Cf::P, Q = Cf::Q, KS = Cf::KS, WB = Cf::WB, WX = Cf::WX;
    constexpr int NBLK = Cf::NBLK, NTW = Cf::NTW, PTW = Cf::PTW, UXR = Cf::UXR, UBR = Cf::UBR;
    constexpr int THREADS = Cf::THREADS;
    constexpr int RX = THREADS / WX, RB = THREADS / WB;  // rows between a thread's x / B pieces
    static_assert(RX % 8 == 0 && RB % 8 == 0, "a thread's pieces share one swizzle");
    typedef typename Vec8<T>::type V8;
    typedef typename Vec4<T>::type V4;
    typedef short i16x8 __attribute__((ext_vector_type(8)));

    __shared__ __align__(16) T bl[Q * N];   // B rows, pieces swizzled for the transposing read
    __shared__ __align__(16) T xs[Q * P];   // x rows
    __shared__ __align__(16) T xd[Q * P];   // dte * x rows
    __shared__ __align__(16) T hb[P * N];   // h_{c-1} rows p, pieces swizzled for 16-byte reads
    // cs, ct, dte rows of a chunk; two objects so that reading one chunk's
    // while the next one's copies are in flight needs no wait for them.
    // (and the block factors, in the fourth 1 KB row).
    __shared__ __align__(16) float tb0[4 * 256], tb1[4 * 256];

    const int H = p.nheads, G = p.ngroups, nc = p.nchunks, HPG = p.heads_per_group;
    const int PF = p.headdim, PS = PF / P;  // channels of a head, items per head
    const int64_t L = p.seqlen;

    // ---- work of this workgroup (one per CU, persistent).  A unit is the
    // chunks [cb, ce) of one item, (b, h, channel half s): item (b*H + h)*PS + s.  Workgroups are
    // dealt to the XCDs in turn (w % 8), and each XCD takes a contiguous
    // range of items, so that the heads sharing B and C rows run on one
    // XCD and share its L2.  Within an XCD, with Ix items on Wx workgroups,
    // each takes F = Ix / Wx whole items; the R = Ix % Wx left over are cut
    // in two halves of their chunks when 2R <= Wx: workgroups 0..R-1 run a
    // first half before their whole items, workgroups R..2R-1 a second half
    // after theirs, taking the state entering it from the first half
    // (written long before it is needed).  Every workgroup then runs F or
    // F + 1/2 items' chunks instead of F or F + 1.
    const int Wg = gridDim.x;
    const int NX = Wg % kXcds == 0 ? kXcds : 1;
    const int xcd = (int)blockIdx.x % NX, w = (int)blockIdx.x / NX, Wx = Wg / NX;
    const int64_t I = p.batch * H * PS;
    const int64_t Ibase = I / NX, Iext = I % NX;
    const int64_t Ix = Ibase + (xcd < Iext ? 1 : 0);
    const int64_t ibeg = xcd * Ibase + min((int64_t)xcd, Iext);  // first item of this XCD
    const int F = (int)(Ix / Wx), R = (int)(Ix - (int64_t)F * Wx);
    const bool split = F >= 1 && R > 0 && 2 * R <= Wx && nc >= 2;
    const int nch = nc / 2;
    const int nunits = F + (split ? (w < 2 * R ? 1 : 0) : (w < R ? 1 : 0));
    struct Unit {
        int64_t item;
        int cb, ce;
    };
    auto unit = [&](int k) -> Unit {
        if (split && w < R) {
            if (k == 0) return Unit{ibeg + (int64_t)F * Wx + w, 0, nch};
            return Unit{ibeg + w + (int64_t)Wx * (k - 1), 0, nc};
        }
        if (split && w < 2 * R && k == F) return Unit{ibeg + (int64_t)F * Wx + (w - R), nch, nc};
        return Unit{ibeg + w + (int64_t)Wx * k, 0, nc};
    };
    if (nunits == 0) return;
    // A step is one chunk of one unit; steps run in order k, then c.
    // (b, h, g of the item are worked out once per unit; items fit 32 bits
    // since batch and nheads are at most 65535.)
    struct Step {
        int k, c;
        int64_t item;
        int cb, ce;
        int64_t b, bh;  // bh = b*H + h
        int h, g, s;
    };
    auto step_of = [&](int k, int c) -> Step {
        const Unit u = unit(k);
        const uint32_t it = (uint32_t)u.item, bh = it / (uint32_t)PS, hh = bh % (uint32_t)H;
        return Step{k,           c,        u.item,  u.cb, u.ce, (int64_t)(bh / (uint32_t)H), (int64_t)bh,
                    (int)hh,     (int)hh / HPG, (int)(it - bh * (uint32_t)PS)};
    };
    auto next_step = [&](const Step &st) -> Step {
        if (st.c + 1 < st.ce) {
            Step n = st;
            n.c = st.c + 1;
            return n;
        }
        return step_of(st.k + 1, unit(st.k + 1).cb);
    };
    int nsteps = 0;
    for (int k = 0; k < nunits; ++k) nsteps += unit(k).ce - unit(k).cb;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int il = lane & 15, grp = lane >> 4;
    const int tile = wide_tile<NIT>(wave), md = tile >> 1;
    // Waves meet md off-diagonal blocks each, so the chunk lasts as long as
    // the waves with the most; issue priority grows with md (0 .. 3), so the
    // others fill the gaps (a SIMD's four waves together meet the same number).
    const int prio = md * 4 / NBLK;
    if (prio >= 3)
        __builtin_amdgcn_s_setprio(3);
    else if (prio == 2)
        __builtin_amdgcn_s_setprio(2);
    else if (prio == 1)
        __builtin_amdgcn_s_setprio(1);
    const int nw = wave % Cf::WPN, pw = wave / Cf::WPN;  // the wave's state tiles

    const uint32_t HP2 = (uint32_t)H * PF * 2, GN2 = (uint32_t)G * N * 2;  // bytes per token row
    auto chunk_len = [&](int c) -> int { return (int)min((int64_t)Q, L - (int64_t)c * Q); };
    // Token rows of a step's chunk: x and y of its head, B and C of its group.
    auto x_rows = [&](const Step &st) {
        return rsrc((const T *)p.x + ((st.b * L + (int64_t)st.c * Q) * H + st.h) * PF + st.s * P,
                    chunk_len(st.c) * HP2);
    };
    auto y_rows = [&](const Step &st) {
        return rsrc((const T *)p.y + ((st.b * L + (int64_t)st.c * Q) * H + st.h) * PF + st.s * P,
                    chunk_len(st.c) * HP2);
    };
    auto b_rows = [&](const Step &st) {
        return rsrc((const T *)p.B + ((st.b * L + (int64_t)st.c * Q) * G + st.g) * N, chunk_len(st.c) * GN2);
    };
    auto c_rows = [&](const Step &st) {
        return rsrc((const T *)p.C + ((st.b * L + (int64_t)st.c * Q) * G + st.g) * N, chunk_len(st.c) * GN2);
    };

    // ---- per-lane offsets, fixed for the whole loop.
    // Global (bytes): the thread's 16-byte pieces of x and B rows, its C
    // fragments (row 16 tile + il, columns 8grp + 32ks) and its y values
    // (row 16 tile + il, columns 4grp + 16q).
    const uint32_t vx = (uint32_t)(tid / WX) * HP2 + (tid % WX) * 16;
    const uint32_t vb = (uint32_t)(tid / WB) * GN2 + (tid % WB) * 16;
    const uint32_t vc = (uint32_t)(16 * tile + il) * GN2 + grp * 16;
    const uint32_t vy = (uint32_t)(16 * tile + il) * HP2 + grp * 8;
    // LDS (elements): where those x and B pieces go (piece swizzles depend on
    // the row modulo 8, the same for all of a thread's pieces).
    const int lx = (tid / WX) * P + 8 * ((tid % WX) ^ swz_tr<WX>(tid / WX));
    const int lb = (tid / WB) * N + 8 * ((tid % WB) ^ swz_tr<WB>(tid / WB));

    V8 xr[UXR], br[UBR];
    Frag<T> cf[KS];  // C rows of the wave's tile (phase A and blue)
    auto load_x = [&](const Step &st) __attribute__((always_inline)) {
        const auto r = x_rows(st);
#pragma unroll
        for (int u = 0; u < UXR; ++u)
            xr[u] = __builtin_bit_cast(V8, __builtin_amdgcn_raw_buffer_load_b128(r, vx, u * RX * HP2, 0));
    };
    auto load_b = [&](const Step &st) __attribute__((always_inline)) {
        const auto r = b_rows(st);
#pragma unroll
        for (int u = 0; u < UBR; ++u)
            br[u] = __builtin_bit_cast(V8, __builtin_amdgcn_raw_buffer_load_b128(r, vb, u * RB * GN2, 0));
    };
    auto load_c = [&](const Step &st) __attribute__((always_inline)) {
        const auto r = c_rows(st);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            cf[ks].v = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, vc + 64 * ks, 0, 0));
    };
    // Table rows of chunk c (one 1 KB copy per table, waves 0-2) and its
    // block factors (64 bytes, wave 3; its other lanes repeat the last piece).
    static_assert(Cf::W >= 4, "four waves copy the tables");
    auto issue_tables = [&](const Step &st, float *dst) __attribute__((always_inline)) {
        const int64_t row = (st.bh * nc + st.c) * (int64_t)Q;  // tables are [b,H,nc,Q]
        int ln = lane;
        asm volatile("" : "+v"(ln));
        if (wave < 3)
            copy16_to_lds((wave == 0 ? p.cs : wave == 1 ? p.ct : p.dte) + row + 4 * min(ln, Q / 4 - 1),
                          dst + 256 * wave);
        else if (wave == 3)
            copy16_to_lds(p.blk + (st.bh * nc + st.c) * (int64_t)kBlkStride + 4 * min(ln, kBlkStride / 4 - 1),
                          dst + 768);
    };

    // ---- per-lane LDS offsets of the fragment reads (elements).  Every
    // swizzle period divides 16 (rows) or 8 (tokens), so a fragment address
    // is a per-lane constant plus a uniform base.
    // Transposing reads (k = tokens): source lane il = 4kr + a points at
    // token row 4grp + kr (and +16), columns 16t + 4a .. +3.
    const int rl = 4 * grp + (il >> 2);
    int xo[PT];  // x / xd fragments of p tile q
#pragma unroll
    for (int q = 0; q < PT; ++q) xo[q] = rl * P + 8 * ((2 * q + ((il & 3) >> 1)) ^ swz_tr<WX>(rl)) + 4 * (il & 1);
    int xos[PTW];  // xd fragments of the wave's state p tiles
#pragma unroll
    for (int q = 0; q < PTW; ++q) {
        const int t = pw * PTW + q;
        xos[q] = rl * P + 8 * ((2 * t + ((il & 3) >> 1)) ^ swz_tr<WX>(rl)) + 4 * (il & 1);
    }
    int bo[NTW];  // B^T fragments of the wave's state n tiles
#pragma unroll
    for (int a = 0; a < NTW; ++a) {
        const int t = nw * NTW + a;
        bo[a] = rl * N + 8 * ((2 * t + ((il & 3) >> 1)) ^ swz_tr<WB>(rl)) + 4 * (il & 1);
    }
    // 16-byte row reads of B (phase A: rows 16a + il, piece 4ks + grp) and of
    // h (blue: rows p = 16q + il, piece 4ks + grp).
    int ro_b[KS], ro_h[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        ro_b[ks] = il * N + 8 * ((4 * ks + grp) ^ swz_tr<WB>(il));
        ro_h[ks] = il * N + 8 * ((4 * ks + grp) ^ swz_rows16<WB>(il));
    }
    auto read_tr = [&](const T *base, int off, int ld) __attribute__((always_inline)) {
        const i16x4 a0 = ds_read_tr16(base + off);
        const i16x4 a1 = ds_read_tr16(base + 16 * ld + off);
        Frag<T> f;
        f.v = __builtin_bit_cast(bf16x8, i16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]});
        return f;
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
    // The item's state handed from a first half to a second half: its rows
    // of entry [b, 0, h] of the workspace's chunk-state region, and its flag.
    auto handoff_rsrc = [&](const Step &st) {
        return buffer_rsrc(p.states + (((st.b * nc) * H + st.h) * PF + st.s * P) * (int64_t)N, (uint32_t)(P * N * 4));
    };
    int *handoff_flag = p.sync + kSyncHeader;
    auto flag_of = [&](const Step &st) { return st.bh * kFlagsPerHead + st.s; };
    bool gave_up = false;  // a hand-off wait timed out (the wave waits no more)
    // Start a unit: h_{cb-1} is the initial state (or 0) for cb = 0, else
    // the state the first half handed over.
    auto begin_unit = [&](const Step &st) __attribute__((always_inline)) {
        uint32_t so[NTW][PTW];
        state_offsets(so);
        // item * P * N = (bh * PF + s * P) * N: the item's rows of its head's state
        const int64_t hst = st.item * (int64_t)P * N;
        if (st.cb == 0) {
#pragma unroll
            for (int a = 0; a < NTW; ++a)
#pragma unroll
                for (int q = 0; q < PTW; ++q)
                    hs[a][q] = p.init_state ? *reinterpret_cast<const f32x4 *>(p.init_state + hst + so[a][q])
                                            : f32x4{0.f, 0.f, 0.f, 0.f};
        } else {
            if (!gave_up && !wait_flag_device(handoff_flag + flag_of(st), kSpinLimit)) {
                gave_up = true;
                set_flag_device(p.sync + 1, 1);
            }
            const auto r = handoff_rsrc(st);
#pragma unroll
            for (int a = 0; a < NTW; ++a)
#pragma unroll
                for (int q = 0; q < PTW; ++q) hs[a][q] = load_f4_device(r, 4 * so[a][q]);
        }
    };
    // End a unit (hs = h_{ce-1}): the final state, or the hand-off.
    auto end_unit = [&](const Step &st) __attribute__((always_inline)) {
        uint32_t so[NTW][PTW];
        state_offsets(so);
        if (st.ce == nc) {
            if (p.final_state) {
                const int64_t hst = st.item * (int64_t)P * N;
#pragma unroll
                for (int a = 0; a < NTW; ++a)
#pragma unroll
                    for (int q = 0; q < PTW; ++q)
                        *reinterpret_cast<f32x4 *>(p.final_state + hst + so[a][q]) = hs[a][q];
            }
        } else {
            const auto r = handoff_rsrc(st);
#pragma unroll
            for (int a = 0; a < NTW; ++a)
#pragma unroll
                for (int q = 0; q < PTW; ++q) store_f4_device(r, 4 * so[a][q], hs[a][q]);
            wait_vmcnt<0>();  // every store of this wave is visible device-wide ...
            barrier_only();   // ... and of every wave
            if (wave == 0) set_flag_device(handoff_flag + flag_of(st), 1);
        }
    };
    // Chunk whose entering state goes to hj (state_out at an index of -1 asks
    // for the initial state, which enters chunk 0), and the skip weight.
    auto cj_of = [&](const Step &st) {
        if (!(p.hj && p.state_out_idx)) return -1;
        const int j = ((const __attribute__((address_space(4))) int *)(uintptr_t)p.state_out_idx)[st.b];
        return j < 0 ? 0 : (int)(min((int64_t)j, L - 1) / Q);
    };
    auto dh_of = [&](const Step &st) {
        return p.D ? ((const __attribute__((address_space(4))) float *)(uintptr_t)p.D)[st.h] : 0.f;
    };

    // ---- per-chunk block factors (uniform).
    float ce[NBLK];   // cs2 at the end of each block
    float gst[NBLK];  // state Horner factors: exp(cs_e(0)), exp(cs_e(m) - cs_e(m-1))
    int Qc = 0, nblk = 0;
    bool live = false, has_prev = false;

    // Switch to chunk c: its x, B and tables have landed (and every wave has
    // finished chunk c-1's LDS reads).
    auto enter = [&](const Step &st, const float *tb) __attribute__((always_inline)) {
        const int c = st.c;
        Qc = chunk_len(c);
        nblk = (Qc + kStep - 1) / kStep;
        live = 16 * tile < Qc;
        has_prev = c > 0 || p.init_state != nullptr;
        // LDS: B rows, x and dte x rows (0 past the sequence), h_{c-1}.
#pragma unroll
        for (int u = 0; u < UBR; ++u) *reinterpret_cast<V8 *>(bl + lb + u * RB * N) = br[u];
#pragma unroll
        for (int u = 0; u < UXR; ++u) {
            *reinterpret_cast<V8 *>(xs + lx + u * RX * P) = xr[u];
            int t = tid;  // opaque copy: the row index is recomputed here, not kept (or spilled)
            asm volatile("" : "+v"(t));
            const float d = tb[512 + t / WX + u * RX];
            V8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (T)(d * (float)xr[u][e]);
            *reinterpret_cast<V8 *>(xd + lx + u * RX * P) = v;
        }
        if (has_prev) {
#pragma unroll
            for (int a = 0; a < NTW; ++a)
#pragma unroll
                for (int q = 0; q < PTW; ++q) {
                    const int pp = 16 * (pw * PTW + q) + il, n = 16 * (nw * NTW + a) + 4 * grp;
                    *reinterpret_cast<V4 *>(hb + pp * N + 8 * ((n >> 3) ^ swz_rows16<WB>(pp)) + (n & 7)) =
                        V4{(T)hs[a][q][0], (T)hs[a][q][1], (T)hs[a][q][2], (T)hs[a][q][3]};
                }
        }
        if (c == cj_of(st)) {
            uint32_t so[NTW][PTW];
            state_offsets(so);
            const int64_t hst = st.item * (int64_t)P * N;
#pragma unroll
            for (int a = 0; a < NTW; ++a)
#pragma unroll
                for (int q = 0; q < PTW; ++q) *reinterpret_cast<f32x4 *>(p.hj + hst + so[a][q]) = hs[a][q];
        }
        // Block factors of the chunk (copied with the tables; uniform).
#pragma unroll
        for (int m = 0; m < NBLK; ++m) {
            ce[m] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(tb[768 + m])));
            gst[m] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(tb[768 + kBlkStride / 2 + m])));
        }
    };

    // One chunk (tables in tb): blue, orange and D skip, stored; then the state.
    auto compute = [&](const Step &st, bool has_next, const Step &nx, const float *tb) __attribute__((always_inline)) {
        const int c = st.c;
        const float dh = dh_of(st);
        const float cs2i = tb[16 * tile + il] * kLog2e;
        f32x4 acc[PT];
#pragma unroll
        for (int q = 0; q < PT; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        // Blue: exp(cs_i) C_i . h_{c-1} (rows p, column i).
        if (has_prev && live) {
#pragma unroll
            for (int q = 0; q < PT; ++q)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    Frag<T> hf;
                    load8(hf, hb + 16 * q * N + ro_h[ks]);
                    mma(hf, cf[ks], acc[q]);
                }
            const float ei = exp2_hw(cs2i);
#pragma unroll
            for (int q = 0; q < PT; ++q) acc[q] = acc[q] * ei;
        }
        // G^T of block m, half `half`, for the wave's rows: lane (il, grp)
        // holds G^T[j][i], i = 16 tile + il, j = 32m + 16half + 4grp + r.
        auto g_half = [&](int m, int half) __attribute__((always_inline)) {
            f32x4 a4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                Frag<T> bf;
                load8(bf, bl + (kStep * m + 16 * half) * N + ro_b[ks]);
                mma(bf, cf[ks], a4);
            }
            return a4;
        };
        // Orange off the diagonal: G times its row factor
        // exp2(cs2_i - cs2_e(m)) <= 1, rounded to bf16 once, on dte x.
        static_for<NBLK - 1>([&](auto mc) __attribute__((always_inline)) {
            constexpr int m = decltype(mc)::value;
            if (!live || m >= md) return;
            const float ai = exp2_hw(cs2i - ce[m]);
            Frag<T> gf;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const f32x4 a4 = g_half(m, half);
#pragma unroll
                for (int r = 0; r < 4; ++r) gf.set(4 * half + r, a4[r] * ai);
            }
#pragma unroll
            for (int q = 0; q < PT; ++q) mma(read_tr(xd + kStep * m * P, xo[q], P), gf, acc[q]);
        });
        // Diagonal block md: G times the exact factors exp2(cs2_i - ct_j)
        // (the exponent is at most log2(dt_j) for j <= i; above the diagonal
        // it is set to -inf, which masks G), plus D at j = i (the skip term),
        // rounded to bf16 once, on raw x.  j - i = 16 half + r - di, with di
        // from an opaque copy so that the comparisons are made here and not
        // kept across the chunk loop.
        if (live) {
            int di = 16 * (tile & 1) + il - 4 * grp;
            asm volatile("" : "+v"(di));
            int g4 = 4 * grp;  // opaque: recomputed here rather than kept (or spilled) across the loop
            asm volatile("" : "+v"(g4));
            const f32x4 ct0 = *reinterpret_cast<const f32x4 *>(tb + 256 + kStep * md + g4);
            const f32x4 ct1 = *reinterpret_cast<const f32x4 *>(tb + 256 + kStep * md + 16 + g4);
            const float ninf = -__builtin_inff();
            Frag<T> lf;
            const f32x4 g0 = g_half(md, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float v = g0[r] * exp2_hw(r > di ? ninf : cs2i - ct0[r]);
                lf.set(r, r == di ? v + dh : v);
            }
            if (tile & 1) {
                const f32x4 g1 = g_half(md, 1);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float v = g1[r] * exp2_hw(16 + r > di ? ninf : cs2i - ct1[r]);
                    lf.set(4 + r, 16 + r == di ? v + dh : v);
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) lf.set(4 + r, 0.f);  // rows above the diagonal
            }
#pragma unroll
            for (int q = 0; q < PT; ++q) mma(read_tr(xs + kStep * md * P, xo[q], P), lf, acc[q]);
        }
        // y, rounded; rows past the sequence fall outside the buffer.  y is
        // written once and not read here: non-temporal stores (kAuxNt) keep
        // it from displacing the B and C rows the other heads still read.
        // Lane (il, grp) holds channels 16q + 4grp .. +3 of row il; the four
        // lanes of a row swap values so that lane g holds channels
        // 32k + 8g .. +7 for k < PT/2 and each store writes 64 contiguous
        // bytes of every row (whole 64-byte pieces, no partial writes).
        if (live) {
            const auto r = y_rows(st);
            int ln = lane;  // opaque: the shuffle sources are recomputed here
            asm volatile("" : "+v"(ln));
            const int g = ln >> 4, s0 = ((ln & 15) + 32 * (g & 1)) << 2, s1 = s0 + 64;
            u32x2 o[PT];
#pragma unroll
            for (int q = 0; q < PT; ++q)
                o[q] = __builtin_bit_cast(u32x2, V4{(T)acc[q][0], (T)acc[q][1], (T)acc[q][2], (T)acc[q][3]});
            const uint32_t vyr = (uint32_t)(16 * tile + (ln & 15)) * HP2 + 16 * g;
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
                __builtin_amdgcn_raw_buffer_store_b128((g >> 1) ? w[1] : w[0], r, vyr + 64 * k, 0, kAuxNt);
            }
        }
        // C rows of the next chunk (cf is no longer needed).
        if (has_next) load_c(nx);
        // State: h_c = exp(cs_last) h_{c-1} + B^T (w x), Horner over the blocks.
        static_for<NBLK>([&](auto mc) __attribute__((always_inline)) {
            constexpr int m = decltype(mc)::value;
            if (m >= nblk) return;
            Frag<T> fa[NTW], fb[PTW];
#pragma unroll
            for (int a = 0; a < NTW; ++a) fa[a] = read_tr(bl + kStep * m * N, bo[a], N);
#pragma unroll
            for (int q = 0; q < PTW; ++q) fb[q] = read_tr(xd + kStep * m * P, xos[q], P);
#pragma unroll
            for (int a = 0; a < NTW; ++a)
#pragma unroll
                for (int q = 0; q < PTW; ++q) {
                    hs[a][q] = hs[a][q] * gst[m];
                    mma(fa[a], fb[q], hs[a][q]);
                }
        });
    };

    // ---- prologue: the first step's inputs.
    Step cur = step_of(0, unit(0).cb);
    issue_tables(cur, tb0);
    load_x(cur);
    load_b(cur);
    load_c(cur);
    wait_vmcnt<0>();
    barrier_only();  // every wave's table copies have landed
    begin_unit(cur);
    enter(cur, tb0);
    if (nsteps > 1) {
        const Step nx = next_step(cur);
        load_x(nx);
        load_b(nx);
        issue_tables(nx, tb1);
    }
    lds_barrier();

    // ---- steps, two per iteration so that each table buffer is a
    // compile-time choice.
    for (int s0 = 0; s0 < nsteps; s0 += 2) {
        static_for<2>([&](auto kc) __attribute__((always_inline)) {
            constexpr int K = decltype(kc)::value;
            const int s = s0 + K;
            if (s >= nsteps) return;
            const bool has_next = s + 1 < nsteps;
            const Step nx = has_next ? next_step(cur) : cur;
            compute(cur, has_next, nx, K == 0 ? tb0 : tb1);
            // The next step's loads and copies were issued before this
            // step's C rows; wait for all of them (after the last step too,
            // so that on every path into the next iteration the C rows have
            // landed and the compiler adds no wait for them).
            wait_vmcnt<0>();
            if (cur.c + 1 == cur.ce) end_unit(cur);
            if (has_next) {
                lds_barrier();  // every wave has finished this step's LDS reads
                if (nx.c == nx.cb) begin_unit(nx);
                enter(nx, K == 0 ? tb1 : tb0);
                if (s + 2 < nsteps) {
                    const Step nn = next_step(nx);
                    load_x(nn);
                    load_b(nn);
                    issue_tables(nn, K == 0 ? tb0 : tb1);
                }
                lds_barrier();
                cur = nx;
            }
        });
    }
}

template <int NT, int PT, int NIT>
hipError_t launch_cfg(const Params &p, hipStream_t stream) {
    using Cf = FusedCfg<NT, PT, NIT>;
    if constexpr (!Cf::OK) {
        return hipErrorNotSupported;
    } else {
        // One workgroup per CU (each takes one CU's LDS); never more than items.
        const int64_t items = p.batch * p.nheads * (p.headdim / Cf::P);
        const int64_t grid = std::min<int64_t>(items, compute_units());
        hipLaunchKernelGGL((chunk_scan_fused_kernel<NT, PT, NIT>), dim3((unsigned)grid), dim3(Cf::THREADS), 0,
                           stream, p);
        return hipGetLastError();
    }
}

template <int NT, int PT>
hipError_t dispatch_q(const Params &p, hipStream_t stream) {
    switch (p.chunk) {
        case 128: return launch_cfg<NT, PT, 8>(p, stream);
        case 256: return launch_cfg<NT, PT, 16>(p, stream);
        default: return hipErrorNotSupported;
    }
}

template <int NT>
hipError_t dispatch_p(const Params &p, hipStream_t stream) {
    switch (p.headdim) {
        case 32: return dispatch_q<NT, 2>(p, stream);
        case 64: return dispatch_q<NT, 4>(p, stream);
        case 128: return dispatch_q<NT, 4>(p, stream);  // two 64-channel items per head
        default: return hipErrorNotSupported;
    }
}

}  // namespace

hipError_t launch_chunk_scan_fused(const Params &p, hipStream_t stream) {
    // One workgroup per item and one CU each: with fewer than a CU's worth
    // of them the chunk-parallel kernels use the GPU better.
    if (p.batch * p.nheads * (p.headdim == 128 ? 2 : 1) < kFusedMinHeads) return hipErrorNotSupported;
    switch (p.dstate) {
        case 64: return dispatch_p<4>(p, stream);
        case 128: return dispatch_p<8>(p, stream);
        default: return hipErrorNotSupported;
    }
}

}  // namespace ssd
