// Chunk states, head-batched (bf16): the green part of the SSD block
// decomposition for all heads of one B/C group in one workgroup.
//
// "Transformers are SSMs" article (cloud.tencent.com.cn), section "SSD算法":
// the green blocks are batched products; section "深入解析分块与状态传递机制":
// each chunk's final state from a zero initial state.  For chunk c, head h of
// group g:
//     S_c[p][n] = sum_{j in chunk} w_j x_j[p] B_j[n],   w_j = exp(cs_last - cs_j) dt_j
//               = sum_j x_j[p] B_j[n] exp2(cs2_last - ct_j),
// with cs2 = cs log2(e) and ct_j = cs2_j - log2(dt_j) from the cumsum tables
// (the argument is at most log2(dt_j); ct = +inf past the sequence gives 0).
//
// B_c does not depend on the head, so a workgroup owns (b, c, g, a slice of
// the group's heads): it copies the chunk's B rows into LDS once (direct
// global -> LDS copies) and then, per head, scales the head's x rows by w_j
// once (fp32, rounded to bf16 to nearest even) into an LDS buffer and forms
// S_c^T = B_c^T (w x) on the matrix cores, both operands read with the
// transposing LDS read (rows are tokens).  x is prefetched into registers
// two heads ahead; two LDS buffers alternate, one barrier per head.
//
// dstate 256 with 256-token chunks: the chunk's B rows (128 KB) and two x
// buffers do not fit in LDS together.  There each of the 8 waves owns 32 of
// the 256 n columns and keeps their B fragments for the whole chunk in
// registers (8 token blocks x 2 tiles), read once at the start from B rows
// staged through the x buffers; per head only x goes through LDS, and every
// wave reads all of it.  Holding B in LDS instead would need the n columns
// split over two workgroups, each reading and scaling x again, for twice the
// LDS bytes per head.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

constexpr int kXcds = 8;
constexpr int kWaves = 8;
constexpr int kStep = 32;  // tokens per contraction block

template <int NT, int PT, int NIT>
struct StateCfg {
    static constexpr int N = NT * 16, P = PT * 16;
    static constexpr int QP = NIT * 16 < kStep ? kStep : NIT * 16;  // token rows held
    static constexpr int NB = QP / kStep;                           // token blocks
    // B fragments held in registers (dstate 256, 256-token chunks, headdim <= 64).
    static constexpr bool BREG = NT == 16 && NIT == 16 && PT <= 4;
    // Otherwise n is split over NS workgroups when one chunk's B rows and
    // two x buffers do not fit in LDS; each workgroup then holds the NL
    // columns of B it contracts.
    static constexpr int NS = BREG || (size_t)(QP * N + 2 * QP * P) * 2 <= 160 * 1024 ? 1 : 2;
    static constexpr int NL = N / NS;
    static constexpr int WB = NL / 8, WX = P / 8;                  // 16-byte pieces per B / x row
    // Waves along p: with B in registers one (each wave all of p); else the
    // split of the NL x P tile over the 8 waves that reads the fewest LDS
    // bytes per token (n and p columns per wave).
    static constexpr int cost(int wp) { return NL / (kWaves / wp) + P / wp; }
    static constexpr int WP = BREG ? 1
                            : PT >= 2 && cost(2) <= cost(PT < kWaves ? PT : kWaves) ? 2
                            : (PT < kWaves ? PT : kWaves);
    static constexpr int WN = kWaves / WP;                         // waves along n
    static constexpr int PTW = PT / WP, NTW = NL / 16 / WN;         // tiles per wave
    static constexpr int IB = QP * WB / 64;                        // 1 KB copies of B
    static constexpr int UB = (IB + kWaves - 1) / kWaves;
    // Register-held B: rows staged per round through both x buffers.
    static constexpr int RROWS = 2 * QP * P / N;
    static constexpr int UBR = RROWS * WB / 64 / kWaves;           // 1 KB copies per wave and round
    static constexpr int XPC = QP * WX;                            // 16-byte pieces of one head's x
    static constexpr int UXR = (XPC + 64 * kWaves - 1) / (64 * kWaves);  // per thread
    static constexpr size_t LDS_BYTES = (size_t)((BREG ? 0 : QP * NL) + 2 * QP * P) * 2;
    static constexpr bool OK = NTW >= 1 && (NL / 16) % WN == 0 && WB >= 2 && WX >= 2 && LDS_BYTES <= 160 * 1024 &&
                               (!BREG || (RROWS % kStep == 0 && QP % RROWS == 0 && UBR * 64 * kWaves == RROWS * WB));
};

template <int NT, int PT, int NIT>
__global__ __launch_bounds__(64 * kWaves) void chunk_state_heads_kernel(Params p, int hps, int nslices) {
    using Cf = StateCfg<NT, PT, NIT>;
    using T = bf16;
    constexpr int N = Cf::N, NL = Cf::NL, P = Cf::P, QP = Cf::QP, WB = Cf::WB, WX = Cf::WX;
    constexpr int PTW = Cf::PTW, NTW = Cf::NTW, UXR = Cf::UXR, NS = Cf::NS, NB = Cf::NB;
    constexpr bool BREG = Cf::BREG;
    typedef typename Vec8<T>::type V8;

    __shared__ __align__(16) T bl[BREG ? 8 : QP * NL];
    __shared__ __align__(16) T xl[2 * QP * P];  // two x buffers (and the B staging area when B is in registers)
    auto xbuf = [&](auto bc) __attribute__((always_inline)) -> T * { return xl + decltype(bc)::value * QP * P; };

    const int Q = p.chunk, H = p.nheads, G = p.ngroups, nc = p.nchunks, HPG = p.heads_per_group;
    const int64_t L = p.seqlen;

    // Workgroup -> (b, c, g, slice, n part); the slices and n parts of one
    // (b, c) run back to back on one XCD (the n parts of a slice read the
    // same x rows, which the second one finds in that XCD's L2).
    const int64_t total = p.batch * nc * G * nslices * NS;
    const int64_t per_xcd = gridDim.x / kXcds;
    const int64_t logical = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (logical >= total) return;
    const int npart = (int)(logical % NS);
    const int64_t lg = logical / NS;
    const int slice = (int)(lg % nslices);
    const int g = (int)((lg / nslices) % G);
    const int c = (int)((lg / ((int64_t)nslices * G)) % nc);
    const int64_t b = lg / ((int64_t)nslices * G * nc);
    const int hbeg = g * HPG + slice * hps;
    const int hcnt = min(hps, HPG - slice * hps);
    if (hcnt <= 0) return;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int il = lane & 15, grp = lane >> 4;
    const int64_t t0 = (int64_t)c * Q;
    const int Qc = (int)(L - t0 < Q ? L - t0 : Q);

    const T *xg = reinterpret_cast<const T *>(p.x);
    const T *bg = reinterpret_cast<const T *>(p.B);

    // ---- B rows of the chunk -> LDS (rows past the chunk repeat its last
    // token: finite, and they meet w = 0).
    if constexpr (!BREG) {
        const T *bsrc = bg + ((b * L + t0) * G + g) * N + npart * NL;
#pragma unroll
        for (int u = 0; u < Cf::UB; ++u) {
            const int ins = wave + kWaves * u;
            if (ins < Cf::IB) {
                const int U = 64 * ins + lane;
                const int row = U / WB, pos = U - row * WB;
                const int j = min(row, Qc - 1);
                copy16_to_lds(bsrc + (int64_t)j * G * N + 8 * (pos ^ swz_tr<WB>(row)), bl + ins * 512);
            }
        }
    }

    // ---- x of one head: each thread holds UXR 16-byte pieces (row, piece)
    // and the ct value of each piece's row.  x is read here once per call
    // and not again until the output kernel: non-temporal loads keep it from
    // displacing the chunk states this kernel writes from the last-level
    // cache (256 MB), where the state pass then finds them (measured at the
    // long-sequence shape: state pass 66 -> 42 us, this kernel 67 -> 62 us).
    V8 xa[UXR], xc[UXR];
    float ca[UXR], cc[UXR];
    auto load_x = [&](int hh, V8 (&xr)[UXR], float (&cr)[UXR]) __attribute__((always_inline)) {
        const int h = hbeg + hh;
        const T *xsrc = xg + ((b * L + t0) * H + h) * P;
        const int64_t trow = ((b * H + h) * nc + c) * (int64_t)Q;
#pragma unroll
        for (int u = 0; u < UXR; ++u) {
            const int U = tid + 64 * kWaves * u;
            if (Cf::XPC % (64 * kWaves) == 0 || U < Cf::XPC) {
                const int row = U / WX, pos = U - row * WX;
                const int j = min(row, Qc - 1);
                xr[u] = __builtin_nontemporal_load(reinterpret_cast<const V8 *>(xsrc + (int64_t)j * H * P + 8 * (pos ^ swz_tr<WX>(row))));
                // (every row is inside the chunk when the rows held are the chunk)
                cr[u] = (QP == NIT * 16 || row < Q) ? p.ct[trow + row] : __builtin_inff();
            }
        }
    };
    // Scale by w_j and store into an LDS buffer (16-byte pieces in place).
    auto store_x = [&](int hh, auto bc, const V8 (&xr)[UXR], const float (&cr)[UXR]) __attribute__((always_inline)) {
        const int h = hbeg + hh;
        const int64_t trow = ((b * H + h) * nc + c) * (int64_t)Q;
        const float cs2_last = ((const __attribute__((address_space(4))) float *)(uintptr_t)p.cs)[trow + Qc - 1] * kLog2e;
        T *xd = xbuf(bc);
#pragma unroll
        for (int u = 0; u < UXR; ++u) {
            const int U = tid + 64 * kWaves * u;
            if (Cf::XPC % (64 * kWaves) == 0 || U < Cf::XPC) {
                const float w = exp2_hw(cs2_last - cr[u]);
                V8 v;
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = (T)(w * (float)xr[u][e]);
                *reinterpret_cast<V8 *>(xd + 8 * U) = v;
            }
        }
    };

    // Wave tiles: p tiles pw*PTW.., n tiles nw*NTW..
    const int pw = wave % Cf::WP, nw = wave / Cf::WP;
    // Per-lane offsets of the transposing reads: source lane (il = 4*kr + a)
    // points at row 16*half + 4*grp + kr, columns 16*tile + 4*a .. +3.
    const int rl = 4 * grp + (il >> 2);
    int boff[NTW], xoff[PTW];
#pragma unroll
    for (int a = 0; a < NTW; ++a) {
        const int t = nw * NTW + a;
        boff[a] = rl * NL + 8 * ((2 * t + ((il & 3) >> 1)) ^ swz_tr<WB>(rl)) + 4 * (il & 1);
    }
#pragma unroll
    for (int q = 0; q < PTW; ++q) {
        const int t = pw * PTW + q;
        xoff[q] = rl * P + 8 * ((2 * t + ((il & 3) >> 1)) ^ swz_tr<WX>(rl)) + 4 * (il & 1);
    }
    // One 32-token block of a 16-column tile: rows 0..15 and 16..31 of the
    // block through the transposing read (ld = row stride in elements).
    auto read_block = [&](Frag<T> &f, const T *src, int ld) __attribute__((always_inline)) {
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        const i16x4 u0 = ds_read_tr16(src);
        const i16x4 u1 = ds_read_tr16(src + 16 * ld);
        f.v = __builtin_bit_cast(bf16x8, i16x8{u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]});
    };
    // Register-held B fragments: block m, tile a of this wave.
    Frag<T> fr[BREG ? NB : 1][NTW];

    auto head = [&](auto bc, int hh) __attribute__((always_inline)) {
        constexpr int BI = decltype(bc)::value;
        lds_barrier();  // head hh's scaled x is in buffer BI for every wave (and B, for the first)
        const T *xs = xbuf(bc);
        f32x4 acc[NTW][PTW];
#pragma unroll
        for (int a = 0; a < NTW; ++a)
#pragma unroll
            for (int q = 0; q < PTW; ++q) acc[a][q] = f32x4{0.f, 0.f, 0.f, 0.f};
        // All QP/kStep blocks, unrolled so that the fragment reads of later
        // blocks are issued while earlier products run.  In the last chunk
        // of a sequence the blocks past its end hold zero-weighted x rows
        // (ct = +inf there) and add exact zeros.
#pragma unroll
        for (int m = 0; m < NB; ++m) {
            const T *xm = xs + kStep * m * P;
            Frag<T> fa[NTW], fb[PTW];
#pragma unroll
            for (int a = 0; a < NTW; ++a) {
                if constexpr (BREG) fa[a] = fr[m][a];
                else read_block(fa[a], bl + kStep * m * NL + boff[a], NL);
            }
#pragma unroll
            for (int q = 0; q < PTW; ++q) read_block(fb[q], xm + xoff[q], P);
#pragma unroll
            for (int a = 0; a < NTW; ++a)
#pragma unroll
                for (int q = 0; q < PTW; ++q) mma(fa[a], fb[q], acc[a][q]);
        }
        // Next head's x: scale and store into the other buffer (it was last
        // read by head hh-1, which every wave finished before the barrier).
        {
            const int hn = min(hh + 1, hcnt - 1);
            if constexpr (BI == 0) store_x(hn, std::integral_constant<int, 1>{}, xc, cc);
            else store_x(hn, std::integral_constant<int, 0>{}, xa, ca);
        }
        // ... and the one after it into the freed registers.
        {
            const int hn = min(hh + 3, hcnt - 1);
            if constexpr (BI == 0) load_x(hn, xc, cc);
            else load_x(hn, xa, ca);
        }
        // acc[a][q][r] = S^T[n = npart*NL + 16*(nw*NTW + a) + 4*grp + r][p = 16*(pw*PTW + q) + il]
        const int h = hbeg + hh;
        bf16 *sd = reinterpret_cast<bf16 *>(p.states) + ((b * nc + c) * H + h) * (int64_t)P * N;
#pragma unroll
        for (int a = 0; a < NTW; ++a)
#pragma unroll
            for (int q = 0; q < PTW; ++q) {
                const int n = npart * NL + 16 * (nw * NTW + a) + 4 * grp, pp = 16 * (pw * PTW + q) + il;
                const f32x4 v = acc[a][q];
                *reinterpret_cast<bf16x4 *>(sd + (int64_t)pp * N + n) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
            }
    };

    // Prologue: heads 0 and 1 into registers, head 0 scaled into buffer 0,
    // head 2 into the freed registers.
    load_x(0, xa, ca);
    if (hcnt > 1) load_x(1, xc, cc);
    if constexpr (BREG) {
        // B rows through the x buffers, RROWS at a time, into this wave's
        // fragments (rows past the chunk repeat its last token, as above).
        constexpr int RR = Cf::RROWS;
        const T *bsrc = bg + ((b * L + t0) * G + g) * N;
#pragma unroll
        for (int r = 0; r < QP / RR; ++r) {
            if (r > 0) lds_barrier();  // every wave has read the previous round's rows
#pragma unroll
            for (int u = 0; u < Cf::UBR; ++u) {
                const int ins = wave + kWaves * u;
                const int U = 64 * ins + lane;
                const int row = U / WB, pos = U - row * WB;
                const int j = min(r * RR + row, Qc - 1);
                copy16_to_lds(bsrc + (int64_t)j * G * N + 8 * (pos ^ swz_tr<WB>(row)), xl + ins * 512);
            }
            wait_vmcnt<0>();  // this wave's copies (and the x loads before them) have landed
            lds_barrier();    // ... and every wave's
#pragma unroll
            for (int mm = 0; mm < RR / kStep; ++mm)
#pragma unroll
                for (int a = 0; a < NTW; ++a) read_block(fr[r * (RR / kStep) + mm][a], xl + kStep * mm * N + boff[a], N);
        }
        lds_barrier();  // every wave holds its fragments before x overwrites the staging rows
    }
    store_x(0, std::integral_constant<int, 0>{}, xa, ca);
    if (hcnt > 2) load_x(2, xa, ca);
    if constexpr (!BREG) wait_vmcnt<0>();  // (also) this wave's B copies have landed; the barrier opening head 0 covers all waves
    for (int h0 = 0; h0 < hcnt; h0 += 2) {
        head(std::integral_constant<int, 0>{}, h0);
        if (h0 + 1 < hcnt) head(std::integral_constant<int, 1>{}, h0 + 1);
    }
}

template <int NT, int PT, int NIT>
hipError_t launch_nit(const Params &p, hipStream_t stream) {
    using Cf = StateCfg<NT, PT, NIT>;
    if constexpr (!Cf::OK) {
        return hipErrorNotSupported;
    } else {
        const int64_t base = p.batch * p.nchunks * (int64_t)p.ngroups * Cf::NS;
        int nslices = (int)std::min<int64_t>(p.heads_per_group, std::max<int64_t>(1, (256 + base - 1) / base));
        const int hps = (p.heads_per_group + nslices - 1) / nslices;
        nslices = (p.heads_per_group + hps - 1) / hps;
        // Few heads per workgroup do not repay loading B into LDS once
        // (measured: the per-head kernel is faster at 4 heads of 128-token
        // chunks).  Register-held B is taken at any count: the per-head
        // kernel reads the chunk's B rows once per head.
        if (!Cf::BREG && hps < 8 && p.chunk > 32) return hipErrorNotSupported;
        const int64_t total = base * nslices;  // n parts included
        const int64_t per_xcd = (total + kXcds - 1) / kXcds;
        hipLaunchKernelGGL((chunk_state_heads_kernel<NT, PT, NIT>), dim3((unsigned)(per_xcd * kXcds)),
                           dim3(64 * kWaves), 0, stream, p, hps, nslices);
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

hipError_t launch_chunk_state_heads(const Params &p, hipStream_t stream) {
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
