// Sequence sharding (context parallelism): the correction a GPU applies to
// its shard once it knows the state entering the shard.
//
// "Transformers are SSMs" article (cloud.tencent.com.cn), section
// "序列并行的两种形式": with the sequence split across GPUs, the SSD form lets
// every GPU compute its local outputs and final state on its own, and only
// states travel between GPUs.  A shard [s0, s0+T) run from a zero initial
// state gives outputs y0_t and a final state F.  Because the recurrence is
// linear in the initial state, the outputs and states the shard would have
// had from its true entering state h_in differ from those by the pure decay
// of h_in:
//     y_t     = y0_t + exp(cs_t) C_t . h_in       (rows p: sum over n of C_t[n] h_in[p][n])
//     h_last  = F + exp(cs_{T-1}) h_in
//     h_j     = h0_j + exp(cs_j) h_in              (the state after an accepted index j)
// with cs_t = A_h * sum_{k<=t} dt_k the cumulative log-decay from the shard's
// first token (inclusive).  This is the blue part of the block decomposition
// with the whole shard as one chunk.
//
// One workgroup (4 waves) per (b, h, slice of at most 64 channels, range of
// 64-token blocks), about 256 workgroups in all, the ranges of one item on
// one XCD.  A range not starting at
// token 0 first sums dt over the tokens before it (fp64); h_in's slice is
// copied once, rounded to the input type, to LDS.  Per block: wave 0 scans
// the next block's dt in fp64 and writes its exp(cs_t) per token to LDS
// (one block ahead, off the other waves' path); every wave
// requests the next block's C fragments (its own 16 tokens, straight from
// memory into registers) and y pieces; wave w forms its 16 tokens x the
// slice's channels on the matrix cores (K = dstate, zero-padded to a
// multiple of 32; fp32 accumulation), scales each row by exp(cs_t) and
// writes the rows to LDS; then every thread adds the corrections to its 8
// consecutive channels of y (read during the previous block), rounds once
// and stores them.  The workgroup of the last range writes the final state;
// the one whose range holds the accepted index updates state_out.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

constexpr int kBlk = 64;      // tokens per block (4 waves x 16 rows)
constexpr int kThreads = 256;
constexpr int kMaxSlice = 64;  // channels per workgroup

template <typename T, int KS, int PT>
__global__ __launch_bounds__(kThreads) void state_correction_kernel(Params p, int ranges) {
    constexpr int NP = 32 * KS, PS = 16 * PT;  // padded dstate, channels of the slice
    // h_in rows padded by 16 bytes: the 16-byte-per-lane fragment reads of 16
    // consecutive rows then start on different banks.
    constexpr int LDH = NP + 16 / (int)sizeof(T), LDY = PS + 4;
    __shared__ __align__(16) T hs[PS * LDH];       // h_in slice, rows p
    __shared__ __align__(16) float cy[kBlk * LDY];  // exp(cs_t) C_t . h_in, rows t
    __shared__ float ev[2][kBlk];                  // exp(cs_t) of a block's tokens (two blocks)
    __shared__ double red[kThreads / kWave];
    __shared__ float cs_at[2];                     // cs at the accepted index, at the last token
    typedef typename Vec8<T>::type V8;
    typedef typename Vec4<T>::type V4;

    const int H = p.nheads, PF = p.headdim, N = p.dstate, G = p.ngroups;
    const int nsl = PF / PS;
    const int64_t L = p.seqlen;
    const int nblk = (int)((L + kBlk - 1) / kBlk);
    // Workgroup w runs on XCD w mod 8 (the hardware deals workgroups to the
    // XCDs in turn): the ranges of one item are given to workgroups of one
    // XCD, so that they share its L2 copy of the item's h_in slice.
    const unsigned nwg = gridDim.x, nx = nwg % 8 == 0 ? 8 : 1;
    const unsigned idx = (blockIdx.x % nx) * (nwg / nx) + blockIdx.x / nx;
    const int item = (int)(idx / (unsigned)ranges), r = (int)(idx % (unsigned)ranges);
    const int s = item % nsl, bh = item / nsl, h = bh % H;
    const int64_t b = bh / H;
    const int g = h / p.heads_per_group;
    // (Wave-uniform values marked as such, so that the buffer descriptors
    // built from them stay in scalar registers.)
    const int blk0 = __builtin_amdgcn_readfirstlane((int)((int64_t)r * nblk / ranges));
    const int blk1 = __builtin_amdgcn_readfirstlane((int)((int64_t)(r + 1) * nblk / ranges));
    const int tid = threadIdx.x, lane = tid & 63, il = lane & 15, grp = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const float a = L > 0 ? p.A[h] : 0.f;  // (A may be NULL for an empty shard)
    const int64_t t0 = (int64_t)blk0 * kBlk;
    const float *dtp = p.dt + b * L * H + h;  // dt of token t at dtp[t * H]
    const T *cg = reinterpret_cast<const T *>(p.C) + (b * L * G + g) * (int64_t)N;  // C row t at cg + t * G * N
    T *yg = reinterpret_cast<T *>(p.y) + (b * L * H + h) * (int64_t)PF + s * PS;   // y row t at yg + t * H * PF

    // Per-block buffer descriptors over the block's rows of C, y and dt: rows
    // past the shard, and every row of a block outside the range, read as
    // zero and take no stores.  Every path round the block loop then issues
    // the same loads and stores, so the compiler's count of loads in flight
    // is exact and no block waits for the next block's prefetch.
    constexpr int ESZ = (int)sizeof(T);
    auto rows_of = [&](int blk) -> int64_t {
        const int64_t tb = (int64_t)blk * kBlk;
        return blk < blk1 ? (L - tb < kBlk ? L - tb : kBlk) : 0;
    };
    auto c_rsrc = [&](int blk) {
        const int64_t n = rows_of(blk);
        return buffer_rsrc(cg + (int64_t)blk * kBlk * G * N, n > 0 ? (uint32_t)(((n - 1) * G * N + N) * ESZ) : 0u);
    };
    auto y_rsrc = [&](int blk) {
        const int64_t n = rows_of(blk);
        return buffer_rsrc(yg + (int64_t)blk * kBlk * H * PF, n > 0 ? (uint32_t)(((n - 1) * H * PF + PS) * ESZ) : 0u);
    };
    auto dt_rsrc = [&](int blk) {
        const int64_t n = rows_of(blk);
        return buffer_rsrc(dtp + (int64_t)blk * kBlk * H, n > 0 ? (uint32_t)(((n - 1) * H + 1) * 4) : 0u);
    };
    auto ld16 = [&](__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    };
    // The wave's C fragments of a block (token 16w + il, dstate 32ks + 8grp ..
    // +7: 16 or 32 contiguous bytes per lane), read one block ahead; zero
    // past dstate (dstate 16 pads the contraction to 32).
    Frag<T> fc[2][KS];
    auto load_c = [&](int blk, Frag<T> (&f)[KS]) __attribute__((always_inline)) {
        const auto rc = c_rsrc(blk);
        const uint32_t row = (uint32_t)(16 * wave + il) * G * N;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int n0 = 32 * ks + 8 * grp;
            const uint32_t off = (row + n0) * ESZ;
            if constexpr (sizeof(T) == 2) {
                f[ks].v = __builtin_bit_cast(bf16x8, ld16(rc, off));
            } else {
                f[ks].lo = __builtin_bit_cast(f32x4, ld16(rc, off));
                f[ks].hi = __builtin_bit_cast(f32x4, ld16(rc, off + 16));
            }
            // Only dstate 16 pads (one k step of 32); elsewhere n0 < N always.
            if constexpr (KS == 1)
                if (n0 >= N) f[ks].zero();
        }
    };
    // This thread's y pieces of a block (8 consecutive channels of one
    // token), read one block ahead.
    constexpr int YPIECES = kBlk * (PS / 8), YU = (YPIECES + kThreads - 1) / kThreads;
    static_assert(YPIECES % kThreads == 0 || YU == 1, "y pieces per thread");
    // Raw loaded bytes, converted where they are used (a conversion right
    // after the load would wait for it).
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    constexpr int YW = sizeof(T) == 2 ? 1 : 2;  // 16-byte words per piece
    u32x4 yv[2][YU][YW];
    auto yoff = [&](int u) -> uint32_t {
        const int e = tid + u * kThreads, row = e / (PS / 8), c0 = 8 * (e % (PS / 8));
        return (uint32_t)(row * H * PF + c0) * ESZ;
    };
    auto load_y = [&](int blk, u32x4 (&v)[YU][YW]) __attribute__((always_inline)) {
        const auto ry = y_rsrc(blk);
#pragma unroll
        for (int u = 0; u < YU; ++u) {
            if (tid + u * kThreads >= YPIECES) continue;  // (whole waves: YPIECES is a multiple of 64)
#pragma unroll
            for (int w = 0; w < YW; ++w) v[u][w] = __builtin_bit_cast(u32x4, ld16(ry, yoff(u) + 16 * w));
        }
    };
    load_c(blk0, fc[0]);
    load_y(blk0, yv[0]);

    // ---- sum of dt over the tokens before the range (fp64).
    // (Four independent partial sums, so that four loads are in flight.)
    double pre = 0.0;
    {
        double part[4] = {0.0, 0.0, 0.0, 0.0};
        const auto rp = buffer_rsrc(dtp, t0 > 0 ? (uint32_t)(((t0 - 1) * H + 1) * 4) : 0u);
        for (int64_t t = tid; t < t0; t += 4 * kThreads) {
            float v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                v[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                     rp, (int)((t + k * kThreads) * H * 4), 0, 0));
#pragma unroll
            for (int k = 0; k < 4; ++k) part[k] += (double)v[k];  // (past t0: read as zero)
        }
        pre = (part[0] + part[1]) + (part[2] + part[3]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) pre += __shfl_xor(pre, o);
    if (lane == 0) red[wave] = pre;
    // ---- h_in slice, rounded once to T, zero past dstate: 4 values per
    // thread and step, every load issued before the first store.
    {
        // (Unconditional loads through a descriptor over the slice: a load
        // under a condition gets a branch and a wait of its own.)
        const auto rh = buffer_rsrc(p.init_state + ((int64_t)bh * PF + (int64_t)s * PS) * N, (uint32_t)(PS * N * 4));
        constexpr int HPC = PS * NP / 4, HU = (HPC + kThreads - 1) / kThreads;
        f32x4 hv[HU];
#pragma unroll
        for (int u = 0; u < HU; ++u) {
            const int e = tid + u * kThreads, pp = e / (NP / 4), n = (e % (NP / 4)) * 4;
            hv[u] = __builtin_bit_cast(f32x4, ld16(rh, (uint32_t)(e < HPC ? (pp * N + n) * 4 : 0)));
        }
        if constexpr (KS == 1) {  // dstate 16: columns 16 .. 31 are padding
#pragma unroll
            for (int u = 0; u < HU; ++u)
                if (((tid + u * kThreads) % (NP / 4)) * 4 >= N) hv[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < HU; ++u) {
            const int e = tid + u * kThreads, pp = e / (NP / 4), n = (e % (NP / 4)) * 4;
            if (e < HPC) {
                if constexpr (sizeof(T) == 2)
                    *reinterpret_cast<V4 *>(hs + pp * LDH + n) = V4{(T)hv[u][0], (T)hv[u][1], (T)hv[u][2], (T)hv[u][3]};
                else
                    *reinterpret_cast<f32x4 *>(hs + pp * LDH + n) = hv[u];
            }
        }
    }
    if (tid < 2) cs_at[tid] = 0.f;
    __syncthreads();
    double run = 0.0;  // wave 0: sum of dt from the shard's first token to the last token done
    int64_t j = -2;  // accepted index of this sequence, clamped to [-1, L-1]
    if (p.state_out) {
        const int jj = p.state_out_idx[b];
        j = jj < 0 ? -1 : (jj < L ? jj : L - 1);
    }
    auto load_dt = [&](int blk) {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(dt_rsrc(blk), lane * H * 4, 0, 0));
    };
    // Wave 0: exp(cs_t) of block blk's tokens into ev[e] (zero past the shard
    // and for a block outside the range), from that block's dt values.
    auto scan = [&](int blk, float d, float *evb) __attribute__((always_inline)) {
        const int64_t t = (int64_t)blk * kBlk + lane;
        double inc = (double)d;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const double u = __shfl_up(inc, o);
            if (lane >= o) inc += u;
        }
        const float cs = (float)((double)a * (run + inc));
        evb[lane] = t < L ? exp_neg(cs) : 0.f;
        if (blk < blk1) {
            if (t == j) cs_at[0] = cs;
            if (t == L - 1) cs_at[1] = cs;
        }
        run += __shfl(inc, 63);
    };
    // dt of the token `lane` of the next block to scan (every wave requests
    // it, so that all waves issue the same loads; wave 0 uses it).
    float dtn = load_dt(blk0 + 1);
    if (wave == 0) {
#pragma unroll
        for (int w = 0; w < kThreads / kWave; ++w) run += red[w];
        scan(blk0, load_dt(blk0), ev[0]);
    }

    // One block with its fragments and y pieces in buffer BI (the next
    // block's go to the other buffer); the buffer index is a compile-time
    // constant so that both stay in registers.
    auto block = [&](auto bc, int blk) __attribute__((always_inline)) {
        constexpr int BI = decltype(bc)::value;
        // The table of the next block (wave 0, while the other waves start
        // this block's products); the dt of the block after it is requested.
        {
            const float d = dtn;
            dtn = load_dt(blk + 2);
            if (wave == 0) scan(blk + 1, d, ev[1 - BI]);
        }
        // The next block's C fragments and y pieces are requested before this
        // block's products.
        load_c(blk + 1, fc[1 - BI]);
        load_y(blk + 1, yv[1 - BI]);
        // Wave w: tokens 16w .. 16w+15 x channels of the slice.
        f32x4 acc[PT];
#pragma unroll
        for (int q = 0; q < PT; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int q = 0; q < PT; ++q) {
                Frag<T> fh;
                load8(fh, hs + (16 * q + il) * LDH + 32 * ks + 8 * grp);
                mma(fc[BI][ks], fh, acc[q]);
            }
        }
        __syncthreads();  // this block's table is written; the previous block's corrections are read
        // acc[q][rr] = (C_t . h_in)[p] for t = 16w + 4grp + rr, p = 16q + il.
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int row = 16 * wave + 4 * grp + rr;
            const float e = ev[BI][row];
#pragma unroll
            for (int q = 0; q < PT; ++q) cy[row * LDY + 16 * q + il] = acc[q][rr] * e;
        }
        __syncthreads();
        // y += correction, rounded once (stores past the shard, and of a
        // block outside the range, are dropped by the descriptor).
        const auto ry = y_rsrc(blk);
#pragma unroll
        for (int u = 0; u < YU; ++u) {
            const int e = tid + u * kThreads, row = e / (PS / 8), c0 = 8 * (e % (PS / 8));
            if (e >= YPIECES) continue;
            const float *cp = cy + row * LDY + c0;
            if constexpr (sizeof(T) == 2) {
                V8 w = __builtin_bit_cast(V8, yv[BI][u][0]);
#pragma unroll
                for (int k = 0; k < 8; ++k) w[k] = (T)((float)w[k] + cp[k]);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w), ry, (int)yoff(u), 0, 0);
            } else {
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    f32x4 v = __builtin_bit_cast(f32x4, yv[BI][u][w]);
#pragma unroll
                    for (int k = 0; k < 4; ++k) v[k] += cp[4 * w + k];
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ry, (int)yoff(u) + 16 * w, 0,
                                                           0);
                }
            }
        }
    };
    // Blocks in pairs; a pair's second block past the range runs with empty
    // descriptors (no loads, no stores), so that every path round the loop
    // is the same.
    for (int blk = blk0; blk < blk1; blk += 2) {
        block(std::integral_constant<int, 0>{}, blk);
        block(std::integral_constant<int, 1>{}, blk + 1);
    }
    __syncthreads();  // cs_at is written

    // ---- states of the slice's rows: final state (last range) and the state
    // after the accepted index (the range that holds it; index -1: the first).
    const bool last = blk1 == nblk;
    const bool has_j = p.state_out && ((j < 0 && r == 0) || (j >= 0 && j >= t0 && j < (int64_t)blk1 * kBlk));
    if (!last && !has_j) return;
    const float ef = last ? exp_neg(cs_at[1]) : 0.f;  // cs_at[1] = 0 when the shard is empty
    const float ej = j >= 0 ? exp_neg(cs_at[0]) : 1.f;
    const int64_t base = ((int64_t)bh * PF + (int64_t)s * PS) * N;
    // Eight 16-byte pieces per thread and step, all loaded before any store,
    // through descriptors over the slice (pieces past it read as zero and
    // are not stored; final_state may be shard_final itself: each piece is
    // read and written by the same thread only).
    const uint32_t sbytes = (uint32_t)(PS * N * 4);
    const bool do_fin = last && p.final_state;
    const float *hb = p.init_state + base;  // (the base of an empty descriptor, where a tensor is absent)
    const auto rh = buffer_rsrc(hb, sbytes);
    const auto rf = buffer_rsrc(do_fin ? p.shard_final + base : hb, do_fin ? sbytes : 0u);
    const auto rfo = buffer_rsrc(do_fin ? p.final_state + base : hb, do_fin ? sbytes : 0u);
    const auto ro = buffer_rsrc(has_j ? p.state_out + base : hb, has_j ? sbytes : 0u);
    constexpr int SU = 8;
    typedef unsigned u32x4s __attribute__((ext_vector_type(4)));
    for (uint32_t o0 = 16 * tid; o0 < sbytes; o0 += 16 * SU * kThreads) {
        f32x4 v[SU], f[SU], so[SU];
#pragma unroll
        for (int u = 0; u < SU; ++u) {
            const uint32_t o = o0 + 16 * u * kThreads;
            v[u] = __builtin_bit_cast(f32x4, ld16(rh, o));
            f[u] = __builtin_bit_cast(f32x4, ld16(rf, o));
            so[u] = __builtin_bit_cast(f32x4, ld16(ro, o));
        }
#pragma unroll
        for (int u = 0; u < SU; ++u) {
            const uint32_t o = o0 + 16 * u * kThreads;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4s, f[u] + ef * v[u]), rfo, (int)o, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4s, so[u] + ej * v[u]), ro, (int)o, 0, 0);
        }
    }
}

template <typename T, int KS>
hipError_t launch_ks(const Params &p, int ps, unsigned grid, int ranges, hipStream_t stream) {
    switch (ps) {
        case 16: hipLaunchKernelGGL((state_correction_kernel<T, KS, 1>), dim3(grid), dim3(kThreads), 0, stream, p, ranges); break;
        case 32: hipLaunchKernelGGL((state_correction_kernel<T, KS, 2>), dim3(grid), dim3(kThreads), 0, stream, p, ranges); break;
        case 64: hipLaunchKernelGGL((state_correction_kernel<T, KS, 4>), dim3(grid), dim3(kThreads), 0, stream, p, ranges); break;
        default: return hipErrorNotSupported;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const Params &p, int ps, unsigned grid, int ranges, hipStream_t stream) {
    switch ((p.dstate + 31) / 32) {
        case 1: return launch_ks<T, 1>(p, ps, grid, ranges, stream);
        case 2: return launch_ks<T, 2>(p, ps, grid, ranges, stream);
        case 4: return launch_ks<T, 4>(p, ps, grid, ranges, stream);
        case 8: return launch_ks<T, 8>(p, ps, grid, ranges, stream);
        default: return hipErrorNotSupported;
    }
}

}  // namespace

hipError_t launch_state_correction(const Params &p, Elem e, hipStream_t stream) {
    const int ps = p.headdim < kMaxSlice ? p.headdim : kMaxSlice;
    const int64_t items = p.batch * p.nheads * (p.headdim / ps);
    const int64_t nblk = (p.seqlen + kBlk - 1) / kBlk;
    // About 256 workgroups: ranges of blocks per item when items are few,
    // so that each workgroup reads its h_in slice and sums the dt before its
    // range once for several blocks (measured at the 2048-token dstate-256
    // shard: 256, 512, 1024 and 2048 workgroups take 28, 31, 36 and 55 us).
    int64_t ranges = (256 + items - 1) / items;
    ranges = std::max<int64_t>(1, std::min<int64_t>({ranges, nblk, 64}));
    const int64_t grid = items * ranges;
    if (items <= 0 || grid >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    return e == Elem::BF16 ? launch_t<bf16>(p, ps, (unsigned)grid, (int)ranges, stream)
                           : launch_t<float>(p, ps, (unsigned)grid, (int)ranges, stream);
}

}  // namespace ssd
