// Host side of libssd: argument checks, workspace layout and the launch
// sequence of the SSD chunked-scan forward.  The public contract is
// include/ssd.h.
//
// Launch sequence on the caller's stream (each step of the block
// decomposition in section "SSD算法" of the "Transformers are SSMs" article):
//   1. chunk_cumsum     dt, A            -> cs, ct, dte  (chunk-local log-decay tables)
//   2. chunk_state      x, B, dt, cs     -> states[c]    (green: S_c from a zero start)
//   3. state_pass       states, cs, h0   -> prev[c] = h_{c-1}, hj, final_state (yellow)
//   4. chunk_output     x, B, C, cs, dt tables, prev, D -> y  (orange + blue + D skip)
//   5. state_at_index   x, B, cs, dt, hj -> state_out  (only with state_out)
// A call whose tokens fit one chunk of at most 32 tokens (the multi-step
// verify) instead runs one fused kernel, one_chunk, which writes y,
// final_state and state_out directly and leaves the workspace untouched.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "ssd.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

ssd_status fail(ssd_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

constexpr size_t kAlign = 256;
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool is_pow2_in(int64_t v, int64_t lo, int64_t hi) {
    return v >= lo && v <= hi && (v & (v - 1)) == 0;
}

ssd_status check_shape(const ssd_shape *s, int chunk, ssd_dtype dtype) {
    if (!s) return fail(SSD_ERR_NULL, "shape is NULL");
    if (s->batch < 0 || s->seqlen < 0)
        return fail(SSD_ERR_SHAPE, "batch (%lld) and seqlen (%lld) must be >= 0", (long long)s->batch,
                    (long long)s->seqlen);
    if (s->nheads <= 0 || s->headdim <= 0 || s->dstate <= 0 || s->ngroups <= 0)
        return fail(SSD_ERR_SHAPE, "nheads, headdim, dstate and ngroups must be > 0");
    if (s->nheads % s->ngroups != 0)
        return fail(SSD_ERR_SHAPE, "ngroups (%lld) must divide nheads (%lld)", (long long)s->ngroups,
                    (long long)s->nheads);
    if (dtype != SSD_DTYPE_F32 && dtype != SSD_DTYPE_BF16) return fail(SSD_ERR_ARGS, "unknown dtype %d", (int)dtype);
    if (!is_pow2_in(chunk, 8, 256))
        return fail(SSD_ERR_CHUNK, "chunk_size %d not in {8, 16, 32, 64, 128, 256}", chunk);
    if (!is_pow2_in(s->headdim, 16, 128))
        return fail(SSD_ERR_UNSUPPORTED, "headdim %lld not in {16, 32, 64, 128}", (long long)s->headdim);
    if (!is_pow2_in(s->dstate, 16, 256))
        return fail(SSD_ERR_UNSUPPORTED, "dstate %lld not in {16, 32, 64, 128, 256}", (long long)s->dstate);
    if (dtype == SSD_DTYPE_F32 && s->headdim * s->dstate > 128 * 128)
        return fail(SSD_ERR_UNSUPPORTED, "fp32 inputs need headdim * dstate <= 16384 (LDS budget)");
    // Index arithmetic inside the kernels: grid dimensions and per-tensor sizes.
    const int64_t lim = (int64_t)1 << 40;
    if (s->batch > 65535 || s->nheads > 65535 || s->seqlen > lim / (s->nheads * s->headdim) ||
        s->batch > lim / ((s->seqlen + 1) * s->nheads * s->headdim))
        return fail(SSD_ERR_SHAPE, "problem too large");
    return SSD_OK;
}

struct Layout {
    size_t cs_off, ct_off, dte_off, blk_off, st_off, prev_off, hj_off, sync_off, total;
    int64_t nc;
};

Layout layout_of(const ssd_shape *s, int chunk, ssd_dtype dtype) {
    Layout L;
    L.nc = (s->seqlen + chunk - 1) / chunk;
    const size_t esz = dtype == SSD_DTYPE_BF16 ? 2 : 4;
    const size_t tab_bytes = round_up((size_t)s->batch * s->nheads * L.nc * chunk * sizeof(float));
    const size_t n_st = (size_t)s->batch * L.nc * s->nheads * s->headdim * s->dstate;
    const size_t n_hj = (size_t)s->batch * s->nheads * s->headdim * s->dstate;
    L.cs_off = 0;
    L.ct_off = tab_bytes;
    L.dte_off = 2 * tab_bytes;
    L.blk_off = 3 * tab_bytes;
    L.st_off = L.blk_off + round_up((size_t)s->batch * s->nheads * L.nc * ssd::kBlkStride * sizeof(float));
    L.prev_off = L.st_off + round_up(n_st * sizeof(float));
    L.hj_off = L.prev_off + round_up(n_st * esz);
    L.sync_off = L.hj_off + round_up(n_hj * sizeof(float));
    L.total = L.nc > 0 ? L.sync_off + round_up((size_t)ssd::sync_words(s->batch, s->nheads) * sizeof(int32_t)) : 0;
    return L;
}

struct Range {
    const char *name;
    uintptr_t lo, hi;  // [lo, hi)
};

Range range(const char *name, const void *p, size_t bytes) {
    uintptr_t lo = (uintptr_t)p;
    return Range{name, lo, p ? lo + bytes : lo};
}

bool overlaps(const Range &a, const Range &b) {
    return a.lo != a.hi && b.lo != b.hi && a.lo < b.hi && b.lo < a.hi;
}

// Runs the launch sequence, stops at the first failure and records the
// caller's timing marks after each kernel.
struct Launcher {
    hipStream_t stream;
    void *const *marks;
    int n_marks;
    const char **names;
    hipError_t err = hipSuccess;
    const char *failed_step = "";
    int count = 0;

    // Records the outcome of one launch and the caller's mark after it.
    void record(const char *name, hipError_t r) {
        err = r;
        if (err != hipSuccess) {
            failed_step = name;
            return;
        }
        ++count;
        if (count < n_marks) {
            err = hipEventRecord(static_cast<hipEvent_t>(marks[count]), stream);
            if (err != hipSuccess) failed_step = "event record";
            if (names) names[count - 1] = name;
        }
    }

    template <typename F>
    void step(const char *name, F &&launch) {
        if (err != hipSuccess) return;
        record(name, launch());
    }

    // Like step, but a launcher answering hipErrorNotSupported (a call or
    // shape it does not take, nothing enqueued) leaves no trace and makes
    // it return false.
    template <typename F>
    bool try_step(const char *name, F &&launch) {
        if (err != hipSuccess) return true;
        const hipError_t r = launch();
        if (r == hipErrorNotSupported) return false;
        record(name, r);
        return true;
    }
};

}  // namespace

extern "C" {

size_t ssd_workspace_bytes(const ssd_shape *shape, int chunk_size, ssd_dtype dtype) {
    if (check_shape(shape, chunk_size, dtype) != SSD_OK) return 0;
    return layout_of(shape, chunk_size, dtype).total;
}

ssd_status ssd_get_workspace_layout(const ssd_shape *shape, int chunk_size, ssd_dtype dtype,
                                    ssd_workspace_layout *out) {
    if (!out) return fail(SSD_ERR_NULL, "out is NULL");
    ssd_status st = check_shape(shape, chunk_size, dtype);
    if (st != SSD_OK) return st;
    const Layout L = layout_of(shape, chunk_size, dtype);
    out->cumsum_offset = L.cs_off;
    out->ct_offset = L.ct_off;
    out->dt_decay_offset = L.dte_off;
    out->block_decay_offset = L.blk_off;
    out->states_offset = L.st_off;
    out->prev_offset = L.prev_off;
    out->hj_offset = L.hj_off;
    out->sync_offset = L.sync_off;
    out->total_bytes = L.total;
    out->nchunks = L.nc;
    return SSD_OK;
}

ssd_status ssd_chunk_scan_fwd_marked(const void *x, const float *dt, const float *A, const void *B,
                                     const void *C, const float *D, const float *init_state, int chunk_size,
                                     void *y, float *final_state, const int32_t *state_out_idx,
                                     float *state_out, const ssd_shape *shape, ssd_dtype dtype, void *workspace,
                                     size_t workspace_bytes, void *hip_stream, void *const *marks, int n_marks,
                                     int *n_kernels, const char **kernel_names) {
    if (n_marks < 0 || (n_marks > 0 && !marks)) return fail(SSD_ERR_ARGS, "marks must hold n_marks events");
    ssd_status st = check_shape(shape, chunk_size, dtype);
    if (st != SSD_OK) return st;
    const int64_t b = shape->batch, T = shape->seqlen, H = shape->nheads, P = shape->headdim, N = shape->dstate,
                  G = shape->ngroups;
    if ((state_out == nullptr) != (state_out_idx == nullptr))
        return fail(SSD_ERR_ARGS, "state_out and state_out_idx must be given together");

    const size_t esz = dtype == SSD_DTYPE_BF16 ? 2 : 4;
    const size_t n_tok = (size_t)b * T;
    const size_t x_bytes = n_tok * H * P * esz, bc_bytes = n_tok * G * N * esz;
    const size_t dt_bytes = n_tok * H * sizeof(float), state_bytes = (size_t)b * H * P * N * sizeof(float);
    const Layout L = layout_of(shape, chunk_size, dtype);

    if (n_tok > 0) {
        if (!x || !dt || !A || !B || !C || !y) return fail(SSD_ERR_NULL, "x, dt, A, B, C and y are required");
        if (!workspace) return fail(SSD_ERR_WORKSPACE, "workspace is NULL");
        if (workspace_bytes < L.total)
            return fail(SSD_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);
    }
    if (b > 0 && state_out_idx == nullptr && state_out != nullptr) return fail(SSD_ERR_ARGS, "state_out_idx missing");

    const void *aligned16[] = {x, B, C, y, init_state, final_state, state_out, workspace};
    const char *names16[] = {"x", "B", "C", "y", "init_state", "final_state", "state_out", "workspace"};
    for (int k = 0; k < 8; ++k)
        if ((uintptr_t)aligned16[k] % 16 != 0) return fail(SSD_ERR_ALIGN, "%s is not 16-byte aligned", names16[k]);
    const void *aligned4[] = {dt, A, D, state_out_idx};
    const char *names4[] = {"dt", "A", "D", "state_out_idx"};
    for (int k = 0; k < 4; ++k)
        if ((uintptr_t)aligned4[k] % 4 != 0) return fail(SSD_ERR_ALIGN, "%s is not 4-byte aligned", names4[k]);

    const Range outs[] = {range("y", y, x_bytes), range("final_state", final_state, state_bytes),
                          range("state_out", state_out, state_bytes)};
    const Range others[] = {range("x", x, x_bytes), range("dt", dt, dt_bytes), range("A", A, H * sizeof(float)),
                            range("B", B, bc_bytes), range("C", C, bc_bytes), range("D", D, H * sizeof(float)),
                            range("init_state", init_state, state_bytes),
                            range("state_out_idx", state_out_idx, b * sizeof(int32_t)),
                            range("workspace", workspace, L.total)};
    // final_state may be init_state itself (an in-place update, e.g. decode):
    // every kernel reads each initial-state element before that element is
    // written, in the same thread, and reads it nowhere else.
    const bool in_place = final_state != nullptr && (const void *)final_state == (const void *)init_state;
    for (int i = 0; i < 3; ++i) {
        for (const Range &o : others) {
            if (in_place && i == 1 && o.lo == (uintptr_t)init_state) continue;
            if (overlaps(outs[i], o)) return fail(SSD_ERR_ALIAS, "%s overlaps %s", outs[i].name, o.name);
        }
        for (int k = i + 1; k < 3; ++k)
            if (overlaps(outs[i], outs[k])) return fail(SSD_ERR_ALIAS, "%s overlaps %s", outs[i].name, outs[k].name);
    }

    if (b == 0 || (T == 0 && !final_state && !state_out)) return SSD_OK;  // nothing to enqueue

    ssd::Params p;
    p.x = x;
    p.dt = dt;
    p.A = A;
    p.B = B;
    p.C = C;
    p.D = D;
    p.init_state = init_state;
    p.state_out_idx = state_out_idx;
    p.y = y;
    p.final_state = final_state;
    p.state_out = state_out;
    char *ws = static_cast<char *>(workspace);
    p.cs = ws ? reinterpret_cast<float *>(ws + L.cs_off) : nullptr;
    p.ct = ws ? reinterpret_cast<float *>(ws + L.ct_off) : nullptr;
    p.dte = ws ? reinterpret_cast<float *>(ws + L.dte_off) : nullptr;
    p.blk = ws ? reinterpret_cast<float *>(ws + L.blk_off) : nullptr;
    p.sync = ws ? reinterpret_cast<int *>(ws + L.sync_off) : nullptr;
    p.states = ws ? reinterpret_cast<float *>(ws + L.st_off) : nullptr;
    p.prev = ws ? static_cast<void *>(ws + L.prev_off) : nullptr;
    p.hj = ws && state_out ? reinterpret_cast<float *>(ws + L.hj_off) : nullptr;
    p.batch = b;
    p.seqlen = T;
    p.nheads = (int)H;
    p.headdim = (int)P;
    p.dstate = (int)N;
    p.ngroups = (int)G;
    p.chunk = chunk_size;
    p.nchunks = (int)L.nc;
    p.heads_per_group = (int)(H / G);
    const ssd::Elem e = dtype == SSD_DTYPE_BF16 ? ssd::Elem::BF16 : ssd::Elem::F32;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);

    (void)hipGetLastError();  // start from a clean error state
    Launcher run{stream, marks, n_marks, kernel_names};
    if (n_marks > 0) run.err = hipEventRecord(static_cast<hipEvent_t>(marks[0]), stream);
    if (T == 0) {
        run.step("empty_sequence", [&] { return ssd::launch_empty_sequence(p, stream); });
    } else if (run.try_step("one_chunk", [&] { return ssd::launch_one_chunk(p, e, stream); })) {
        // short call: the whole forward in one kernel
    } else {
        run.step("chunk_cumsum", [&] { return ssd::launch_chunk_cumsum(p, stream); });
        const bool fused = e == ssd::Elem::BF16 &&
                           run.try_step("chunk_scan_fused", [&] { return ssd::launch_chunk_scan_fused(p, stream); });
        if (!fused) {
        run.step("chunk_state", [&] {
            if (e == ssd::Elem::BF16) {
                const hipError_t r = ssd::launch_chunk_state_heads(p, stream);
                if (r != hipErrorNotSupported) return r;
            }
            return ssd::launch_chunk_state(p, e, stream);
        });
        run.step("state_pass", [&] { return ssd::launch_state_pass(p, e, stream); });
        run.step("chunk_output", [&] {
            if (e == ssd::Elem::BF16) {
                const hipError_t r = ssd::launch_chunk_output_heads(p, stream);
                if (r != hipErrorNotSupported) return r;
            }
            return ssd::launch_chunk_output(p, e, stream);
        });
        }
        if (state_out) run.step("state_at_index", [&] { return ssd::launch_state_at_index(p, e, stream); });
    }
    if (run.err != hipSuccess)
        return fail(SSD_ERR_HIP, "%s launch failed: %s", run.failed_step, hipGetErrorString(run.err));
    if (n_kernels) *n_kernels = run.count;
    return SSD_OK;
}

ssd_status ssd_chunk_scan_fwd(const void *x, const float *dt, const float *A, const void *B, const void *C,
                              const float *D, const float *init_state, int chunk_size, void *y,
                              float *final_state, const int32_t *state_out_idx, float *state_out,
                              const ssd_shape *shape, ssd_dtype dtype, void *workspace, size_t workspace_bytes,
                              void *hip_stream) {
    return ssd_chunk_scan_fwd_marked(x, dt, A, B, C, D, init_state, chunk_size, y, final_state, state_out_idx,
                                     state_out, shape, dtype, workspace, workspace_bytes, hip_stream, nullptr, 0,
                                     nullptr, nullptr);
}

const char *ssd_status_string(ssd_status s) {
    switch (s) {
        case SSD_OK: return "ok";
        case SSD_ERR_NULL: return "a required pointer is NULL";
        case SSD_ERR_SHAPE: return "invalid shape";
        case SSD_ERR_CHUNK: return "unsupported chunk_size";
        case SSD_ERR_ALIGN: return "misaligned pointer";
        case SSD_ERR_WORKSPACE: return "workspace missing or too small";
        case SSD_ERR_ALIAS: return "an output overlaps another buffer";
        case SSD_ERR_ARGS: return "inconsistent arguments";
        case SSD_ERR_HIP: return "HIP launch failure";
        case SSD_ERR_UNSUPPORTED: return "unsupported size";
    }
    return "unknown status";
}

const char *ssd_last_error(void) { return g_last_error.c_str(); }

int ssd_abi_version(void) { return SSD_ABI_VERSION; }

}  // extern "C"
