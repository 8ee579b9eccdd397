// Host side of libssd: argument checks, path choice, workspace layout and
// the launch sequence of the SSD chunked-scan forward.  The public contract
// is include/ssd.h.
//
// Paths (one is chosen per call from the shape, chunk size and dtype; see
// select_path):
//   one_chunk        a call of at most 32 tokens in one chunk (the multi-step
//                    verify): one kernel writes y, final_state and state_out.
//   single pass      bf16, dstate 64/128, headdim 32/64/128, at least 64
//                    items: chunk_scan_fused runs the whole forward with the
//                    state carried in registers (no workspace).
//   chunk parallel   everything else, each step of the block decomposition in
//                    section "SSD算法" of the "Transformers are SSMs" article:
//     1. chunk_cumsum     dt, A            -> cs, ct, dte  (chunk-local log-decay tables)
//     2. chunk_state      x, B, dt, cs     -> states[c]    (green: S_c from a zero start)
//     3. state_pass       states, cs, h0   -> prev[c] = h_{c-1}, hj, final_state (yellow)
//     4. chunk_output     x, B, C, cs, dt tables, prev, D -> y  (orange + blue + D skip)
//     5. state_at_index   x, B, cs, dt, hj -> state_out  (only with state_out)
// A call of zero tokens copies init_state (or zeros) to the requested states.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
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
    size_t cs_off, ct_off, dte_off, st_off, prev_off, hj_off, total;
    int64_t nc;
};

// Workspace of the chunk-parallel path.
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
    L.st_off = 3 * tab_bytes;
    L.prev_off = L.st_off + round_up(n_st * esz);
    L.hj_off = L.prev_off + round_up(n_st * esz);
    L.total = L.nc > 0 && s->batch > 0 ? L.hj_off + round_up(n_hj * sizeof(float)) : 0;
    return L;
}

// Size fields of the kernel parameters (no pointers).
ssd::Params shape_params(const ssd_shape *s, int chunk) {
    ssd::Params p = {};
    p.batch = s->batch;
    p.seqlen = s->seqlen;
    p.nheads = (int)s->nheads;
    p.headdim = (int)s->headdim;
    p.dstate = (int)s->dstate;
    p.ngroups = (int)s->ngroups;
    p.chunk = chunk;
    p.nchunks = (int)((s->seqlen + chunk - 1) / chunk);
    p.heads_per_group = (int)(s->nheads / s->ngroups);
    return p;
}

// The path a call takes when none is asked for.  Shape checks have passed.
ssd_path select_path(const ssd::Params &p, ssd_dtype dtype) {
    if (p.batch == 0 || p.seqlen == 0) return SSD_PATH_AUTO;  // nothing to compute but state copies
    if (ssd::one_chunk_takes(p)) return SSD_PATH_ONE_CHUNK;
    if (dtype == SSD_DTYPE_BF16 && ssd::chunk_scan_fused_takes(p)) return SSD_PATH_SINGLE_PASS;
    return SSD_PATH_CHUNK_PARALLEL;
}

bool path_takes(ssd_path path, const ssd::Params &p, ssd_dtype dtype) {
    switch (path) {
        case SSD_PATH_ONE_CHUNK: return ssd::one_chunk_takes(p);
        case SSD_PATH_SINGLE_PASS: return dtype == SSD_DTYPE_BF16 && ssd::chunk_scan_fused_takes(p);
        case SSD_PATH_CHUNK_PARALLEL: return true;
        default: return false;
    }
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
};

}  // namespace

// Workspace of ssd_chunk_scan_fwd_noalloc: every GPU the library runs on holds
// its own copy from the time the library's device code is loaded there until
// the process ends.  In host code `scratch` only names the variable; its
// device address on each GPU comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, looked up once

// The device address of `scratch` on the current device, looked up on the
// first call on that device (with it current).  `stream` must belong to it.
ssd_status scratch_ptr(hipStream_t stream, void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SSD_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(SSD_ERR_HIP, "device %d beyond the %d supported", dev, kMaxDevices);
    if (stream != nullptr) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess) return fail(SSD_ERR_HIP, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
        if (sdev != dev)
            return fail(SSD_ERR_ARGS, "hip_stream belongs to device %d, the current device is %d", (int)sdev, dev);
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr)
            return fail(SSD_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SSD_OK;
}

}  // namespace

extern "C" {

size_t ssd_workspace_bytes(const ssd_shape *shape, int chunk_size, ssd_dtype dtype) {
    if (check_shape(shape, chunk_size, dtype) != SSD_OK) return 0;
    if (select_path(shape_params(shape, chunk_size), dtype) != SSD_PATH_CHUNK_PARALLEL) return 0;
    return layout_of(shape, chunk_size, dtype).total;
}

int ssd_select_path(const ssd_shape *shape, int chunk_size, ssd_dtype dtype) {
    if (check_shape(shape, chunk_size, dtype) != SSD_OK) return -1;
    return (int)select_path(shape_params(shape, chunk_size), dtype);
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
    out->states_offset = L.st_off;
    out->prev_offset = L.prev_off;
    out->hj_offset = L.hj_off;
    out->total_bytes = L.total;
    out->nchunks = L.nc;
    return SSD_OK;
}

ssd_status ssd_chunk_scan_fwd_ex(const void *x, const float *dt, const float *A, const void *B, const void *C,
                                 const float *D, const float *init_state, int chunk_size, void *y,
                                 float *final_state, const int32_t *state_out_idx, float *state_out,
                                 const ssd_shape *shape, ssd_dtype dtype, void *workspace, size_t workspace_bytes,
                                 void *hip_stream, int path, void *const *marks, int n_marks, int *n_kernels,
                                 const char **kernel_names) {
    if (n_marks < 0 || (n_marks > 0 && !marks)) return fail(SSD_ERR_ARGS, "marks must hold n_marks events");
    ssd_status st = check_shape(shape, chunk_size, dtype);
    if (st != SSD_OK) return st;
    const int64_t b = shape->batch, T = shape->seqlen, H = shape->nheads, P = shape->headdim, N = shape->dstate,
                  G = shape->ngroups;
    if ((state_out == nullptr) != (state_out_idx == nullptr))
        return fail(SSD_ERR_ARGS, "state_out and state_out_idx must be given together");

    ssd::Params p = shape_params(shape, chunk_size);
    const ssd_path chosen = select_path(p, dtype);
    ssd_path run_path = chosen;
    if (path != SSD_PATH_AUTO) {
        if (path != SSD_PATH_ONE_CHUNK && path != SSD_PATH_SINGLE_PASS && path != SSD_PATH_CHUNK_PARALLEL)
            return fail(SSD_ERR_ARGS, "unknown path %d", path);
        // Zero-token and zero-batch calls only copy states, whatever the path.
        if (chosen != SSD_PATH_AUTO) {
            if (!path_takes((ssd_path)path, p, dtype))
                return fail(SSD_ERR_UNSUPPORTED, "path %d does not take this call", path);
            run_path = (ssd_path)path;
        }
    }

    const size_t esz = dtype == SSD_DTYPE_BF16 ? 2 : 4;
    const size_t n_tok = (size_t)b * T;
    const size_t x_bytes = n_tok * H * P * esz, bc_bytes = n_tok * G * N * esz;
    const size_t dt_bytes = n_tok * H * sizeof(float), state_bytes = (size_t)b * H * P * N * sizeof(float);
    const Layout L = layout_of(shape, chunk_size, dtype);
    const size_t ws_need = run_path == SSD_PATH_CHUNK_PARALLEL ? L.total : 0;

    if (n_tok > 0) {
        if (!x || !dt || !A || !B || !C || !y) return fail(SSD_ERR_NULL, "x, dt, A, B, C and y are required");
        if (ws_need > 0 && !workspace) return fail(SSD_ERR_WORKSPACE, "workspace is NULL");
        if (workspace_bytes < ws_need)
            return fail(SSD_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, ws_need);
    }

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
                            range("workspace", workspace, ws_need)};
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

    if (n_kernels) *n_kernels = 0;
    if (b == 0 || (T == 0 && !final_state && !state_out)) return SSD_OK;  // nothing to enqueue

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
    char *ws = run_path == SSD_PATH_CHUNK_PARALLEL ? static_cast<char *>(workspace) : nullptr;
    p.cs = ws ? reinterpret_cast<float *>(ws + L.cs_off) : nullptr;
    p.ct = ws ? reinterpret_cast<float *>(ws + L.ct_off) : nullptr;
    p.dte = ws ? reinterpret_cast<float *>(ws + L.dte_off) : nullptr;
    p.states = ws ? static_cast<void *>(ws + L.st_off) : nullptr;
    p.prev = ws ? static_cast<void *>(ws + L.prev_off) : nullptr;
    p.hj = ws && state_out ? reinterpret_cast<float *>(ws + L.hj_off) : nullptr;
    p.no_split = in_place ? 1 : 0;
    const ssd::Elem e = dtype == SSD_DTYPE_BF16 ? ssd::Elem::BF16 : ssd::Elem::F32;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);

    (void)hipGetLastError();  // start from a clean error state
    Launcher run{stream, marks, n_marks, kernel_names};
    if (n_marks > 0) run.err = hipEventRecord(static_cast<hipEvent_t>(marks[0]), stream);
    if (T == 0) {
        run.step("empty_sequence", [&] { return ssd::launch_empty_sequence(p, stream); });
    } else if (run_path == SSD_PATH_ONE_CHUNK) {
        run.step("one_chunk", [&] { return ssd::launch_one_chunk(p, e, stream); });
    } else if (run_path == SSD_PATH_SINGLE_PASS) {
        run.step("chunk_scan_fused", [&] { return ssd::launch_chunk_scan_fused(p, stream); });
    } else {
        run.step("chunk_cumsum", [&] { return ssd::launch_chunk_cumsum(p, stream); });
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
    return ssd_chunk_scan_fwd_ex(x, dt, A, B, C, D, init_state, chunk_size, y, final_state, state_out_idx,
                                 state_out, shape, dtype, workspace, workspace_bytes, hip_stream, SSD_PATH_AUTO,
                                 nullptr, 0, nullptr, nullptr);
}

ssd_status ssd_chunk_scan_fwd_noalloc(const void *x, const float *dt, const float *A, const void *B, const void *C,
                                      const float *D, const float *init_state, int chunk_size, void *y,
                                      float *final_state, const int32_t *state_out_idx, float *state_out,
                                      const ssd_shape *shape, ssd_dtype dtype, void *hip_stream) {
    ssd_status st = check_shape(shape, chunk_size, dtype);
    if (st != SSD_OK) return st;
    const size_t need = ssd_workspace_bytes(shape, chunk_size, dtype);
    if (need > (size_t)SSD_NOALLOC_SCRATCH_BYTES)
        return fail(SSD_ERR_WORKSPACE, "the call needs %zu bytes of workspace, the static scratch holds %zu", need,
                    (size_t)SSD_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    if (need > 0) {
        st = scratch_ptr(static_cast<hipStream_t>(hip_stream), &ws);
        if (st != SSD_OK) return st;
    }
    return ssd_chunk_scan_fwd(x, dt, A, B, C, D, init_state, chunk_size, y, final_state, state_out_idx, state_out,
                              shape, dtype, ws, need > 0 ? (size_t)SSD_NOALLOC_SCRATCH_BYTES : 0, hip_stream);
}

ssd_status ssd_state_correction(void *y, const float *dt, const float *A, const void *C, const float *h_in,
                                const float *shard_final, float *final_state, const int32_t *state_out_idx,
                                float *state_out, const ssd_shape *shape, ssd_dtype dtype, void *hip_stream) {
    ssd_status st = check_shape(shape, 256, dtype);
    if (st != SSD_OK) return st;
    const int64_t b = shape->batch, T = shape->seqlen, H = shape->nheads, P = shape->headdim, N = shape->dstate,
                  G = shape->ngroups;
    if ((state_out == nullptr) != (state_out_idx == nullptr))
        return fail(SSD_ERR_ARGS, "state_out and state_out_idx must be given together");
    if (final_state && !shard_final) return fail(SSD_ERR_NULL, "final_state needs shard_final");
    if (b > 0 && !h_in) return fail(SSD_ERR_NULL, "h_in is required");
    if (b > 0 && T > 0 && (!y || !dt || !A || !C)) return fail(SSD_ERR_NULL, "y, dt, A and C are required");
    // The kernel addresses a 64-token block's rows of y and C, and a
    // sequence's dt, with 32-bit byte offsets.
    const int64_t esz_i = dtype == SSD_DTYPE_BF16 ? 2 : 4, lim31 = (int64_t)1 << 31;
    if (64 * H * P * esz_i >= lim31 || 64 * G * N * esz_i >= lim31 || T * H * 4 >= lim31)
        return fail(SSD_ERR_UNSUPPORTED, "state correction needs 64*nheads*headdim, 64*ngroups*dstate "
                                         "(in elements of dtype) and seqlen*nheads*4 below 2^31 bytes");

    const size_t esz = dtype == SSD_DTYPE_BF16 ? 2 : 4;
    const size_t n_tok = (size_t)b * T;
    const size_t y_bytes = n_tok * H * P * esz, c_bytes = n_tok * G * N * esz;
    const size_t dt_bytes = n_tok * H * sizeof(float), state_bytes = (size_t)b * H * P * N * sizeof(float);
    const void *aligned16[] = {y, C, h_in, shard_final, final_state, state_out};
    const char *names16[] = {"y", "C", "h_in", "shard_final", "final_state", "state_out"};
    for (int k = 0; k < 6; ++k)
        if ((uintptr_t)aligned16[k] % 16 != 0) return fail(SSD_ERR_ALIGN, "%s is not 16-byte aligned", names16[k]);
    const void *aligned4[] = {dt, A, state_out_idx};
    const char *names4[] = {"dt", "A", "state_out_idx"};
    for (int k = 0; k < 3; ++k)
        if ((uintptr_t)aligned4[k] % 4 != 0) return fail(SSD_ERR_ALIGN, "%s is not 4-byte aligned", names4[k]);

    const Range outs[] = {range("y", y, y_bytes), range("final_state", final_state, state_bytes),
                          range("state_out", state_out, state_bytes)};
    const Range others[] = {range("dt", dt, dt_bytes), range("A", A, H * sizeof(float)), range("C", C, c_bytes),
                            range("h_in", h_in, state_bytes), range("shard_final", shard_final, state_bytes),
                            range("state_out_idx", state_out_idx, b * sizeof(int32_t))};
    // final_state may be shard_final itself: each element is read before it
    // is written, by the same thread, and read nowhere else.
    const bool in_place = final_state != nullptr && (const void *)final_state == (const void *)shard_final;
    for (int i = 0; i < 3; ++i) {
        for (const Range &o : others) {
            if (in_place && i == 1 && o.lo == (uintptr_t)shard_final) continue;
            if (overlaps(outs[i], o)) return fail(SSD_ERR_ALIAS, "%s overlaps %s", outs[i].name, o.name);
        }
        for (int k = i + 1; k < 3; ++k)
            if (overlaps(outs[i], outs[k])) return fail(SSD_ERR_ALIAS, "%s overlaps %s", outs[i].name, outs[k].name);
    }
    if (b == 0 || (T == 0 && !final_state && !state_out)) return SSD_OK;  // nothing to enqueue

    ssd::Params p = shape_params(shape, 256);
    p.dt = dt;
    p.A = A;
    p.C = C;
    p.init_state = h_in;
    p.shard_final = shard_final;
    p.state_out_idx = state_out_idx;
    p.y = y;
    p.final_state = final_state;
    p.state_out = state_out;
    (void)hipGetLastError();  // start from a clean error state
    const hipError_t r = ssd::launch_state_correction(
        p, dtype == SSD_DTYPE_BF16 ? ssd::Elem::BF16 : ssd::Elem::F32, static_cast<hipStream_t>(hip_stream));
    if (r != hipSuccess) return fail(SSD_ERR_HIP, "state_correction launch failed: %s", hipGetErrorString(r));
    return SSD_OK;
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
