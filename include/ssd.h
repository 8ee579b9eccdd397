/*
 * libssd -- Mamba-2 SSD (state space duality) chunked selective-scan forward
 * for AMD MI355X (gfx950).  C ABI; no HIP or torch types appear here.
 *
 * The operation
 * -------------
 * For every sequence b, head h (B/C group g = floor(h*G/H)) and token t:
 *
 *     h_t[p][n] = exp(dt[b,t,h] * A[h]) * h_{t-1}[p][n] + dt[b,t,h] * x[b,t,h,p] * B[b,t,g,n]
 *     y[b,t,h,p] = sum_n C[b,t,g,n] * h_t[p][n] + D[h] * x[b,t,h,p]
 *
 * with h_{-1} = init_state[b,h] (zero when absent).  This is the selective
 * SSM with one scalar decay per head that the Mamba-2 SSD layer evaluates
 * ("Transformers are SSMs" article, cloud.tencent.com.cn, section
 * "核心创新——SSD"; the page's formula image is lost and the recurrence above
 * is the reading used, with y read after the state update).
 *
 * It is evaluated by the block decomposition of section "SSD算法" of that
 * article: the sequence is cut into chunks of `chunk_size` tokens; inside a
 * chunk the output is computed in the attention-like quadratic form from a
 * zero state (orange part), each chunk's final state from a zero start is a
 * batched matrix product (green), a short scan over chunks turns those into
 * every chunk's true initial state (yellow), and each chunk's output gains
 * the contribution of that initial state (blue).  Section
 * "深入解析分块与状态传递机制" describes the same four steps.  The result equals
 * the recurrence up to floating-point rounding for every chunk size.
 *
 * Multi-step verify ("3天把Llama训成Mamba" article, blog.csdn.net, section
 * "推测解码"): started from a cached state, one call returns every output,
 * the state after the last token (final_state) and the state after a
 * per-sequence accepted index (state_out), the only extra state the
 * speculative-decoding verifier keeps.
 *
 * Conventions common to every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers, owned by the caller, dense and
 *   row-major in the shapes given below (last dimension fastest).  The
 *   library never allocates, frees or synchronises device memory.
 * - Work is enqueued asynchronously on `hip_stream` (a hipStream_t passed as
 *   void*; NULL = the default stream) in stream order.
 * - Every argument check runs on the host before the first launch: a return
 *   other than SSD_OK means nothing was enqueued and no output was touched.
 * - Device-side values are preconditions, not checked (checking would need
 *   a synchronisation): dt finite and >= 0, A finite and <= 0, state_out_idx
 *   in [-1, seqlen-1].  Violations give unspecified values but never an
 *   out-of-bounds access (indices are clamped).
 * - ssd_last_error() holds a description of the last non-OK return on the
 *   calling thread.
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 8

/* Element type of x, B, C and y.  dt, A, D and every state are always fp32. */
typedef enum {
    SSD_DTYPE_F32 = 0,
    SSD_DTYPE_BF16 = 1
} ssd_dtype;

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL = 1,        /* a required pointer is NULL                          */
    SSD_ERR_SHAPE = 2,       /* a size is negative, or ngroups does not divide nheads */
    SSD_ERR_CHUNK = 3,       /* chunk_size not in {8, 16, 32, 64, 128, 256}          */
    SSD_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned              */
    SSD_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than the call's path needs */
    SSD_ERR_ALIAS = 6,       /* an output overlaps an input, another output or the workspace */
    SSD_ERR_ARGS = 7,        /* state_out without state_out_idx or vice versa, an unknown
                                dtype or path, or marks missing for n_marks > 0      */
    SSD_ERR_HIP = 8,         /* a kernel launch failed; outputs are unspecified      */
    SSD_ERR_UNSUPPORTED = 9  /* headdim not in {16,32,64,128}, dstate not in {16,32,64,128,256},
                                fp32 with headdim*dstate > 16384, or a requested path
                                that does not take the call                          */
} ssd_status;

/* Problem sizes.  batch and seqlen may be 0. */
typedef struct {
    int64_t batch;    /* b: independent sequences                     */
    int64_t seqlen;   /* T: tokens per sequence                       */
    int64_t nheads;   /* H: heads (one scalar decay A[h] each)         */
    int64_t headdim;  /* P: channels per head                         */
    int64_t dstate;   /* N: state size per channel                    */
    int64_t ngroups;  /* G: B/C groups; head h reads group h*G/H      */
} ssd_shape;

/* How a call is computed.  Every path gives the same results up to
 * floating-point rounding; the automatic choice depends only on the shape,
 * chunk_size and dtype (ssd_select_path).
 *   SSD_PATH_ONE_CHUNK       at most 32 tokens in one chunk (the multi-step
 *                            verify, a decode step): one kernel reads the
 *                            initial state once and writes y, final_state
 *                            and state_out.  Needs headdim a multiple of
 *                            1024 / dstate.
 *   SSD_PATH_SINGLE_PASS     bf16, dstate 64 or 128, headdim 32, 64 or 128,
 *                            at least 64 items (an item is a (b, h) pair, or
 *                            a 64-channel half of a head of headdim 128):
 *                            one kernel walks each item's sequence in
 *                            128-token blocks with the state in registers
 *                            (the state passing of section
 *                            "深入解析分块与状态传递机制" of the "Transformers
 *                            are SSMs" article, carried inside the kernel).
 *                            When there are fewer items than workgroups, an
 *                            item's blocks are split into ranges; a range
 *                            not starting at token 0 first recomputes the
 *                            state it starts from, so no workgroup ever
 *                            waits for another.  Its internal block length
 *                            does not depend on chunk_size.
 *   SSD_PATH_CHUNK_PARALLEL  any call: the four steps of the block
 *                            decomposition as separate kernels, with the
 *                            intermediates in the workspace.
 * No path uses the workspace except SSD_PATH_CHUNK_PARALLEL. */
typedef enum {
    SSD_PATH_AUTO = 0,
    SSD_PATH_ONE_CHUNK = 1,
    SSD_PATH_SINGLE_PASS = 2,
    SSD_PATH_CHUNK_PARALLEL = 3
} ssd_path;

/* The path ssd_chunk_scan_fwd takes for this problem; SSD_PATH_AUTO (0) when
 * batch or seqlen is 0 (no kernel but a state copy runs), -1 when the
 * arguments are invalid (ssd_last_error() says why). */
int ssd_select_path(const ssd_shape *shape, int chunk_size, ssd_dtype dtype);

/* The workspace of SSD_PATH_CHUNK_PARALLEL: byte offsets from the workspace
 * pointer of the intermediates that path leaves there, exposed so that the
 * individual steps can be checked.
 *   cumsum   fp32 [batch, nheads, nchunks, chunk_size]: the chunk-local
 *            cumulative log-decay A[h] * sum_{k<=i} dt[b, c*Q+k, h]; tokens
 *            past seqlen count as dt = 0.
 *   ct       fp32, same layout: cs * log2(e) - log2(dt) (+inf past seqlen),
 *            so that dt_j exp(cs_i - cs_j) = exp2(cs_i log2(e) - ct_j).
 *   dt_decay fp32, same layout: dt_i * exp(cs_e - cs_i), e = the last token
 *            (within seqlen) of the 32-token block holding i.
 *   states   dtype [batch, nchunks, nheads, headdim, dstate]: entry c is the
 *            state chunk c reaches from a zero initial state (accumulated in
 *            fp32, rounded to nearest even to dtype once).
 *   prev     dtype, same layout: entry c is the state entering chunk c,
 *            rounded to nearest even to dtype; entry 0 is written only when
 *            init_state is given (otherwise it is never read).
 *   hj       fp32 [batch, nheads, headdim, dstate]: the state entering the
 *            chunk that holds state_out_idx[b] (written only with state_out).
 * Every region a kernel reads was written earlier in the same call: the
 * contents on entry never matter. */
typedef struct {
    size_t cumsum_offset;
    size_t ct_offset;
    size_t dt_decay_offset;
    size_t states_offset;
    size_t prev_offset;
    size_t hj_offset;
    size_t total_bytes;   /* bytes SSD_PATH_CHUNK_PARALLEL needs (0 when batch or seqlen is 0) */
    int64_t nchunks;
} ssd_workspace_layout;

/* Bytes of device workspace ssd_chunk_scan_fwd needs for this problem: the
 * layout's total_bytes when the call takes SSD_PATH_CHUNK_PARALLEL, else 0
 * (then workspace may be NULL).  0 also when the arguments are invalid
 * (ssd_last_error() says why). */
size_t ssd_workspace_bytes(const ssd_shape *shape, int chunk_size, ssd_dtype dtype);

/* Fills *out with the workspace layout of SSD_PATH_CHUNK_PARALLEL for this
 * problem (also for problems that take another path automatically). */
ssd_status ssd_get_workspace_layout(const ssd_shape *shape, int chunk_size, ssd_dtype dtype,
                                    ssd_workspace_layout *out);

/* The SSD chunked-scan forward.
 *
 *   x             [b,T,H,P]  dtype      input channels
 *   dt            [b,T,H]    fp32       step sizes, already positive (no
 *                                       softplus, bias or clamp is applied)
 *   A             [H]        fp32       per-head decay rate (<= 0)
 *   B, C          [b,T,G,N]  dtype      input / output projections of the state
 *   D             [H]        fp32       skip weight; NULL = no skip term
 *   init_state    [b,H,P,N]  fp32       state before token 0; NULL = zeros
 *   chunk_size    Q in {8,16,32,64,128,256}; any T >= 0 (the last chunk may
 *                 be partial).  Results do not depend on Q beyond rounding.
 *   y             [b,T,H,P]  dtype      outputs, fully overwritten (rounded
 *                                       to nearest even from fp32 for bf16)
 *   final_state   [b,H,P,N]  fp32       state after token T-1; NULL = not returned
 *   state_out_idx [b]        int32      accepted index j_b per sequence; NULL = none
 *   state_out     [b,H,P,N]  fp32       state after token j_b (0-based,
 *                                       inclusive; j_b = -1 gives init_state);
 *                                       non-NULL exactly when state_out_idx is
 *   shape, dtype             sizes and element type as above
 *   workspace     device scratch of at least ssd_workspace_bytes(...) bytes,
 *                 16-byte aligned; contents on entry are ignored; may be
 *                 NULL when ssd_workspace_bytes(...) is 0
 *   hip_stream    hipStream_t as void*, NULL for the default stream
 *
 * Outputs must not overlap inputs, each other or the workspace, with one
 * exception: final_state may be init_state itself (same pointer), updating
 * the state in place (a decode step, a verifier keeping its cache).  An
 * in-place call on SSD_PATH_SINGLE_PASS runs every item whole on one
 * workgroup (no ranges), since a range's recomputation reads init_state.
 * Errors: see ssd_status; checks are host-side and happen before any launch. */
ssd_status ssd_chunk_scan_fwd(const void *x, const float *dt, const float *A,
                              const void *B, const void *C, const float *D,
                              const float *init_state, int chunk_size,
                              void *y, float *final_state,
                              const int32_t *state_out_idx, float *state_out,
                              const ssd_shape *shape, ssd_dtype dtype,
                              void *workspace, size_t workspace_bytes, void *hip_stream);

/* Same as ssd_chunk_scan_fwd with two additions.
 *   path    SSD_PATH_AUTO, or the path to take (SSD_ERR_UNSUPPORTED when it
 *           does not take the call; calls of zero tokens or sequences only
 *           copy states whatever the path).  The workspace must then hold the
 *           bytes that path needs: the layout's total_bytes for
 *           SSD_PATH_CHUNK_PARALLEL, none for the others.
 *   marks   caller-created HIP events (hipEvent_t as void*) recorded on
 *           hip_stream around the kernels, so that a caller can time each
 *           kernel in place: marks[0] before the first kernel, marks[k]
 *           after the k-th kernel launched (k = 1 .. n_marks-1).  Marks
 *           beyond the kernels launched are not recorded.  n_marks may be 0
 *           (marks NULL).
 * On SSD_OK, *n_kernels (if non-NULL) is the number of kernels launched and
 * kernel_names[k-1] (if kernel_names is non-NULL and k < n_marks) names the
 * kernel that marks[k] ends. */
ssd_status ssd_chunk_scan_fwd_ex(const void *x, const float *dt, const float *A,
                                 const void *B, const void *C, const float *D,
                                 const float *init_state, int chunk_size,
                                 void *y, float *final_state,
                                 const int32_t *state_out_idx, float *state_out,
                                 const ssd_shape *shape, ssd_dtype dtype,
                                 void *workspace, size_t workspace_bytes, void *hip_stream,
                                 int path, void *const *marks, int n_marks, int *n_kernels,
                                 const char **kernel_names);

/* Bytes of the library's static device scratch (64 MiB), the workspace of
 * ssd_chunk_scan_fwd_noalloc. */
#define SSD_NOALLOC_SCRATCH_BYTES (64u << 20)

/* ssd_chunk_scan_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  A call that needs a workspace (the
 * chunk-parallel path, ssd_workspace_bytes(...) > 0) uses a static array of
 * SSD_NOALLOC_SCRATCH_BYTES in the library's device code instead; every GPU
 * holds its own copy until the process ends, and its device address is
 * looked up once per GPU on the first such call there.  Neither this entry
 * point nor anything it calls allocates or frees memory.
 *   - Calls needing more than SSD_NOALLOC_SCRATCH_BYTES return
 *     SSD_ERR_WORKSPACE before anything is enqueued.
 *   - hip_stream must belong to the current device (else SSD_ERR_ARGS).
 *   - All calls on one GPU share its scratch: calls that may overlap in time
 *     on one GPU (on different streams, or from several threads without
 *     ordering) race and give unspecified results.  Calls in one stream's
 *     order are safe.  The scratch keeps the last call's intermediates;
 *     nothing in a call depends on what it held before.
 * Arguments, results and every other error are as for ssd_chunk_scan_fwd. */
ssd_status ssd_chunk_scan_fwd_noalloc(const void *x, const float *dt, const float *A,
                                      const void *B, const void *C, const float *D,
                                      const float *init_state, int chunk_size,
                                      void *y, float *final_state,
                                      const int32_t *state_out_idx, float *state_out,
                                      const ssd_shape *shape, ssd_dtype dtype, void *hip_stream);

/* Sequence sharding (context parallelism): the step a GPU runs on its shard
 * once it knows the state entering the shard.
 *
 * "Transformers are SSMs" article (cloud.tencent.com.cn), section
 * "序列并行的两种形式": with the sequence split over GPUs, each GPU computes
 * its shard's outputs and final state on its own and only states pass between
 * GPUs.  A shard run with ssd_chunk_scan_fwd from a zero initial state gives
 * y0, F (its final_state) and, with an accepted index, h0_j (its state_out).
 * The recurrence is linear in its initial state, so from the true entering
 * state h_in the shard's results are
 *     y_t   = y0_t + exp(cs_t) * sum_n C[b,t,g,n] * h_in[b,h,p,n]
 *     final = F + exp(cs_{T-1}) * h_in
 *     h_j   = h0_j + exp(cs_j) * h_in          (j = -1: h0_j + h_in)
 * with cs_t = A[h] * sum_{k<=t} dt[b,k,h] over the shard's own tokens.  This
 * call applies them in place; the exchange of states between GPUs is the
 * caller's.
 *
 *   y             [b,T,H,P]  dtype  in/out: y0 on entry, y on return (rounded
 *                                   to nearest even from fp32 for bf16)
 *   dt, A, C      as passed to ssd_chunk_scan_fwd for the shard
 *   h_in          [b,H,P,N]  fp32   state entering the shard (required)
 *   shard_final   [b,H,P,N]  fp32   F; required when final_state is given
 *   final_state   [b,H,P,N]  fp32   out: F + exp(cs_{T-1}) h_in; NULL = not
 *                                   returned; may be shard_final itself
 *   state_out_idx [b]        int32  the accepted index j_b within the shard
 *                                   (as given to the shard's forward); NULL = none
 *   state_out     [b,H,P,N]  fp32   in/out: h0_j on entry, h_j on return;
 *                                   non-NULL exactly when state_out_idx is
 * h_in rounds once to dtype before its product with C (fp32 accumulation).
 * Outputs must not overlap the inputs or each other (final_state ==
 * shard_final excepted).  Same shape limits, alignment rules and errors as
 * ssd_chunk_scan_fwd, and SSD_ERR_UNSUPPORTED unless 64*nheads*headdim and
 * 64*ngroups*dstate elements of dtype, and seqlen*nheads*4 bytes, stay below
 * 2^31 bytes (32-bit offsets within a 64-token block and within dt); no
 * workspace; T = 0 gives final = F + h_in. */
ssd_status ssd_state_correction(void *y, const float *dt, const float *A, const void *C,
                                const float *h_in, const float *shard_final, float *final_state,
                                const int32_t *state_out_idx, float *state_out,
                                const ssd_shape *shape, ssd_dtype dtype, void *hip_stream);

/* Static description of a status code. */
const char *ssd_status_string(ssd_status status);

/* Detail for the last non-OK return on the calling thread ("" if none). */
const char *ssd_last_error(void);

/* SSD_ABI_VERSION of the built library. */
int ssd_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */
