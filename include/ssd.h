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

#define SSD_ABI_VERSION 5

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
    SSD_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than ssd_workspace_bytes   */
    SSD_ERR_ALIAS = 6,       /* an output overlaps an input, another output or the workspace */
    SSD_ERR_ARGS = 7,        /* state_out given without state_out_idx or vice versa  */
    SSD_ERR_HIP = 8,         /* a kernel launch failed; outputs are unspecified      */
    SSD_ERR_UNSUPPORTED = 9  /* headdim not in {16,32,64,128} or dstate not in {16,32,64,128,256} */
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

/* Where the intermediates live inside the workspace after a call (byte
 * offsets from the workspace pointer).  Exposed so that the individual steps
 * can be checked.  A call whose tokens fit one chunk and number at most 32
 * is computed by one fused kernel and leaves the workspace untouched.  bf16
 * calls with dstate 64 or 128, headdim 32, 64 or 128, chunk_size 128 or 256
 * and at least 256 items (an item is a (b, h) pair, or a 64-channel half of
 * a head of headdim 128) run the single-pass kernel after the cumsum: it
 * fills cumsum, ct, dt_decay, block_decay, sync and (with state_out) hj,
 * uses only hand-off entries of states and leaves prev unwritten.  Every
 * other call runs the chunk-parallel kernels, which fill every region (sync
 * is only cleared).
 *   cumsum   fp32 [batch, nheads, nchunks, chunk_size]: the chunk-local
 *            cumulative log-decay A[h] * sum_{k<=i} dt[b, c*Q+k, h]; tokens
 *            past seqlen count as dt = 0.
 *   ct       fp32, same layout: cs * log2(e) - log2(dt) (+inf past seqlen),
 *            so that dt_j exp(cs_i - cs_j) = exp2(cs_i log2(e) - ct_j).
 *   dt_decay fp32, same layout: dt_i * exp(cs_e - cs_i), e = the last token
 *            (within seqlen) of the 32-token block holding i.
 *   block_decay fp32 [batch, nheads, nchunks, 16]: for the chunk's 32-token
 *            blocks m = 0..7, entry m is cs * log2(e) at the block's last
 *            token e(m) and entry 8+m is exp(cs_e(m) - cs_e(m-1))
 *            (exp(cs_e(0)) for m = 0); blocks past the chunk repeat its
 *            last token.
 *   states   fp32 [batch, nchunks, nheads, headdim, dstate]: entry c is the
 *            state chunk c reaches from a zero initial state.
 *   prev     dtype, same layout: entry c is the state entering chunk c,
 *            rounded to nearest even to dtype; entry 0 is written only when
 *            init_state is given (otherwise it is zero and left unwritten).
 *   hj       fp32 [batch, nheads, headdim, dstate]: the state entering the
 *            chunk that holds state_out_idx[b] (written only with state_out).
 *   sync     int32 [2 + 2*batch*nheads]: a time-out word (nonzero if a wait of
 *            the single-pass kernel for a state handed over by another
 *            workgroup gave up, which only a fault elsewhere can cause;
 *            outputs are then unspecified) and two hand-off flags per
 *            (b, h) (one per half of the channels when headdim 128 is
 *            split in two); cleared by the first kernel of each call.  The
 *            single-pass kernel hands a state over through the states region
 *            (entry [b, 0, h], the half's rows) when it splits a sequence's
 *            chunks between two workgroups. */
typedef struct {
    size_t cumsum_offset;
    size_t ct_offset;
    size_t dt_decay_offset;
    size_t block_decay_offset;
    size_t states_offset;
    size_t prev_offset;
    size_t hj_offset;
    size_t sync_offset;
    size_t total_bytes;
    int64_t nchunks;
} ssd_workspace_layout;

/* Bytes of device workspace ssd_chunk_scan_fwd needs for this problem
 * (0 when the arguments are invalid; ssd_last_error() says why). */
size_t ssd_workspace_bytes(const ssd_shape *shape, int chunk_size, ssd_dtype dtype);

/* Fills *out with the workspace layout for this problem. */
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
 *                 16-byte aligned; contents on entry are ignored
 *   hip_stream    hipStream_t as void*, NULL for the default stream
 *
 * Outputs must not overlap inputs, each other or the workspace, with one
 * exception: final_state may be init_state itself (same pointer), updating
 * the state in place (a decode step, a verifier keeping its cache).
 * Errors: see ssd_status; checks are host-side and happen before any launch. */
ssd_status ssd_chunk_scan_fwd(const void *x, const float *dt, const float *A,
                              const void *B, const void *C, const float *D,
                              const float *init_state, int chunk_size,
                              void *y, float *final_state,
                              const int32_t *state_out_idx, float *state_out,
                              const ssd_shape *shape, ssd_dtype dtype,
                              void *workspace, size_t workspace_bytes, void *hip_stream);

/* Same as ssd_chunk_scan_fwd, and additionally records caller-created HIP
 * events (hipEvent_t passed as void*) on hip_stream around the kernels, so
 * that a caller can time each kernel in place:
 *   marks[0]  before the first kernel,
 *   marks[k]  after the k-th kernel launched (k = 1 .. n_marks-1).
 * On SSD_OK, *n_kernels (if non-NULL) is the number of kernels launched and
 * kernel_names[k-1] (if kernel_names is non-NULL and k < n_marks) names the
 * kernel that marks[k] ends.  Marks beyond the kernels launched are not
 * recorded.  Used by the benchmark to measure per-kernel durations. */
ssd_status ssd_chunk_scan_fwd_marked(const void *x, const float *dt, const float *A,
                                     const void *B, const void *C, const float *D,
                                     const float *init_state, int chunk_size,
                                     void *y, float *final_state,
                                     const int32_t *state_out_idx, float *state_out,
                                     const ssd_shape *shape, ssd_dtype dtype,
                                     void *workspace, size_t workspace_bytes, void *hip_stream,
                                     void *const *marks, int n_marks, int *n_kernels,
                                     const char **kernel_names);

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
