// Internal interface between the host orchestrator (ssd_api.hip) and the
// kernels.  Not installed; the public boundary is include/ssd.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

enum class Elem { F32, BF16 };

constexpr int kBlkStride = 16;  // floats per (b, h, c) in the block-factor table
constexpr int kSyncHeader = 2;  // words before the hand-off flags in the sync region
// The single-pass kernel may split a head's channels p in two (headdim 128:
// two independent 64-channel halves), so each (b, h) has two flags.
constexpr int kFlagsPerHead = 2;
inline int64_t sync_words(int64_t batch, int64_t nheads) { return kSyncHeader + kFlagsPerHead * batch * nheads; }

// Everything a kernel needs, passed by value.  Pointers are device pointers
// with the layouts documented in include/ssd.h; `cs` and `states` point into
// the caller's workspace.
struct Params {
    const void *x;            // [b,T,H,P]  T_elem
    const float *dt;          // [b,T,H]
    const float *A;           // [H]
    const void *B;            // [b,T,G,N]  T_elem
    const void *C;            // [b,T,G,N]  T_elem
    const float *D;           // [H] or null
    const float *init_state;  // [b,H,P,N] or null
    const int32_t *state_out_idx;  // [b] or null
    void *y;                  // [b,T,H,P]  T_elem
    float *final_state;       // [b,H,P,N] or null
    float *state_out;         // [b,H,P,N] or null
    float *cs;                // workspace [b,H,nc,Q]: chunk-local cumulative log-decay
    float *ct;                // workspace [b,H,nc,Q]: cs * log2(e) - log2(dt) (+inf past the end)
    float *dte;               // workspace [b,H,nc,Q]: dt_i * exp(cs_e - cs_i), e = last token of i's 32-token block
    float *states;            // workspace [b,nc,H,P,N] fp32: chunk states S_c (from a zero start)
    void *prev;               // workspace [b,nc,H,P,N] T_elem: state entering each chunk (chunk 0 only with init_state)
    float *hj;                // workspace [b,H,P,N] fp32: state entering the chunk of state_out_idx[b]
    int *sync;                // workspace int32 [2 + b*H]: [0] unused, [1] wait time-out word, then one
                              // hand-off flag per (b, h) of the single-pass kernel
    float *blk;               // workspace [b,H,nc,kBlkStride] fp32: per 32-token block m of the chunk,
                              // [m] = cs*log2(e) at the block's last token, [8+m] = exp(cs_e(m) - cs_e(m-1))
                              // (exp(cs_e(0)) for m = 0)
    int64_t batch, seqlen;
    int nheads, headdim, dstate, ngroups, chunk, nchunks;
    int heads_per_group;
    int no_split;             // single pass: run every item whole on one workgroup (in-place calls)
};

// Each launcher enqueues one kernel on `stream` and returns hipGetLastError().
hipError_t launch_chunk_cumsum(const Params &p, hipStream_t stream);
hipError_t launch_chunk_state(const Params &p, Elem e, hipStream_t stream);
// Head-batched bf16 chunk states; returns hipErrorNotSupported when the shape
// does not fit its LDS budget or wave split (the caller then uses launch_chunk_state).
hipError_t launch_chunk_state_heads(const Params &p, hipStream_t stream);
hipError_t launch_state_pass(const Params &p, Elem e, hipStream_t stream);
hipError_t launch_chunk_output(const Params &p, Elem e, hipStream_t stream);
// Head-batched bf16 chunk outputs; returns hipErrorNotSupported when the
// shape does not fit its LDS budget (the caller then uses launch_chunk_output).
hipError_t launch_chunk_output_heads(const Params &p, hipStream_t stream);
hipError_t launch_state_at_index(const Params &p, Elem e, hipStream_t stream);
// Single-pass bf16 forward: one kernel for the whole call (its own
// chunk-local tables from dt and A; y, final_state and state_out written
// directly; the workspace is not used).  A grid of two workgroups per
// compute unit in which one workgroup at a time runs an item ((b, h), or a
// 64-channel half of a head of headdim 128), or a range of its blocks, in
// order with the state in registers.  chunk_scan_fused_takes says whether
// it takes a call; launch_chunk_scan_fused returns hipErrorNotSupported for
// calls it does not take.
constexpr int64_t kFusedMinItems = 64;
bool chunk_scan_fused_takes(const Params &p);
hipError_t launch_chunk_scan_fused(const Params &p, hipStream_t stream);
// Whole forward of a one-chunk call of at most 32 tokens in one kernel (y,
// final_state, state_out; the workspace is not used).  Returns
// hipErrorNotSupported for other calls and unsupported shapes.
hipError_t launch_one_chunk(const Params &p, Elem e, hipStream_t stream);
hipError_t launch_empty_sequence(const Params &p, hipStream_t stream);

}  // namespace ssd
