// Internal interface between the host orchestrator (ssd_api.hip) and the
// kernels.  Not installed; the public boundary is include/ssd.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

enum class Elem { F32, BF16 };

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
    void *states;             // workspace [b,nc,H,P,N] T_elem: chunk states S_c (from a zero start),
                              // rounded once to the input type
    void *prev;               // workspace [b,nc,H,P,N] T_elem: state entering each chunk (chunk 0 only with init_state)
    float *hj;                // workspace [b,H,P,N] fp32: state entering the chunk of state_out_idx[b]
    const float *shard_final; // [b,H,P,N] fp32: a shard's final state from a zero start (state correction only)
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
// final_state, state_out; the workspace is not used).  one_chunk_takes says
// whether it takes a call; launch_one_chunk returns hipErrorNotSupported for
// calls it does not take.
bool one_chunk_takes(const Params &p);
hipError_t launch_one_chunk(const Params &p, Elem e, hipStream_t stream);
hipError_t launch_empty_sequence(const Params &p, hipStream_t stream);
// Sequence-shard correction: y += exp(cs_t) C_t . init_state over the whole
// shard (cs from the shard's first token), final_state = shard_final +
// exp(cs_{T-1}) init_state, state_out += exp(cs_j) init_state.  Reads
// init_state (the state entering the shard), dt, A, C, shard_final and
// state_out_idx; updates y and state_out in place.
hipError_t launch_state_correction(const Params &p, Elem e, hipStream_t stream);

}  // namespace ssd
