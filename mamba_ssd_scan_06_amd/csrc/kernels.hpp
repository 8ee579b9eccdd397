// Internal interface between the host orchestrator (ssd_api.hip) and the
// kernels.  Not installed; the public boundary is include/ssd.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

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
    float *cs;                // workspace [b,H,nc,Q]
    float *states;            // workspace [b,nc,H,P,N]
    int64_t batch, seqlen;
    int nheads, headdim, dstate, ngroups, chunk, nchunks;
    int heads_per_group;
};

enum class Elem { F32, BF16 };

// Each launcher enqueues one kernel on `stream` and returns hipGetLastError().
hipError_t launch_chunk_cumsum(const Params &p, hipStream_t stream);
hipError_t launch_chunk_state(const Params &p, Elem e, hipStream_t stream);
hipError_t launch_state_pass(const Params &p, hipStream_t stream);
hipError_t launch_chunk_output(const Params &p, Elem e, hipStream_t stream);
hipError_t launch_state_at_index(const Params &p, Elem e, hipStream_t stream);
hipError_t launch_empty_sequence(const Params &p, hipStream_t stream);

}  // namespace ssd
