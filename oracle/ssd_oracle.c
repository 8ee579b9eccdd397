/*
 * TEST INFRASTRUCTURE -- the fp64 CPU oracle for the SSD forward.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  It shares no code, header, table or helper with
 * the HIP path and is never called by it.
 *
 * What it computes: the selective state-space recurrence that the Mamba-2
 * SSD layer evaluates, token by token, in fp64 ("Transformers are SSMs"
 * article on cloud.tencent.com.cn, section "核心创新——SSD": the SSD layer is
 * a selective SSM with one scalar decay per head, whose linear-time form is
 * this recurrence).  The printed formula is missing from the page; the
 * reading used is
 *
 *     h_t[p][n] = exp(dt_t * A_h) * h_{t-1}[p][n] + dt_t * x_t[p] * B_t[n]
 *     y_t[p]    = sum_n C_t[n] * h_t[p][n] + D_h * x_t[p]
 *
 * with y read from the state after the update, B and C taken from group
 * g = floor(h * G / H), and h_{-1} the initial state (zero when absent).
 *
 * Multi-step verify ("3天把Llama训成Mamba" article on blog.csdn.net, section
 * "推测解码": the verifier returns the K outputs, the state at the last
 * accepted position and the state after the last position): state_out[b]
 * is the state after consuming token j = state_out_idx[b] (0-based,
 * inclusive); j = -1 returns the initial state.
 *
 * Optionally the state entering every chunk of `chunk` tokens is recorded
 * (the "true initial state" of each chunk in section
 * "深入解析分块与状态传递机制" of the Mamba-2 article): entry c is h_{cQ-1}.
 *
 * Rows (b, h, p) are independent and are spread over OpenMP threads; within
 * a row the loop runs over t in order, so the result does not depend on the
 * thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_abi_version(void) { return 1; }

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Returns 0 on success, a negative number on a bad argument. */
int oracle_ssd_forward(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                       int64_t dstate, int64_t ngroups,
                       const double *x,          /* [batch, seqlen, nheads, headdim] */
                       const double *dt,         /* [batch, seqlen, nheads]          */
                       const double *A,          /* [nheads]                         */
                       const double *B,          /* [batch, seqlen, ngroups, dstate] */
                       const double *C,          /* [batch, seqlen, ngroups, dstate] */
                       const double *D,          /* [nheads] or NULL                 */
                       const double *init_state, /* [batch, nheads, headdim, dstate] or NULL */
                       const int32_t *state_out_idx, /* [batch] or NULL              */
                       double *y,                /* [batch, seqlen, nheads, headdim] */
                       double *final_state,      /* [batch, nheads, headdim, dstate] or NULL */
                       double *state_out,        /* [batch, nheads, headdim, dstate] or NULL */
                       int64_t chunk,            /* > 0 to record chunk-start states */
                       double *chunk_states,     /* [batch, nchunks, nheads, headdim, dstate] or NULL */
                       int nthreads)
{
    if (batch < 0 || seqlen < 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0)
        return -1;
    if (nheads % ngroups != 0) return -2;
    if (!x || !dt || !A || !B || !C || !y) return -3;
    if ((state_out_idx == NULL) != (state_out == NULL)) return -4;
    if (chunk_states && chunk <= 0) return -5;

    const int64_t T = seqlen, H = nheads, P = headdim, N = dstate, G = ngroups;
    const int64_t heads_per_group = H / G;
    const int64_t nchunks = chunk > 0 ? (T + chunk - 1) / chunk : 0;
    const int64_t rows = batch * H * P;
    if (nthreads <= 0) nthreads = oracle_max_threads();
    int failed = 0;

#pragma omp parallel num_threads(nthreads)
    {
        double *hs = (double *)malloc(sizeof(double) * (size_t)N);
        if (!hs) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t row = 0; row < rows; ++row) {
            if (!hs) continue;
            const int64_t b = row / (H * P);
            const int64_t h = (row / P) % H;
            const int64_t p = row % P;
            const int64_t g = h / heads_per_group;
            const int64_t state_off = ((b * H + h) * P + p) * N;

            for (int64_t n = 0; n < N; ++n)
                hs[n] = init_state ? init_state[state_off + n] : 0.0;

            const int64_t j = state_out_idx ? (int64_t)state_out_idx[b] : -2;
            if (state_out && j == -1)
                memcpy(state_out + state_off, hs, sizeof(double) * (size_t)N);

            for (int64_t t = 0; t < T; ++t) {
                if (chunk_states && t % chunk == 0) {
                    const int64_t c = t / chunk;
                    double *dst = chunk_states + (((b * nchunks + c) * H + h) * P + p) * N;
                    memcpy(dst, hs, sizeof(double) * (size_t)N);
                }
                const double d = dt[(b * T + t) * H + h];
                const double decay = exp(d * A[h]);
                const double xv = x[((b * T + t) * H + h) * P + p];
                const double *Bt = B + ((b * T + t) * G + g) * N;
                const double *Ct = C + ((b * T + t) * G + g) * N;
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    hs[n] = decay * hs[n] + d * xv * Bt[n];
                    acc += Ct[n] * hs[n];
                }
                y[((b * T + t) * H + h) * P + p] = acc + (D ? D[h] * xv : 0.0);
                if (state_out && t == j)
                    memcpy(state_out + state_off, hs, sizeof(double) * (size_t)N);
            }
            if (final_state)
                memcpy(final_state + state_off, hs, sizeof(double) * (size_t)N);
        }
        free(hs);
    }
    return failed ? -6 : 0;
}
