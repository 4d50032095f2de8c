/*
 * ssd_oracle.h -- fp64 CPU oracle for the SSD layer forward and backward (test
 * infrastructure only).
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg use this
 * library.  It is independent of the HIP library: no shared code or headers.
 *
 * ssd_ref runs the scalar-decay selective SSM recurrence token by token in double
 * precision ("Mamba-2: Attention's Distant Cousin", sections "Writing an SSM as a
 * Matrix" and "Reducing A to a Single Number"), with decay exp(dt*A[h]), input scale
 * dt, a D[h]*x skip and B/C shared by the heads of a group.
 *
 * Arguments (host pointers, row-major, caller-owned):
 *   x [B][T][H][P], dt [B][T][H], A [H], B and C [B][T][G][N], D [H]
 *   init_state [B][H][N][P] or NULL (zeros)
 *   chunk_len   >0 to fill boundary_states, 0 when boundary_states is NULL
 *   y [B][T][H][P] (written), final_state [B][H][N][P] or NULL,
 *   boundary_states [B][H][ceil(T/chunk_len)][N][P] or NULL: the state after the last
 *     step of every chunk (the last chunk may be partial)
 *   nthreads    worker threads; <= 0 means one per online CPU (capped at B*H)
 * Returns 0 on success, otherwise one of the codes below; nothing is written on a
 * validation error.
 */
#ifndef SSD_ORACLE_H
#define SSD_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int64_t batch, seqlen, nheads, headdim, dstate, ngroups;
} ssd_ref_dims;

enum { SSD_REF_OK = 0, SSD_REF_ERR_NULL = 1, SSD_REF_ERR_DIMS = 2, SSD_REF_ERR_ALLOC = 3 };

int ssd_ref(const ssd_ref_dims* d, const double* x, const double* dt, const double* A,
            const double* B, const double* C, const double* D, const double* init_state,
            int64_t chunk_len, double* y, double* final_state, double* boundary_states,
            int nthreads);

/*
 * ssd_bwd_ref: gradients of a scalar loss through the same recurrence, by reverse-mode
 * differentiation step by step (fp64).  Inputs as for ssd_ref plus dy [B][T][H][P]
 * (dL/dy) and d_final [B][H][N][P] (dL/d final state) or NULL (zero).  Outputs:
 *   dx [B][T][H][P], ddt [B][T][H]
 *   dB_heads, dC_heads [B][T][H][N]: each head's share of dL/dB_t, dL/dC_t (the
 *     gradient of a group's B or C is the sum over the heads of that group)
 *   dA_parts, dD_parts [B][H]: each (batch, head)'s share of dL/dA[h], dL/dD[h]
 *   d_init [B][H][N][P] or NULL: dL/d init_state
 *   boundary_grads [B][H][ceil(T/chunk_len)][N][P] or NULL (then chunk_len may be 0):
 *     for every chunk, dL/d(state after its last step) through the later steps only
 */
int ssd_bwd_ref(const ssd_ref_dims* d, const double* x, const double* dt, const double* A,
                const double* B, const double* C, const double* D, const double* init_state,
                const double* dy, const double* d_final, int64_t chunk_len, double* dx,
                double* ddt, double* dB_heads, double* dC_heads, double* dA_parts,
                double* dD_parts, double* d_init, double* boundary_grads, int nthreads);

/* The number of threads ssd_ref runs with for these dims and this request. */
int ssd_ref_threads_used(const ssd_ref_dims* d, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
