/*
 * ssd.h -- libssd: the Mamba-2 SSD (state space dual) layer on AMD MI355X (gfx950): the
 * forward, its backward, the single-token recurrent step, and the block's prologue and
 * epilogue around the layer (convolution, step sizes, gate, normalisation).
 *
 * The operation ("Mamba-2: Attention's Distant Cousin", docsaid.org, sections "Writing an
 * SSM as a Matrix" and "Reducing A to a Single Number"; structured summary of arXiv
 * 2405.21060, section "The SSD Layer: Formal Definition"): for every batch element b and
 * head h, a scalar-decay selective SSM with an N x P state S,
 *
 *     S_t = exp(dt[b,t,h] * A[h]) * S_{t-1} + dt[b,t,h] * B[b,t,g] x[b,t,h]^T
 *     y[b,t,h] = C[b,t,g]^T S_t + D[h] * x[b,t,h]
 *
 * where g = h / (H / G) is the B/C group of head h (heads share B and C within a group,
 * summary section "The Mamba-2 Architecture", head patterns) and S_{-1} is init_state.
 * Equivalently y = M x per head with M = L o (C B^T), L the 1-semiseparable decay mask.
 *
 * It is computed by the block decomposition of M into chunks of chunk_len steps
 * (summary section "The Block-Decomposition SSD Algorithm", stages 0 to 5), as four
 * stage calls that ssd_fwd makes in order on one stream, each also exported on its own:
 *   ssd_chunk_cumsum   stage 0: chunk-local inclusive prefix sums of dt*A (log decays)
 *   ssd_chunk_state    stage 2: every chunk's final state from a zero start (and, given a
 *                      gram buffer, the first half of stage 1 below in the same pass)
 *   ssd_state_passing  stage 3: the 1-SS scan over chunks that carries states across them
 *   ssd_chunk_gram     stage 1, first half: the causal blocks of C B^T of every chunk,
 *                      once per group (bf16 MFMA path only; a no-op elsewhere)
 *   ssd_chunk_scan     stages 1, 4, 5: the masked quadratic form inside each chunk plus
 *                      the carried state read out by C, plus the D skip
 *
 * Conventions for every entry point
 *   - Pointers are device pointers (hipMalloc'd or equivalent), row-major and
 *     contiguous.  x, B, C, y, dt_chunk, cs, the state buffers and the workspace must be
 *     16-byte aligned; dt, A, D, init_state and final_state 4-byte aligned (else
 *     SSD_ERR_ALIGN).  The caller owns every buffer.  The library allocates nothing.  The
 *     only state it keeps between calls is per device and per kernel: on a kernel's first
 *     launch on a device it raises the kernel's LDS limit and notes how many of its
 *     workgroups fit on the device at once (held in atomics, so concurrent first calls
 *     from several host threads are safe).  Calls on different streams are therefore
 *     independent; calls that share output or workspace buffers race.
 *   - No output or workspace may overlap an input, another output or the workspace of
 *     the same call (not checked: kernels read inputs that other workgroups' outputs
 *     would already have overwritten), except where an entry point states otherwise.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default stream.  Work is
 *     enqueued asynchronously; a return of SSD_OK means "enqueued".
 *   - Arguments are validated before any launch; on an error nothing is enqueued.
 *   - Values are not checked: dt >= 0 and A <= 0 (so every decay lies in (0, 1]) are the
 *     caller's contract.  Other values still give the same arithmetic, but a positive
 *     dt*A sum inside a chunk can overflow exp.
 *   - Supported sizes: chunk_len in {64, 128, 256}; dstate N in {16, 32, 64, 128, 256};
 *     headdim P in {16, 32, 64, 128}; ngroups G >= 1 dividing nheads H; any seqlen
 *     T >= 0 (the last chunk may be partial); batch >= 0; fewer than 2^31 elements in
 *     x, in B and in the chunk states, counting T rounded up to whole chunks (else
 *     SSD_ERR_DIMS).  dtype SSD_F32 or SSD_BF16 for x, B, C and y (and the stored chunk and
 *     entry states); dt, A, D, init_state, final_state and cs are always fp32.
 *
 * Tensor layouts
 *   x, y           [batch][seqlen][nheads][headdim]       in `dtype`
 *   dt             [batch][seqlen][nheads]                fp32
 *   A, D           [nheads]                               fp32
 *   B, C           [batch][seqlen][ngroups][dstate]       in `dtype`
 *   init_state, final_state  [batch][nheads][dstate][headdim]   fp32
 *   dt_chunk, cs   [batch][nheads][nchunks][chunk_len]    fp32, nchunks = ceil(T/chunk_len)
 *   chunk states   [batch][nheads][nchunks][headdim][dstate]   in `dtype`
 *   entry states   [batch][nheads][nchunks][headdim][dstate]   in `dtype` (the chunk scan
 *                  consumes them as operands of that dtype; the state carried from chunk
 *                  to chunk is fp32, and each chunk's state is rounded to `dtype` once
 *                  when it is stored)
 *     (state buffers are headdim-major: the transpose of the N x P state of the formulas)
 */
#ifndef LIBSSD_SSD_H
#define LIBSSD_SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL = 1,        /* a required pointer is NULL */
    SSD_ERR_DIMS = 2,        /* a size is negative, zero where it must not be, too large,
                                or nheads is not a multiple of ngroups */
    SSD_ERR_UNSUPPORTED = 3, /* chunk_len, dstate, headdim or dtype outside the supported set */
    SSD_ERR_ALIGN = 4,       /* a pointer is not aligned as the conventions require */
    SSD_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than ssd_fwd_workspace_size() */
    SSD_ERR_HIP = 6          /* the HIP runtime reported an error at launch */
} ssd_status;

typedef struct {
    int64_t batch;   /* B */
    int64_t seqlen;  /* T */
    int64_t nheads;  /* H */
    int64_t headdim; /* P */
    int64_t dstate;  /* N */
    int64_t ngroups; /* G */
} ssd_dims;

/* Human-readable name of a status code (a static string; never NULL). */
const char* ssd_status_string(ssd_status status);

/* Bytes of device workspace ssd_fwd needs for these sizes, for either dtype (0 if the
 * sizes are invalid).  It holds dt_chunk, cs, the chunk states, the entry states and the
 * C B^T blocks (ssd_chunk_gram_size for SSD_BF16), each 256-byte aligned, in that order. */
size_t ssd_fwd_workspace_size(const ssd_dims* dims, int chunk_len);

/* The whole SSD forward: y and (optionally) final_state from x, dt, A, B, C, D and an
 * optional init_state.  Runs the four stage kernels below on `stream`.
 *   init_state   NULL for a zero initial state
 *   final_state  NULL to skip writing the state after the last step
 *   workspace    device buffer of at least ssd_fwd_workspace_size(dims, chunk_len) bytes;
 *                its contents on return are the stage intermediates (see the stage calls)
 * Errors: SSD_ERR_NULL, SSD_ERR_DIMS, SSD_ERR_UNSUPPORTED, SSD_ERR_ALIGN,
 * SSD_ERR_WORKSPACE before any launch; SSD_ERR_HIP if a launch fails. */
ssd_status ssd_fwd(const ssd_dims* dims, ssd_dtype dtype, const void* x, const float* dt,
                   const float* A, const void* B, const void* C, const float* D,
                   int chunk_len, const float* init_state, void* y, float* final_state,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the fixed device array ssd_fwd_noalloc keeps its stage buffers in (one per GPU). */
#define SSD_NOALLOC_SCRATCH_BYTES (256u << 20)

/* ssd_fwd for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The same computation and kernels
 * as ssd_fwd (bit-identical y and final_state), with the stage buffers (dt_chunk, cs, chunk
 * and entry states in `dtype`, C B^T blocks) taken from a fixed array of
 * SSD_NOALLOC_SCRATCH_BYTES inside the library instead of a caller's workspace.  Nothing is
 * allocated by the call: the runtime reserves the array on each GPU when the library's code
 * is first loaded there, and it stays reserved until the process ends.  The first call on a
 * device looks up the array's device address (hipGetSymbolAddress); later calls reuse it.
 * Limit: the stage buffers, 8*B*H*ceil(T/Q)*Q + 2*B*H*ceil(T/Q)*P*N*sizeof(dtype) bytes plus
 * the C B^T blocks (ssd_chunk_gram_size), each rounded up to 256 bytes, must fit the array
 * (e.g. B=4, T=4096, H=80, P=64, N=128, Q=256 in bf16 needs 183 MB); larger problems return
 * SSD_ERR_WORKSPACE before any launch.  Every call on one GPU shares its array: calls that
 * overlap in time on one GPU (concurrent streams, or host threads) race and must not be
 * issued.  Arguments and other errors as ssd_fwd. */
ssd_status ssd_fwd_noalloc(const ssd_dims* dims, ssd_dtype dtype, const void* x, const float* dt,
                           const float* A, const void* B, const void* C, const float* D,
                           int chunk_len, const float* init_state, void* y, float* final_state,
                           void* stream);

/* Stage 0 (summary section "The Block-Decomposition SSD Algorithm", step 0, and the log
 * form of the 1-SS mask entries a_j ... a_{i+1}): for every (b, h, chunk c) and
 * position i < chunk_len, with t = c*chunk_len + i,
 *     dt_chunk[b][h][c][i] = dt[b][t][h]                (0 when t >= T)
 *     cs[b][h][c][i]       = sum_{k <= i} dt_chunk[b][h][c][k] * A[h]
 * so positions past a partial last chunk repeat the chunk's last prefix sum. */
ssd_status ssd_chunk_cumsum(const ssd_dims* dims, int chunk_len, const float* dt,
                            const float* A, float* dt_chunk, float* cs, void* stream);

/* Stage 2 (same section, "Compute chunk-final states"): the state at the end of every
 * chunk when the chunk starts from zero, i.e. from the chunk's own inputs only:
 *     states[b][h][c][p][n] = sum_i exp(cs[c][Q-1] - cs[c][i]) * dt_chunk[c][i]
 *                                   * B[b][cQ+i][g][n] * x[b][cQ+i][h][p]
 * (sum over the chunk's valid positions i), accumulated in fp32 and stored in `dtype`.
 * dt_chunk and cs come from ssd_chunk_cumsum.
 * gram: NULL, or a buffer of ssd_chunk_gram_size bytes that is also filled exactly as
 * ssd_chunk_gram(dims, dtype, chunk_len, B, C, gram) would fill it (C is then required;
 * where ssd_chunk_gram_size is 0 both are ignored).  The states kernel already holds each
 * chunk's B, so for some shapes the blocks come from the same pass. */
ssd_status ssd_chunk_state(const ssd_dims* dims, ssd_dtype dtype, int chunk_len,
                           const void* x, const void* B, const float* dt_chunk,
                           const float* cs, void* states, const void* C, void* gram,
                           void* stream);

/* Stage 3 (same section, "Propagate states between chunks"): the sequential 1-SS scan
 * over chunks.  With E_0 = init_state (zeros if NULL), carried in fp32,
 *     entry_states[c] = E_c,   E_{c+1} = exp(cs[c][Q-1]) * E_c + states[c]
 * and final_state = E_nchunks (the state after the last step, fp32; NULL to skip).
 * states are read and entry_states written in `dtype` (bf16: rounded to nearest even).
 * entry_states may not alias states (SSD_ERR_DIMS).  init_state/final_state use the
 * [N][P] layout, states/entry_states the [P][N] one. */
ssd_status ssd_state_passing(const ssd_dims* dims, ssd_dtype dtype, int chunk_len,
                             const void* states, const float* cs, const float* init_state,
                             void* entry_states, float* final_state, void* stream);

/* Bytes of the `gram` buffer that ssd_chunk_gram fills and ssd_chunk_scan reads for these
 * sizes and dtype; 0 where the chunk scan does not use one (SSD_F32, or invalid sizes). */
size_t ssd_chunk_gram_size(const ssd_dims* dims, ssd_dtype dtype, int chunk_len);

/* Stage 1, first half (same section, "Compute the diagonal blocks", and summary section
 * "The Mamba-2 Architecture": B and C are shared by the heads of a group, so C B^T is
 * too): for every (b, g, chunk c), the causal 32 x 32 blocks (row block >= column block)
 * of the chunk's Q x Q matrix G[j][i] = C_j . B_i, rounded to bf16, with rows and
 * columns past the end of a partial chunk set to zero.  The buffer's layout is private to
 * the library: it holds the blocks as the chunk scan's matrix-core operands, is
 * ssd_chunk_gram_size bytes long and is only meant to be passed to ssd_chunk_scan with
 * the same dims, dtype and chunk_len.  With no gram buffer for these sizes (size 0) the
 * call does nothing and returns SSD_OK; otherwise B, C and gram must be non-NULL and
 * 16-byte aligned. */
ssd_status ssd_chunk_gram(const ssd_dims* dims, ssd_dtype dtype, int chunk_len,
                          const void* B, const void* C, void* gram, void* stream);

/* Stages 1, 4 and 5 (same section: intra-chunk outputs, inter-chunk outputs, combine):
 * for every position j of chunk c (t = cQ + j < T),
 *     y[b][t][h][p] = sum_{i <= j} (C_j . B_i) exp(cs[j] - cs[i]) dt_chunk[i] x[cQ+i][p]
 *                   + exp(cs[j]) sum_n C_j[n] entry_states[c][p][n]
 *                   + D[h] x[b][t][h][p]
 * with C_j = C[b][cQ+j][g], B_i = B[b][cQ+i][g]; entry_states are read in `dtype`.
 * gram is the buffer ssd_chunk_gram filled from the same B and C (the bf16 path takes
 * C_j . B_i from it, rounded to bf16, and does not read B); where
 * ssd_chunk_gram_size is 0 it is ignored and may be NULL. */
ssd_status ssd_chunk_scan(const ssd_dims* dims, ssd_dtype dtype, int chunk_len,
                          const void* x, const void* B, const void* C, const float* dt_chunk,
                          const float* cs, const float* D, const void* entry_states,
                          const void* gram, void* y, void* stream);

/* ---- backward ----------------------------------------------------------------------
 * The pages' headline claim is training speed (structured summary of arXiv 2405.21060,
 * section "1. Executive Summary": 2-8x faster training than Mamba's selective scan), and
 * training needs the gradient of the layer.  The pages define only the forward; the
 * backward here is its exact derivative, computed with the same block decomposition run in
 * reverse: the chunk states and entry states are recomputed, each chunk's entry-state
 * gradient through its own outputs (Z_c = sum_i exp(cs_i) C_i dy_i^T) is carried from the
 * last chunk to the first (dE_c = Z_c + exp(cs[c][Q-1]) dE_{c+1}, dE_nchunks = d_final),
 * and inside each chunk the transposed quadratic form gives dx, dB, dC and the gradients of
 * the log decays, from which ddt and dA follow by suffix sums over the chunk. */

/* Bytes of device workspace ssd_bwd needs for these sizes, for either dtype (0 if the
 * sizes are invalid). */
size_t ssd_bwd_workspace_size(const ssd_dims* dims, int chunk_len);

/* Gradients of a scalar loss L through ssd_fwd with the same inputs, given
 *   dy       dL/dy        [batch][seqlen][nheads][headdim]        in `dtype`
 *   d_final  dL/d final_state [batch][nheads][dstate][headdim] fp32, NULL for zero
 * (x, dt, A, B, C, D, chunk_len and init_state exactly as passed to ssd_fwd).  Writes
 *   dx [B][T][H][P] and dB, dC [B][T][G][N] in `dtype` (dB, dC summed over the heads of
 *     each group, in fp32, then rounded once),
 *   ddt [B][T][H], dA [H], dD [H] fp32 (dA and dD summed over batch and time),
 *   d_init [B][H][N][P] fp32 (dL/d init_state; NULL to skip -- with a NULL init_state it is
 *     still the gradient with respect to the zero initial state).
 * The result does not depend on chunk_len beyond rounding.  Every output is written in
 * full; dA and dD even when batch or seqlen is 0 (then zero), and d_init = d_final (or
 * zero) when seqlen is 0.  Reductions run in a fixed order: results are bitwise
 * reproducible run to run.  Alignment: x, B, C, dy, dx, dB, dC and workspace 16 bytes;
 * the fp32 arguments 4 bytes.  workspace: ssd_bwd_workspace_size bytes, contents
 * unspecified on return.  Errors as ssd_fwd. */
ssd_status ssd_bwd(const ssd_dims* dims, ssd_dtype dtype, const void* x, const float* dt,
                   const float* A, const void* B, const void* C, const float* D,
                   int chunk_len, const float* init_state, const void* dy,
                   const float* d_final, void* dx, float* ddt, float* dA, void* dB, void* dC,
                   float* dD, float* d_init, void* workspace, size_t workspace_bytes,
                   void* stream);

/* ssd_bwd for training, where the forward has just run: the same gradients, reading the
 * log decays (dt_chunk, cs) and the entry states from the workspace of the ssd_fwd call
 * instead of recomputing them (three of ssd_bwd's launches fewer).
 *   fwd_workspace  the workspace passed to ssd_fwd with the same dims, dtype, chunk_len and
 *                  inputs (x, dt, A, B, C, init_state), not modified since; read only;
 *                  16-byte aligned; NULL is SSD_ERR_NULL
 * Every other argument and the result are as for ssd_bwd (bit-identical: the same kernels
 * produce the same intermediates). */
ssd_status ssd_bwd_saved(const ssd_dims* dims, ssd_dtype dtype, const void* x, const float* dt,
                         const float* A, const void* B, const void* C, const float* D,
                         int chunk_len, const float* init_state, const void* dy,
                         const float* d_final, const void* fwd_workspace, void* dx, float* ddt,
                         float* dA, void* dB, void* dC, float* dD, float* d_init,
                         void* workspace, size_t workspace_bytes, void* stream);

/* One recurrent step for a batch of sequences ("Mamba-2: Attention's Distant Cousin",
 * section "Working Through Four Tokens": the recurrent form, the one generation uses, with
 * a state of fixed size).  For every (b, h), g = h / (H / G):
 *     state[b][h] <- exp(dt[b][h] * A[h]) * state[b][h] + dt[b][h] * B[b][g] x[b][h]^T
 *     y[b][h]      = C[b][g]^T state[b][h] + D[h] * x[b][h]
 * computed in fp32 -- exactly one step of the recurrence that ssd_fwd computes by chunks.
 * dims->seqlen is ignored (one step); the other sizes are checked as for ssd_fwd.
 *   x, y     [batch][nheads][headdim]            in `dtype`
 *   dt       [batch][nheads]                     fp32
 *   A, D     [nheads]                            fp32
 *   B, C     [batch][ngroups][dstate]            in `dtype`
 *   state    [batch][nheads][dstate][headdim]    fp32, read and updated in place (the
 *            layout of init_state / final_state: ssd_fwd's final_state continues here)
 * x and state must be 16-byte aligned, the others 4-byte aligned.  Errors as ssd_fwd;
 * nothing needs a workspace. */
ssd_status ssd_decode_step(const ssd_dims* dims, ssd_dtype dtype, const void* x,
                           const float* dt, const float* A, const void* B, const void* C,
                           const float* D, float* state, void* y, void* stream);

/* ---- packed variable-length rows -------------------------------------------------------
 * Several independent sequences laid end to end in one row of steps (batch 1), sequence s
 * covering steps cu_seqlens[s] .. cu_seqlens[s+1]-1.  Each starts from a zero state and no
 * state passes from one into the next ("Mamba-2: Attention's Distant Cousin", section
 * "Working Through Four Tokens": a sequence starts from zero; the reproduction page for
 * arXiv 2405.21060 (citeark.co), reported claims: context parallelism passes a state
 * between contiguous pieces of one sequence).  The four forward stages run unchanged:
 * ssd_chunk_cumsum's running log-decay sum drops by a gap of 120 at every sequence start,
 * which makes every decay across a start exactly zero in fp32.  The gaps cost some
 * precision inside a chunk that holds several starts: with k starts in one chunk the
 * log-decays reach about -(120 k + 254), and each decay carries a relative error of
 * about ulp(120 k + 254), e.g. 6e-5 for k = 3.  Measured with about 100 starts per chunk
 * (sequences of 1-4 steps), rel-L2 against the fp64 oracle: in fp32 1.8e-5 on y and
 * 2.5e-4 on the final states (above ssd_fwd's fp32 bound of 1e-4: this is that limit); in
 * bf16 1.7e-3, within ssd_fwd's bf16 bound. */

/* Bytes of workspace ssd_fwd_varlen needs: ssd_fwd's for these sizes (0 if the sizes are
 * invalid or batch != 1). */
size_t ssd_fwd_varlen_workspace_size(const ssd_dims* dims, int chunk_len);

/* y [1][T][H][P] for a packed row, and optionally every sequence's final state.
 *   dims         batch must be 1 (else SSD_ERR_DIMS); T = total steps
 *   cu_seqlens   device int32 [nseq + 1], rising from 0 to T (not checked: the caller's
 *                contract, like dt >= 0); empty sequences are allowed
 *   nseq         number of sequences, >= 1
 *   final_states NULL, or [nseq][H][N][P] fp32: the state after each sequence's last step
 *                (zero for an empty sequence)
 * x, dt, A, B, C, D, chunk_len, y and the alignment rules as for ssd_fwd (no init_state:
 * every sequence starts from zero); workspace of ssd_fwd_varlen_workspace_size bytes. */
ssd_status ssd_fwd_varlen(const ssd_dims* dims, ssd_dtype dtype, const void* x, const float* dt,
                          const float* A, const void* B, const void* C, const float* D,
                          int chunk_len, const int32_t* cu_seqlens, int64_t nseq, void* y,
                          float* final_states, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ---- the block around the layer ----------------------------------------------------
 * The Mamba-2 block between its input and output projections ("Mamba-2: Attention's
 * Distant Cousin", section "The Mamba-2 Block", Figure 6; structured summary of arXiv
 * 2405.21060, section "The Mamba-2 Architecture" and section 6.4): one projection yields,
 * per token, the rows [z | x | B | C | dt_raw] of widths H*P, H*P, G*N, G*N, H.  The x, B, C
 * channels pass through a depthwise causal convolution of width K (3-4 on the pages) and
 * SiLU (the activation after the convolution, and the default feature map on B and C); the
 * step size is made positive by softplus after a per-head bias.  After the layer, y is
 * gated by SiLU(z) and normalised per token over contiguous channel groups (GroupNorm,
 * the default extra normalisation, or its RMS variant).  The projections themselves are
 * plain GEMMs and not part of this library.  Computation in fp32; x, B, C, z, y and out in
 * `dtype`. */

/* Prologue.  With Cd = H*P + 2*G*N, for every b, t < T and channel c < Cd:
 *   v[b][t][c] = SiLU(conv_b[c] + sum_{k<K} conv_w[c*K + k] * xbc[b][t-(K-1)+k][c])
 *   (xbc = 0 before t = 0; conv_w[c*K + K-1] weights the current step), and
 *   x[b][t][h][p] = v[b][t][h*P + p],  B[b][t][g][n] = v[b][t][H*P + g*N + n],
 *   C[b][t][g][n] = v[b][t][H*P + G*N + g*N + n],
 *   dt[b][t][h] = softplus(dt_raw[b][t][h] + dt_bias[h]) = log(1 + exp(.)).
 *   xbc     device, rows of Cd channels in `dtype`, row r = b*T + t at r * xbc_stride
 *           elements (xbc_stride >= Cd); rows may sit inside a wider projection output
 *   conv_w  [Cd][K] fp32, conv_b [Cd] fp32 or NULL (zero); conv_k = K in 1..8
 *   dt_raw  rows of H values in `dtype` at dt_stride elements (>= H); dt_bias [H] or NULL
 *   x, B, C [B][T][H][P], [B][T][G][N], [B][T][G][N] in `dtype` (16-byte aligned), and
 *   dt      [B][T][H] fp32: the inputs ssd_fwd takes.
 * xbc and dt_raw need only element alignment (16-byte alignment of xbc and a row stride
 * that is a multiple of 16 bytes take the vector path).  Errors as ssd_fwd; SSD_ERR_DIMS
 * for a stride below the row width; SSD_ERR_UNSUPPORTED for K outside 1..8. */
ssd_status ssd_block_prologue(const ssd_dims* dims, ssd_dtype dtype, const void* xbc,
                              int64_t xbc_stride, const float* conv_w, const float* conv_b,
                              int conv_k, const void* dt_raw, int64_t dt_stride,
                              const float* dt_bias, void* x, void* B, void* C, float* dt,
                              void* stream);

/* Epilogue.  With D = H*P channels split into norm_groups contiguous groups of S = D /
 * norm_groups, for every b, t and group q, over its channels c:
 *   v[c] = y[b][t][c] * SiLU(z[b][t][c])
 *   GroupNorm (rms = 0): m = mean(v), s2 = mean((v - m)^2),
 *                        out[c] = (v[c] - m) / sqrt(s2 + eps) * norm_w[c] + norm_b[c]
 *   RMS (rms != 0):      out[c] = v[c] / sqrt(mean(v^2) + eps) * norm_w[c]   (no norm_b)
 *   y    [B][T][H][P] in `dtype` (16-byte aligned: ssd_fwd's output)
 *   z    rows of D values in `dtype` at z_stride elements (>= D)
 *   norm_w [D] fp32, norm_b [D] fp32 or NULL (zero); eps >= 0
 *   out  [B][T][H*P] in `dtype`, 16-byte aligned (may alias y).
 * Errors as ssd_fwd; SSD_ERR_DIMS if norm_groups does not divide H*P. */
ssd_status ssd_block_epilogue(const ssd_dims* dims, ssd_dtype dtype, const void* y,
                              const void* z, int64_t z_stride, const float* norm_w,
                              const float* norm_b, int norm_groups, int rms, float eps,
                              void* out, void* stream);

/* Bytes of workspace ssd_block_fwd needs (0 if the sizes are invalid): x, y, B, C of the
 * layer and ssd_fwd's own workspace. */
size_t ssd_block_fwd_workspace_size(const ssd_dims* dims, ssd_dtype dtype, int chunk_len);

/* 1 if ssd_block_fwd applies the gate and the norm inside the chunk scan for these sizes
 * (bf16 on the matrix-core scan, headdim 32 or 64, every norm group inside one head: S =
 * H*P / norm_groups channels, S a multiple of 16 that divides P, and 8-byte aligned
 * projection rows of which chunk_len span under 2^31 bytes), given 16-byte aligned norm_w
 * and norm_b; 0 otherwise, also for invalid sizes.  Reads no device state. */
int ssd_block_fwd_norm_in_scan(const ssd_dims* dims, ssd_dtype dtype, int chunk_len,
                               int norm_groups);

/* The block between the projections: ssd_block_prologue on the x|B|C and dt_raw columns of
 * zxbcdt ([B][T] rows of 2*H*P + 2*G*N + H values, [z | x | B | C | dt_raw], contiguous,
 * 16-byte aligned), ssd_fwd (A, D, chunk_len, init_state, final_state as there), then
 * ssd_block_epilogue with z from the first H*P columns; out [B][T][H*P] in `dtype`.  The
 * step sizes softplus(dt_raw + dt_bias) are made inside the forward's cumsum pass, straight
 * from the dt_raw columns (the same arithmetic as ssd_block_prologue's), and dt is never
 * stored.  Where ssd_block_fwd_norm_in_scan says so and norm_w, norm_b are 16-byte aligned,
 * the gate and the norm run in the chunk scan's store (y is never stored, no epilogue pass):
 * the result then differs from the three calls only by the rounding of y to `dtype` before
 * the norm; otherwise it equals the three calls bit for bit.  Errors as the three calls, all
 * checked before the first launch. */
ssd_status ssd_block_fwd(const ssd_dims* dims, ssd_dtype dtype, const void* zxbcdt,
                         const float* conv_w, const float* conv_b, int conv_k,
                         const float* dt_bias, const float* A, const float* D, int chunk_len,
                         const float* init_state, const float* norm_w, const float* norm_b,
                         int norm_groups, int rms, float eps, void* out, float* final_state,
                         void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LIBSSD_SSD_H */
