"""Algorithmic FLOP and byte counts of the four stage kernels, and the MI355X peaks.

"Algorithmic" means what the method must do, not what a kernel issues: every input is
read once and every output written once per launch; the quadratic part counts only the
causal half of each Q x Q diagonal block (the method never needs the upper triangle),
and C B^T is counted once per (batch, group, chunk) because the heads of a group share
it.  Bytes use the dtype sizes of the boundary (x, B, C, y and the stored chunk and
entry states in the input dtype; dt, cs, init and final states in fp32).  Where the chunk scan takes C B^T from a gram buffer (gram_bytes > 0:
the bf16 matrix-core path), the chunk_state stage also computes it (reading C, writing
the blocks once) and the scan reads the blocks once in place of B.
"""
from dataclasses import dataclass

# MI355X published peaks (dense; no sparsity).
PEAK_HBM_GBPS = 8000.0
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp32": 157.3, "fp64": 78.6}


@dataclass
class KernelCost:
    name: str
    bytes: float
    flops: float


def kernel_costs(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_len, dtype="bf16",
                 init_state=False, final_state=True, gram_bytes=0):
    B, T, H, P, N, G, Q = batch, seqlen, nheads, headdim, dstate, ngroups, chunk_len
    e = 2 if dtype == "bf16" else 4
    nC = (T + Q - 1) // Q
    chunk_f32 = B * H * nC * Q * 4          # dt_chunk or cs
    state_e = B * H * nC * P * N * e      # chunk states, in the input dtype
    entry = B * H * nC * P * N * e          # entry states, in the input dtype
    io_xy = B * T * H * P * e               # x or y
    io_bc = B * T * G * N * e               # B or C
    st1 = B * H * N * P * 4                 # init or final state
    cumsum = KernelCost("chunk_cumsum", B * T * H * 4 + H * 4 + 2 * chunk_f32, 2.0 * B * T * H)
    full, rem = divmod(T, Q)
    tri = full * Q * (Q + 1) + rem * (rem + 1)          # sum of 2*(j+1) over valid rows
    gram_flops = B * G * tri * N
    state = KernelCost("chunk_state", io_xy + io_bc + 2 * chunk_f32 + state_e
                       + (io_bc + gram_bytes if gram_bytes else 0),
                       2.0 * B * H * T * N * P + (gram_flops if gram_bytes else 0))
    passing = KernelCost("state_passing",
                         state_e + entry + B * H * nC * 4 + (st1 if init_state else 0)
                         + (st1 if final_state else 0),
                         2.0 * B * H * nC * N * P)
    # intra-chunk: sum over rows j of (j+1) MACs x P, per (b, h, chunk); C B^T likewise
    # per (b, g, chunk) over N; off-chunk: Q x N x P MACs per (b, h, chunk)
    if gram_bytes:
        scan = KernelCost("chunk_scan",
                          2 * io_xy + io_bc + gram_bytes + 2 * chunk_f32 + entry + H * 4,
                          B * H * tri * P + 2.0 * B * H * T * N * P)
        return [cumsum, state, passing, scan]
    scan = KernelCost("chunk_scan",
                      2 * io_xy + 2 * io_bc + 2 * chunk_f32 + entry + H * 4,
                      B * H * tri * P + gram_flops + 2.0 * B * H * T * N * P)
    return [cumsum, state, passing, scan]


def compulsory_bytes(batch, seqlen, nheads, headdim, dstate, ngroups, dtype="bf16",
                     init_state=False, final_state=True):
    e = 2 if dtype == "bf16" else 4
    B, T, H, P, N, G = batch, seqlen, nheads, headdim, dstate, ngroups
    st1 = B * H * N * P * 4
    return (2 * B * T * H * P * e + 2 * B * T * G * N * e + B * T * H * 4 + 2 * H * 4
            + (st1 if init_state else 0) + (st1 if final_state else 0))


def decode_cost(batch, nheads, headdim, dstate, ngroups, dtype="bf16"):
    """One decode step: the fp32 state read and written once, plus the step's inputs and
    output (x, y in the input dtype; B, C per group; dt per head; A, D)."""
    e = 2 if dtype == "bf16" else 4
    B, H, P, N, G = batch, nheads, headdim, dstate, ngroups
    nbytes = 2 * B * H * N * P * 4 + 2 * B * H * P * e + 2 * B * G * N * e + B * H * 4 + 2 * H * 4
    return KernelCost("decode_step", nbytes, 4.0 * B * H * N * P)


def bwd_costs(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_len, dtype="bf16",
              init_state=False, final_grad=True):
    """The kernels of the backward pass (ssd_bwd), in launch order: the forward stages it
    recomputes (cumsum, chunk states, entry states), the entry-state gradients of every
    chunk through its own outputs (bwd_dstate), their reverse carry (bwd_passing), the
    in-chunk gradients (bwd_chunk) and the ddt / dA / dD reductions (bwd_finalize).

    Counts follow the forward's conventions.  In-chunk FLOPs per (b, h): the causal
    dy x^T and the transposed masked product for dx (each Q(Q+1)/2 x P MACs per chunk),
    and three Q x N x P contractions (B F, F x, E dy); per (b, g): C B^T and the two
    head-summed products W^T C and W B for dB and dC (each causal, over N)."""
    B, T, H, P, N, G, Q = batch, seqlen, nheads, headdim, dstate, ngroups, chunk_len
    e = 2 if dtype == "bf16" else 4
    nC = (T + Q - 1) // Q
    chunk_f32 = B * H * nC * Q * 4
    state_e = B * H * nC * P * N * e
    io_xy = B * T * H * P * e
    io_bc = B * T * G * N * e
    st1 = B * H * N * P * 4
    full, rem = divmod(T, Q)
    tri = full * Q * (Q + 1) + rem * (rem + 1)
    fwd = kernel_costs(B, T, H, P, N, G, Q, dtype, init_state=init_state, final_state=False)
    cumsum, state, passing = fwd[0], fwd[1], fwd[2]
    dstate = KernelCost("bwd_dstate", io_xy + io_bc + chunk_f32 + state_e, 2.0 * B * H * T * N * P)
    rpass = KernelCost("bwd_passing",
                       2 * state_e + B * H * nC * 4 + (st1 if final_grad else 0) + st1,
                       2.0 * B * H * nC * N * P)
    chunk = KernelCost("bwd_chunk",
                       3 * io_xy + 4 * io_bc + 4 * chunk_f32 + 2 * state_e + H * 4,
                       B * H * (2.0 * tri * P + 6.0 * T * N * P) + 3.0 * B * G * tri * N)
    fin = KernelCost("bwd_finalize", 3 * chunk_f32 + B * T * H * 4 + 2 * H * 4, 4.0 * B * T * H)
    return [cumsum, state, passing, dstate, rpass, chunk, fin]


def block_costs(batch, seqlen, nheads, headdim, dstate, ngroups, conv_k, dtype="bf16",
                norm_bias=True):
    """The block's own kernels around the layer.

    block_prologue: reads the x|B|C columns (Cd = H*P + 2*G*N per token) and dt_raw of the
      projection output plus the filters; writes x, B, C in dtype and dt in fp32.  FLOPs per
      channel element: 2K for the filter and 4 for SiLU (exp, add, reciprocal, multiply);
      per step size 4 (softplus and the bias).
    block_epilogue: reads y and z (H*P per token) and the scale/shift; writes out.  FLOPs
      per element: 5 for the gate (SiLU and the product), 3 for the two reductions, 3 to
      normalise and scale (4 with the shift)."""
    e = 2 if dtype == "bf16" else 4
    bt = batch * seqlen
    d = nheads * headdim
    cd = d + 2 * ngroups * dstate
    pro = KernelCost("block_prologue",
                     bt * cd * e * 2 + bt * nheads * (e + 4) + cd * (conv_k + 1) * 4 + nheads * 4,
                     bt * cd * (2.0 * conv_k + 4) + 4.0 * bt * nheads)
    epi = KernelCost("block_epilogue",
                     3 * bt * d * e + (2 if norm_bias else 1) * d * 4,
                     bt * d * (11.0 + (1 if norm_bias else 0)))
    return [pro, epi]
