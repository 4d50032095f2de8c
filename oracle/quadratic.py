"""The quadratic (attention-like) dual form of the SSD layer, in numpy fp64.

Test infrastructure only.  This is the second, independent oracle form: it never runs
the recurrence.  It builds the T x T matrix M = L o (C B^T) explicitly and multiplies.
Cost is O(T^2) memory and O(T^3) for the mask, so it is for tiny inputs only.

Sources
  "Mamba-2: Attention's Distant Cousin" (docsaid.org), section "Reducing A to a Single
  Number": with A_t = a_t I the matrix factors as M = L o (C B^T), with L_ji the product
  a_j ... a_{i+1} for j >= i (1 on the diagonal) and 0 above it.
  Structured summary of arXiv 2405.21060 (paper-graph-ui), sections "The 1-Semiseparable
  Matrix" (equation 6, the 1SS matrix) and "The SSD Layer: Formal Definition"
  (M_ji = a_{j:i} C_j^T B_i, Y = M X).

The input-side scale dt_i, the D skip and the init-state term follow the same reading
as the recurrence oracle: decay a_t = exp(dt_t A_h), input dt_t x_t, y += D_h x, and a
state entering step 0 that is decayed by a_0 ... a_j before it is read at step j.
"""
import numpy as np


def one_ss_mask(a):
    """L = 1SS(a): L[j, i] = a[i+1] * ... * a[j] for j >= i (empty product 1), else 0."""
    a = np.asarray(a, dtype=np.float64)
    T = a.shape[0]
    L = np.zeros((T, T))
    for j in range(T):
        for i in range(j + 1):
            L[j, i] = np.prod(a[i + 1:j + 1])
    return L


def ssd_quadratic(x, dt, A, B, C, D, init_state=None):
    """y and final state of the SSD layer by the quadratic form.

    Shapes as for the recurrence oracle: x [B,T,H,P], dt [B,T,H], A [H], B/C [B,T,G,N],
    D [H], init_state [B,H,N,P] or None.  Returns (y [B,T,H,P], final [B,H,N,P]).
    The final state is the unrolled sum h_{T-1} = sum_s a_{T-1:s} dt_s B_s x_s^T plus the
    decayed init state.
    """
    x = np.asarray(x, dtype=np.float64)
    dt = np.asarray(dt, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    bsz, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    y = np.zeros_like(x)
    final = np.zeros((bsz, H, N, P))
    for b in range(bsz):
        for h in range(H):
            g = h // hpg
            a = np.exp(dt[b, :, h] * A[h])                  # decay of every step
            L = one_ss_mask(a)                              # T x T
            Gm = C[b, :, g, :] @ B[b, :, g, :].T            # G[j, i] = C_j . B_i
            M = L * Gm
            u = dt[b, :, h, None] * x[b, :, h, :]           # dt-scaled input [T, P]
            yh = M @ u + D[h] * x[b, :, h, :]
            # unrolled state: h_T-1 = sum_s (a_{s+1} ... a_{T-1}) dt_s B_s x_s^T
            wlast = L[T - 1, :] if T > 0 else np.zeros(0)
            fin = (B[b, :, g, :] * wlast[:, None]).T @ u
            if init_state is not None:
                s0 = np.asarray(init_state, dtype=np.float64)[b, h]       # [N, P]
                pref = np.array([np.prod(a[:j + 1]) for j in range(T)])   # a_0 ... a_j
                yh = yh + pref[:, None] * (C[b, :, g, :] @ s0)
                fin = fin + (np.prod(a) * s0)
            y[b, :, h, :] = yh
            final[b, h] = fin
    return y, final
