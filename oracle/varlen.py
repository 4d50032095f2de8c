"""fp64 CPU oracle for packed variable-length sequences: several independent sequences laid
end to end in one row of tokens, each running the SSD recurrence from a zero state.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's CPU-baseline
leg are the only code allowed to import this module.  It shares no code with the HIP
library and never imports it.

Sources: "Mamba-2: Attention's Distant Cousin" (docsaid.org), section "Working Through
Four Tokens": the recurrence starts a sequence from a zero state.  The reproduction page
for arXiv 2405.21060 (citeark.co), in its list of reported claims: under sequence (context)
parallelism, the devices process contiguous pieces of one sequence and pass recurrent
states between them.  A state therefore belongs to one sequence.  Reading (the pages do
not discuss packing): sequence s covers the steps cu_seqlens[s] .. cu_seqlens[s+1]-1 of
the row and starts from a zero state; its final state is the state after its last step;
no state passes from one packed sequence into the next.

Functions
  ssd_varlen_ref     each sequence through the recurrence oracle (ssd_ref) on its own
  ssd_varlen_loop    the same by a plain Python loop over the whole row that resets the
                     state at every sequence start (tiny sizes; an independent check)
"""
import numpy as np


def _check_cu(cu_seqlens, T):
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 2 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must rise from 0 to T")
    return cu


def ssd_varlen_ref(x, dt, A, B, C, D, cu_seqlens, nthreads=0):
    """y [1,T,H,P] and final states [nseq,H,N,P] for the packed row (batch 1).

    x [1,T,H,P], dt [1,T,H], A [H], B/C [1,T,G,N], D [H]; cu_seqlens [nseq+1].  An empty
    sequence has a zero final state."""
    from . import ssd_ref
    x = np.asarray(x, dtype=np.float64)
    _, T, H, P = x.shape
    N = np.asarray(B).shape[3]
    cu = _check_cu(cu_seqlens, T)
    y = np.zeros_like(x)
    finals = np.zeros((cu.size - 1, H, N, P))
    for s in range(cu.size - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        ys, fs, _ = ssd_ref(x[:, a:b], np.asarray(dt)[:, a:b], A, np.asarray(B)[:, a:b],
                            np.asarray(C)[:, a:b], D, nthreads=nthreads)
        y[:, a:b] = ys
        finals[s] = fs[0]
    return y, finals


def ssd_varlen_loop(x, dt, A, B, C, D, cu_seqlens):
    """The packed row step by step in Python: one state per head, set to zero at the first
    step of every sequence.  O(T H N P) Python work: tiny inputs only."""
    x = np.asarray(x, dtype=np.float64)
    dt = np.asarray(dt, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    Bm = np.asarray(B, dtype=np.float64)
    Cm = np.asarray(C, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    _, T, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    cu = _check_cu(cu_seqlens, T)
    starts = set(int(v) for v in cu[:-1])
    y = np.zeros_like(x)
    finals = np.zeros((cu.size - 1, H, N, P))
    for h in range(H):
        g = h // (H // G)
        S = np.zeros((N, P))
        seq = -1
        for t in range(T):
            while seq + 1 < cu.size - 1 and t >= cu[seq + 1]:
                seq += 1
            if t in starts:
                S = np.zeros((N, P))
            a = np.exp(dt[0, t, h] * A[h])
            S = a * S + dt[0, t, h] * np.outer(Bm[0, t, g], x[0, t, h])
            y[0, t, h] = Cm[0, t, g] @ S + D[h] * x[0, t, h]
            if t == cu[seq + 1] - 1:
                finals[seq, h] = S
    return y, finals
