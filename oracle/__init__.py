"""fp64 CPU oracle for the SSD layer, forward and backward.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only code allowed to import this package.  It shares no
code with the HIP library and never imports it.

Contents
  ssd_ref          token-by-token recurrence (C, fp64, threads over (batch, head))
  ssd_bwd_ref      gradients by reverse-mode differentiation of the recurrence (C, fp64)
  ssd_quadratic    the dual quadratic form y = (L o C B^T) (dt x) + ...  (numpy, tiny sizes)
  chunk_cumsum     chunk-local inclusive prefix sums of dt*A
  chunk_states     per-chunk states that start from zero (the chunk's own input only)
  entry_states     the state entering every chunk (init for chunk 0)
  chunk_entry_grads  dL/d(entry state of a chunk) through that chunk's own outputs only

Sources: "Mamba-2: Attention's Distant Cousin" (docsaid.org), sections "Writing an SSM
as a Matrix", "Reducing A to a Single Number", "Working Through Four Tokens"; and the
structured summary of arXiv 2405.21060 (paper-graph-ui), sections "The SSD Layer:
Formal Definition" and "The Block-Decomposition SSD Algorithm" (stages 0 to 3).
"""
import ctypes
import os

import numpy as np

from . import build as _build
from .quadratic import ssd_quadratic, one_ss_mask  # noqa: F401

_LIB = None


class _Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("headdim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64)]


def library():
    """Load oracle/libssd_oracle.so, compiling it with gcc first if it is absent."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIBRARY):
            _build.compile_oracle()
        _LIB = load_library(_build.LIBRARY)
    return _LIB


def load_library(path):
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.ssd_ref.restype = ctypes.c_int
    lib.ssd_ref.argtypes = [ctypes.POINTER(_Dims), dp, dp, dp, dp, dp, dp, dp,
                            ctypes.c_int64, dp, dp, dp, ctypes.c_int]
    lib.ssd_bwd_ref.restype = ctypes.c_int
    lib.ssd_bwd_ref.argtypes = [ctypes.POINTER(_Dims), dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                ctypes.c_int64, dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int]
    lib.ssd_ref_threads_used.restype = ctypes.c_int
    lib.ssd_ref_threads_used.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int]
    return lib


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def dims_of(x, B):
    b, t, h, p = x.shape
    g, n = B.shape[2], B.shape[3]
    return _Dims(b, t, h, p, n, g)


def ssd_ref(x, dt, A, B, C, D, init_state=None, chunk_len=0, nthreads=0, lib=None):
    """Run the recurrence in fp64.

    x [B,T,H,P], dt [B,T,H], A [H], B/C [B,T,G,N], D [H], init_state [B,H,N,P] or None.
    Returns (y [B,T,H,P], final_state [B,H,N,P], boundary_states [B,H,nC,N,P] or None),
    where boundary_states holds the state after the last step of every chunk of
    chunk_len steps (only when chunk_len > 0).
    """
    lib = lib or library()
    x, dt, A, B, C, D = (_f64(v) for v in (x, dt, A, B, C, D))
    init = None if init_state is None else _f64(init_state)
    bsz, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if dt.shape != (bsz, T, H) or A.shape != (H,) or D.shape != (H,):
        raise ValueError("dt/A/D shapes do not match x")
    if B.shape != (bsz, T, G, N) or C.shape != B.shape:
        raise ValueError("B/C shapes do not match x")
    if init is not None and init.shape != (bsz, H, N, P):
        raise ValueError("init_state shape must be [B,H,N,P]")
    y = np.empty_like(x)
    final = np.empty((bsz, H, N, P))
    bound = None
    if chunk_len > 0:
        nC = (T + chunk_len - 1) // chunk_len
        bound = np.empty((bsz, H, nC, N, P))
    d = dims_of(x, B)
    rc = lib.ssd_ref(ctypes.byref(d), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                     _ptr(init), int(chunk_len), _ptr(y), _ptr(final), _ptr(bound),
                     int(nthreads))
    if rc != 0:
        raise RuntimeError(f"ssd_ref failed with code {rc}")
    return y, final, bound


def ssd_bwd_ref(x, dt, A, B, C, D, dy, init_state=None, d_final=None, chunk_len=0,
                nthreads=0, lib=None):
    """Gradients of a scalar loss L through the recurrence, in fp64.

    Inputs as for ssd_ref, plus dy = dL/dy [B,T,H,P] and d_final = dL/d final_state
    [B,H,N,P] (None: zero).  Returns a dict with
      dx [B,T,H,P], ddt [B,T,H], dA [H], dB [B,T,G,N], dC [B,T,G,N], dD [H],
      d_init [B,H,N,P] (zeros-init gradient when init_state is None, still returned),
      dB_heads / dC_heads [B,T,H,N] (each head's share of dB / dC),
      boundary_grads [B,H,nC,N,P] or None (only when chunk_len > 0): for every chunk,
        dL/d(state after the chunk's last step) through the later steps only.
    A group's dB and dC are the sums of its heads' shares, dA and dD the sums over batch.
    """
    lib = lib or library()
    x, dt, A, B, C, D, dy = (_f64(v) for v in (x, dt, A, B, C, D, dy))
    init = None if init_state is None else _f64(init_state)
    dfin = None if d_final is None else _f64(d_final)
    bsz, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if dt.shape != (bsz, T, H) or A.shape != (H,) or D.shape != (H,):
        raise ValueError("dt/A/D shapes do not match x")
    if B.shape != (bsz, T, G, N) or C.shape != B.shape:
        raise ValueError("B/C shapes do not match x")
    if dy.shape != x.shape:
        raise ValueError("dy must have the shape of x")
    for name, v in (("init_state", init), ("d_final", dfin)):
        if v is not None and v.shape != (bsz, H, N, P):
            raise ValueError(f"{name} shape must be [B,H,N,P]")
    dx = np.empty_like(x)
    ddt = np.empty((bsz, T, H))
    dBh = np.empty((bsz, T, H, N))
    dCh = np.empty((bsz, T, H, N))
    dAp = np.empty((bsz, H))
    dDp = np.empty((bsz, H))
    d_init = np.empty((bsz, H, N, P))
    bgr = None
    if chunk_len > 0:
        bgr = np.empty((bsz, H, (T + chunk_len - 1) // chunk_len, N, P))
    d = dims_of(x, B)
    rc = lib.ssd_bwd_ref(ctypes.byref(d), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                         _ptr(init), _ptr(dy), _ptr(dfin), int(chunk_len), _ptr(dx), _ptr(ddt),
                         _ptr(dBh), _ptr(dCh), _ptr(dAp), _ptr(dDp), _ptr(d_init), _ptr(bgr),
                         int(nthreads))
    if rc != 0:
        raise RuntimeError(f"ssd_bwd_ref failed with code {rc}")
    hpg = H // G
    return dict(dx=dx, ddt=ddt, dA=dAp.sum(axis=0), dD=dDp.sum(axis=0),
                dB=dBh.reshape(bsz, T, G, hpg, N).sum(axis=3),
                dC=dCh.reshape(bsz, T, G, hpg, N).sum(axis=3),
                d_init=d_init, dB_heads=dBh, dC_heads=dCh, boundary_grads=bgr)


def threads_used(batch, nheads, nthreads=0):
    d = _Dims(batch, 1, nheads, 1, 1, 1)
    return library().ssd_ref_threads_used(ctypes.byref(d), int(nthreads))


def chunk_cumsum(dt, A, chunk_len):
    """Stage 0 and the log form of the 1-SS mask: for every chunk, the inclusive prefix
    sum of dt*A over the chunk's steps.  Returns cs [B,H,nC,Q]; positions past the end
    of a partial last chunk repeat the chunk's last value (no further decay)."""
    dt = _f64(dt)
    bsz, T, H = dt.shape
    Q = int(chunk_len)
    nC = (T + Q - 1) // Q
    dA = dt * _f64(A)[None, None, :]
    padded = np.zeros((bsz, nC * Q, H))
    padded[:, :T, :] = dA
    cs = np.cumsum(padded.reshape(bsz, nC, Q, H), axis=2)
    return np.ascontiguousarray(cs.transpose(0, 3, 1, 2))


def chunk_states(x, dt, A, B, C, D, chunk_len, nthreads=0):
    """Stage 2: the state at the end of every chunk when the chunk starts from zero
    state, i.e. the chunk's own inputs only.  Computed by running the recurrence on
    each chunk alone.  Returns [B,H,nC,N,P]."""
    x = _f64(x)
    bsz, T, H, P = x.shape
    N = np.asarray(B).shape[3]
    Q = int(chunk_len)
    nC = (T + Q - 1) // Q
    out = np.empty((bsz, H, nC, N, P))
    for c in range(nC):
        sl = slice(c * Q, min(T, (c + 1) * Q))
        _, fin, _ = ssd_ref(x[:, sl], _f64(dt)[:, sl], A, _f64(B)[:, sl], _f64(C)[:, sl], D,
                            nthreads=nthreads)
        out[:, :, c] = fin
    return out


def entry_states(x, dt, A, B, C, D, chunk_len, init_state=None, nthreads=0):
    """Stage 3 output as consumed by stage 4: the state entering every chunk (the
    init state for chunk 0, else the state after the previous chunk's last step).
    Returns ([B,H,nC,N,P], final_state [B,H,N,P])."""
    x = _f64(x)
    bsz, T, H, P = x.shape
    N = np.asarray(B).shape[3]
    _, final, bound = ssd_ref(x, dt, A, B, C, D, init_state=init_state, chunk_len=chunk_len,
                              nthreads=nthreads)
    ent = np.empty_like(bound)
    ent[:, :, 0] = 0.0 if init_state is None else _f64(init_state)
    ent[:, :, 1:] = bound[:, :, :-1]
    return ent, final


def chunk_entry_grads(x, dt, A, B, C, D, dy, chunk_len, init_state=None, nthreads=0):
    """For every chunk c, the gradient of L = <y, dy> with respect to the state entering
    chunk c through the outputs of chunk c alone (the later chunks' use of it excluded):
    the init-state gradient of a run over chunk c's steps, started from its true entry
    state, with dy restricted to the chunk and no final-state gradient.
    Returns [B,H,nC,N,P]."""
    x = _f64(x)
    bsz, T, H, P = x.shape
    N = np.asarray(B).shape[3]
    Q = int(chunk_len)
    nC = (T + Q - 1) // Q
    ent, _ = entry_states(x, dt, A, B, C, D, Q, init_state=init_state, nthreads=nthreads)
    out = np.empty((bsz, H, nC, N, P))
    dy = _f64(dy)
    for c in range(nC):
        sl = slice(c * Q, min(T, (c + 1) * Q))
        g = ssd_bwd_ref(x[:, sl], _f64(dt)[:, sl], A, _f64(B)[:, sl], _f64(C)[:, sl], D,
                        dy[:, sl], init_state=ent[:, :, c], nthreads=nthreads)
        out[:, :, c] = g["d_init"]
    return out
