"""ctypes binding for libssd.so (include/ssd.h), with the same entry point names.

Argument marshalling only: shapes are read off the tensors, output tensors are
allocated with torch when the caller passes none, and device pointers plus the current
HIP stream go to the C ABI.  Every step of the computation runs in libssd's kernels;
there is no fallback of any kind: if libssd.so is missing the first call raises.
"""
import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libssd.so")

SSD_F32, SSD_BF16 = 0, 1
_DTYPE_CODE = {torch.float32: SSD_F32, torch.bfloat16: SSD_BF16}
EXPORTED = ("ssd_status_string", "ssd_fwd_workspace_size", "ssd_fwd", "ssd_chunk_cumsum",
            "ssd_chunk_state", "ssd_state_passing", "ssd_chunk_gram_size", "ssd_chunk_gram",
            "ssd_chunk_scan", "ssd_decode_step", "ssd_bwd_workspace_size", "ssd_bwd",
            "ssd_block_prologue", "ssd_block_epilogue", "ssd_block_fwd_workspace_size",
            "ssd_block_fwd", "ssd_fwd_varlen_workspace_size", "ssd_fwd_varlen",
            "ssd_bwd_saved", "ssd_fwd_noalloc", "ssd_block_fwd_norm_in_scan")


class SsdDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("headdim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64)]

    def tuple(self):
        return (self.batch, self.seqlen, self.nheads, self.headdim, self.dstate, self.ngroups)


class SsdError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(msg)
        self.code = code


_LIB = None


def library(path=LIB_PATH):
    """Load libssd.so (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is not None and path == LIB_PATH:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m mamba_ssd_chunked_03_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    vp, fp, i, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    dims = ctypes.POINTER(SsdDims)
    lib.ssd_status_string.restype = ctypes.c_char_p
    lib.ssd_status_string.argtypes = [i]
    lib.ssd_fwd_workspace_size.restype = sz
    lib.ssd_fwd_workspace_size.argtypes = [dims, i]
    lib.ssd_fwd.restype = i
    lib.ssd_fwd.argtypes = [dims, i, vp, fp, fp, vp, vp, fp, i, fp, vp, fp, vp, sz, vp]
    lib.ssd_fwd_noalloc.restype = i
    lib.ssd_fwd_noalloc.argtypes = [dims, i, vp, fp, fp, vp, vp, fp, i, fp, vp, fp, vp]
    lib.ssd_chunk_cumsum.restype = i
    lib.ssd_chunk_cumsum.argtypes = [dims, i, fp, fp, fp, fp, vp]
    lib.ssd_chunk_state.restype = i
    lib.ssd_chunk_state.argtypes = [dims, i, i, vp, vp, fp, fp, fp, vp, vp, vp]
    lib.ssd_state_passing.restype = i
    lib.ssd_state_passing.argtypes = [dims, i, i, fp, fp, fp, vp, fp, vp]
    lib.ssd_chunk_gram_size.restype = sz
    lib.ssd_chunk_gram_size.argtypes = [dims, i, i]
    lib.ssd_chunk_gram.restype = i
    lib.ssd_chunk_gram.argtypes = [dims, i, i, vp, vp, vp, vp]
    lib.ssd_decode_step.restype = i
    lib.ssd_decode_step.argtypes = [dims, i, vp, fp, fp, vp, vp, fp, fp, vp, vp]
    lib.ssd_chunk_scan.restype = i
    lib.ssd_chunk_scan.argtypes = [dims, i, i, vp, vp, vp, fp, fp, fp, vp, vp, vp, vp]
    lib.ssd_bwd_workspace_size.restype = sz
    lib.ssd_bwd_workspace_size.argtypes = [dims, i]
    lib.ssd_bwd.restype = i
    lib.ssd_bwd.argtypes = [dims, i, vp, fp, fp, vp, vp, fp, i, fp, vp, fp, vp, fp, fp, vp, vp,
                            fp, fp, vp, sz, vp]
    i64, f = ctypes.c_int64, ctypes.c_float
    lib.ssd_block_prologue.restype = i
    lib.ssd_block_prologue.argtypes = [dims, i, vp, i64, fp, fp, i, vp, i64, fp, vp, vp, vp, fp,
                                       vp]
    lib.ssd_block_epilogue.restype = i
    lib.ssd_block_epilogue.argtypes = [dims, i, vp, vp, i64, fp, fp, i, i, f, vp, vp]
    lib.ssd_block_fwd_workspace_size.restype = sz
    lib.ssd_block_fwd_workspace_size.argtypes = [dims, i, i]
    lib.ssd_block_fwd_norm_in_scan.restype = i
    lib.ssd_block_fwd_norm_in_scan.argtypes = [dims, i, i, i]
    lib.ssd_block_fwd.restype = i
    lib.ssd_block_fwd.argtypes = [dims, i, vp, fp, fp, i, fp, fp, fp, i, fp, fp, fp, i, i, f, vp,
                                  fp, vp, sz, vp]
    lib.ssd_bwd_saved.restype = i
    lib.ssd_bwd_saved.argtypes = [dims, i, vp, fp, fp, vp, vp, fp, i, fp, vp, fp, vp, vp, fp, fp,
                                  vp, vp, fp, fp, vp, sz, vp]
    lib.ssd_fwd_varlen_workspace_size.restype = sz
    lib.ssd_fwd_varlen_workspace_size.argtypes = [dims, i]
    lib.ssd_fwd_varlen.restype = i
    lib.ssd_fwd_varlen.argtypes = [dims, i, vp, fp, fp, vp, vp, fp, i, vp, i64, vp, fp, vp, sz,
                                   vp]
    if path == LIB_PATH:
        _LIB = lib
    return lib


def status_string(code):
    return library().ssd_status_string(int(code)).decode()


def _check(code):
    if code != 0:
        raise SsdError(code, status_string(code))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def dims_of(x, B):
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError(f"x must be [B,T,H,P] and B [B,T,G,N], got {tuple(x.shape)} and "
                         f"{tuple(B.shape)}")
    b, t, h, p = x.shape
    if tuple(B.shape[:2]) != (b, t):
        raise ValueError(f"x and B must agree in batch and length: {tuple(x.shape)} and "
                         f"{tuple(B.shape)}")
    return SsdDims(b, t, h, p, B.shape[3], B.shape[2])


def nchunks(seqlen, chunk_len):
    return (seqlen + chunk_len - 1) // chunk_len


def _shape(t, name, shape):
    """t, when given, must have exactly this shape.  The C ABI receives bare pointers, so a
    tensor of any other size would be read or written past its end."""
    if t is not None and t.shape != shape:  # torch.Size compares equal to a tuple of ints
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _nbytes(t):
    return t.numel() * t.element_size()


def _out(t, name, dtype, device, shape):
    """A caller-provided output: dtype, device, contiguity and shape checked."""
    if t is not None:
        _need(t, name, dtype, device)
        _shape(t, name, shape)
    return t


def _layer_inputs(d, dt, A, C, D, init_state=None):
    """Shapes of the layer's other inputs against the dims read off x and B."""
    bz, T, H, P, N, G = d.tuple()
    _shape(C, "C", (bz, T, G, N))
    _shape(dt, "dt", (bz, T, H))
    _shape(A, "A", (H,))
    _shape(D, "D", (H,))
    _shape(init_state, "init_state", (bz, H, N, P))


def _stage_shapes(dims, chunk_len):
    bz, T, H, P, N, G = dims.tuple()
    nC = nchunks(T, chunk_len)
    return dict(x=(bz, T, H, P), bc=(bz, T, G, N), dt=(bz, T, H), head=(H,),
                chunk=(bz, H, nC, chunk_len), state=(bz, H, nC, P, N), final=(bz, H, N, P))


def _need(t, name, dtype=None, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def ssd_fwd_workspace_size(dims, chunk_len):
    return int(library().ssd_fwd_workspace_size(ctypes.byref(dims), int(chunk_len)))


def ssd_fwd(x, dt, A, B, C, D, chunk_len, init_state=None, y=None, final_state=None,
            workspace=None, want_final=True, stream=None):
    """y, final_state = SSD(x, dt, A, B, C, D) on the GPU through libssd.ssd_fwd.

    x [B,T,H,P] and B/C [B,T,G,N] in fp32 or bf16; dt [B,T,H], A [H], D [H] fp32;
    init_state [B,H,N,P] fp32 or None.  Returns (y, final_state or None)."""
    dev = x.device
    f32 = torch.float32
    _need(x, "x", device=dev)
    code = _DTYPE_CODE.get(x.dtype)
    if code is None:
        raise TypeError(f"x must be fp32 or bf16, got {x.dtype}")
    for t, n in ((B, "B"), (C, "C")):
        _need(t, n, x.dtype, dev)
    for t, n in ((dt, "dt"), (A, "A"), (D, "D")):
        _need(t, n, f32, dev)
    if init_state is not None:
        _need(init_state, "init_state", f32, dev)
    d = dims_of(x, B)
    _layer_inputs(d, dt, A, C, D, init_state)
    if y is None:
        y = torch.empty_like(x)
    _out(y, "y", x.dtype, dev, x.shape)
    fshape = (d.batch, d.nheads, d.dstate, d.headdim)
    if final_state is None and want_final:
        final_state = torch.empty(fshape, dtype=f32, device=dev)
    _out(final_state, "final_state", f32, dev, fshape)
    if workspace is None:
        ws = ssd_fwd_workspace_size(d, chunk_len)
        workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", device=dev)
    _check(library().ssd_fwd(ctypes.byref(d), code, _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                             _ptr(D), int(chunk_len), _ptr(init_state), _ptr(y),
                             _ptr(final_state), _ptr(workspace), _nbytes(workspace),
                             _stream(dev, stream)))
    return y, final_state


def ssd_fwd_noalloc(x, dt, A, B, C, D, chunk_len, init_state=None, y=None, final_state=None,
                    want_final=True, stream=None):
    """ssd_fwd with the stage buffers in the library's fixed device array (no workspace, no
    allocation inside the call; y and final_state are allocated here only when not given).
    Raises SsdError (SSD_ERR_WORKSPACE) when the problem does not fit the array."""
    dev = x.device
    f32 = torch.float32
    _need(x, "x", device=dev)
    code = _DTYPE_CODE.get(x.dtype)
    if code is None:
        raise TypeError(f"x must be fp32 or bf16, got {x.dtype}")
    for t, n in ((B, "B"), (C, "C")):
        _need(t, n, x.dtype, dev)
    for t, n in ((dt, "dt"), (A, "A"), (D, "D")):
        _need(t, n, f32, dev)
    if init_state is not None:
        _need(init_state, "init_state", f32, dev)
    d = dims_of(x, B)
    _layer_inputs(d, dt, A, C, D, init_state)
    if y is None:
        y = torch.empty_like(x)
    _out(y, "y", x.dtype, dev, x.shape)
    fshape = (d.batch, d.nheads, d.dstate, d.headdim)
    if final_state is None and want_final:
        final_state = torch.empty(fshape, dtype=f32, device=dev)
    _out(final_state, "final_state", f32, dev, fshape)
    _check(library().ssd_fwd_noalloc(ctypes.byref(d), code, _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                     _ptr(C), _ptr(D), int(chunk_len), _ptr(init_state), _ptr(y),
                                     _ptr(final_state), _stream(dev, stream)))
    return y, final_state


def fwd_stage_calls(x, dt, A, B, C, D, chunk_len, init_state, y, final_state, workspace,
                    stream=None):
    """The four stage calls ssd_fwd makes, on the stage buffers of its workspace laid out as
    ssd_fwd lays them: a list of (name, call) with every argument checked and marshalled
    once here, so that each call(), a C-ABI call and a status check, costs little host time
    (the benchmark records an event between stages).  Running the calls in order gives
    exactly ssd_fwd's y, final state and workspace contents."""
    dev = x.device
    f32 = torch.float32
    d = dims_of(x, B)
    code = _DTYPE_CODE.get(x.dtype)
    if code is None:
        raise TypeError(f"x must be fp32 or bf16, got {x.dtype}")
    for t, n in ((B, "B"), (C, "C")):
        _need(t, n, x.dtype, dev)
    for t, n in ((dt, "dt"), (A, "A"), (D, "D")):
        _need(t, n, f32, dev)
    _need(x, "x", device=dev)
    if init_state is not None:
        _need(init_state, "init_state", f32, dev)
    _layer_inputs(d, dt, A, C, D, init_state)
    _out(_need(y, "y", x.dtype, dev), "y", x.dtype, dev, x.shape)
    _out(final_state, "final_state", f32, dev, (d.batch, d.nheads, d.dstate, d.headdim))
    _need(workspace, "workspace", torch.uint8, dev)
    if _nbytes(workspace) < ssd_fwd_workspace_size(d, chunk_len):
        raise ValueError("workspace smaller than ssd_fwd_workspace_size")
    sh = _stage_shapes(d, chunk_len)
    nchunk = 1
    for v in sh["chunk"]:
        nchunk *= v
    nstate = 1
    for v in sh["state"]:
        nstate *= v
    rnd = lambda b: (b + 255) // 256 * 256
    base = workspace.data_ptr()
    offs = [0]
    for nb in (nchunk * 4, nchunk * 4, nstate * 4, nstate * 4):
        offs.append(offs[-1] + rnd(nb))
    gram_n = ssd_chunk_gram_size(d, x.dtype, chunk_len)
    dtc, cs, states, entry, gram = (ctypes.c_void_p(base + o) for o in offs)
    lib = library()
    st = _stream(dev, stream)
    q = int(chunk_len)
    dref = ctypes.byref(d)
    gp = gram if gram_n else None

    def call(fn, *args):
        def run():
            _check(fn(*args))
        run.dims = d  # keeps the dims alive with the call
        return run
    return [
        ("chunk_cumsum", call(lib.ssd_chunk_cumsum, dref, q, _ptr(dt), _ptr(A), dtc, cs, st)),
        ("chunk_state", call(lib.ssd_chunk_state, dref, code, q, _ptr(x), _ptr(B), dtc, cs,
                             states, _ptr(C) if gram_n else None, gp, st)),
        ("state_passing", call(lib.ssd_state_passing, dref, code, q, states, cs,
                               _ptr(init_state), entry, _ptr(final_state), st)),
        ("chunk_scan", call(lib.ssd_chunk_scan, dref, code, q, _ptr(x), _ptr(B), _ptr(C), dtc,
                            cs, _ptr(D), entry, gp, _ptr(y), st)),
    ]


def ssd_chunk_cumsum(dims, chunk_len, dt, A, dt_chunk=None, cs=None, stream=None):
    dev = dt.device
    sh = _stage_shapes(dims, chunk_len)
    f32 = torch.float32
    _shape(_need(dt, "dt", f32, dev), "dt", sh["dt"])
    _shape(_need(A, "A", f32, dev), "A", sh["head"])
    shape = sh["chunk"]
    dt_chunk = torch.empty(shape, dtype=f32, device=dev) if dt_chunk is None else dt_chunk
    cs = torch.empty(shape, dtype=f32, device=dev) if cs is None else cs
    _out(dt_chunk, "dt_chunk", f32, dev, shape)
    _out(cs, "cs", f32, dev, shape)
    _check(library().ssd_chunk_cumsum(ctypes.byref(dims), int(chunk_len), _ptr(dt), _ptr(A),
                                      _ptr(dt_chunk), _ptr(cs), _stream(dev, stream)))
    return dt_chunk, cs


def _state_shape(dims, chunk_len):
    return (dims.batch, dims.nheads, nchunks(dims.seqlen, chunk_len), dims.headdim, dims.dstate)


def ssd_chunk_state(dims, chunk_len, x, B, dt_chunk, cs, states=None, C=None, gram=None,
                    stream=None):
    """Chunk states; given C and a gram buffer (ssd_chunk_gram_size bytes) it also fills the
    C B^T blocks that ssd_chunk_scan reads, as ssd_chunk_gram would."""
    dev = x.device
    sh = _stage_shapes(dims, chunk_len)
    _shape(_need(x, "x", device=dev), "x", sh["x"])
    _shape(_need(B, "B", x.dtype, dev), "B", sh["bc"])
    for t, n in ((dt_chunk, "dt_chunk"), (cs, "cs")):
        _shape(_need(t, n, torch.float32, dev), n, sh["chunk"])
    if states is None:
        states = torch.empty(_state_shape(dims, chunk_len), dtype=x.dtype, device=dev)
    _out(states, "states", x.dtype, dev, sh["state"])
    if C is not None:
        _shape(_need(C, "C", x.dtype, dev), "C", sh["bc"])
    _gram_fits(dims, x.dtype, chunk_len, gram)
    gp = _ptr(gram) if gram is not None and gram.numel() else None
    _check(library().ssd_chunk_state(ctypes.byref(dims), _DTYPE_CODE[x.dtype], int(chunk_len),
                                     _ptr(x), _ptr(B), _ptr(dt_chunk), _ptr(cs), _ptr(states),
                                     _ptr(C), gp, _stream(dev, stream)))
    return states


def ssd_state_passing(dims, chunk_len, states, cs, init_state=None, entry_states=None,
                      final_state=None, want_final=True, stream=None):
    """Chunk states in, entry states out, both in the input dtype (fp32 or bf16);
    final_state is fp32."""
    dev = cs.device
    sh = _stage_shapes(dims, chunk_len)
    f32 = torch.float32
    _shape(_need(states, "states", device=dev), "states", sh["state"])
    _shape(_need(cs, "cs", f32, dev), "cs", sh["chunk"])
    if init_state is not None:
        _shape(_need(init_state, "init_state", f32, dev), "init_state", sh["final"])
    if entry_states is None:
        entry_states = torch.empty(_state_shape(dims, chunk_len), dtype=states.dtype, device=dev)
    if entry_states.dtype != states.dtype:
        raise TypeError("states and entry_states must have the same dtype")
    _out(entry_states, "entry_states", states.dtype, dev, sh["state"])
    if final_state is None and want_final:
        final_state = torch.empty(sh["final"], dtype=f32, device=dev)
    _out(final_state, "final_state", f32, dev, sh["final"])
    _check(library().ssd_state_passing(ctypes.byref(dims), _DTYPE_CODE[entry_states.dtype],
                                       int(chunk_len), _ptr(states), _ptr(cs), _ptr(init_state),
                                       _ptr(entry_states), _ptr(final_state),
                                       _stream(dev, stream)))
    return entry_states, final_state


def ssd_chunk_gram_size(dims, dtype, chunk_len):
    return int(library().ssd_chunk_gram_size(ctypes.byref(dims), _DTYPE_CODE[dtype],
                                             int(chunk_len)))


def _gram_fits(dims, dtype, chunk_len, gram):
    """A gram buffer, when given, holds at least ssd_chunk_gram_size bytes."""
    if gram is not None and gram.numel():
        _need(gram, "gram", device=gram.device)
        if _nbytes(gram) < ssd_chunk_gram_size(dims, dtype, chunk_len):
            raise ValueError(f"gram holds {_nbytes(gram)} bytes, "
                             f"{ssd_chunk_gram_size(dims, dtype, chunk_len)} needed")


def ssd_chunk_gram(dims, chunk_len, B, C, gram=None, stream=None):
    """The C B^T blocks ssd_chunk_scan reads (a uint8 buffer; empty where none is used)."""
    dev = B.device
    sh = _stage_shapes(dims, chunk_len)
    _shape(_need(B, "B", device=dev), "B", sh["bc"])
    _shape(_need(C, "C", B.dtype, dev), "C", sh["bc"])
    if gram is None:
        gram = torch.empty(ssd_chunk_gram_size(dims, B.dtype, chunk_len), dtype=torch.uint8,
                           device=dev)
    _gram_fits(dims, B.dtype, chunk_len, gram)
    _check(library().ssd_chunk_gram(ctypes.byref(dims), _DTYPE_CODE[B.dtype], int(chunk_len),
                                    _ptr(B), _ptr(C), _ptr(gram) if gram.numel() else None,
                                    _stream(dev, stream)))
    return gram


def ssd_chunk_scan(dims, chunk_len, x, B, C, dt_chunk, cs, D, entry_states, gram=None, y=None,
                   stream=None):
    """gram: the buffer ssd_chunk_gram filled from the same B and C (needed where
    ssd_chunk_gram_size is non-zero)."""
    dev = x.device
    sh = _stage_shapes(dims, chunk_len)
    f32 = torch.float32
    _shape(_need(x, "x", device=dev), "x", sh["x"])
    for t, n in ((B, "B"), (C, "C")):
        _shape(_need(t, n, x.dtype, dev), n, sh["bc"])
    for t, n in ((dt_chunk, "dt_chunk"), (cs, "cs")):
        _shape(_need(t, n, f32, dev), n, sh["chunk"])
    _shape(_need(D, "D", f32, dev), "D", sh["head"])
    _shape(_need(entry_states, "entry_states", x.dtype, dev), "entry_states", sh["state"])
    _gram_fits(dims, x.dtype, chunk_len, gram)
    y = torch.empty_like(x) if y is None else y
    _out(y, "y", x.dtype, dev, sh["x"])
    gp = _ptr(gram) if gram is not None and gram.numel() else None
    _check(library().ssd_chunk_scan(ctypes.byref(dims), _DTYPE_CODE[x.dtype], int(chunk_len),
                                    _ptr(x), _ptr(B), _ptr(C), _ptr(dt_chunk), _ptr(cs), _ptr(D),
                                    _ptr(entry_states), gp, _ptr(y), _stream(dev, stream)))
    return y


def ssd_decode_step(x, dt, A, B, C, D, state, y=None, stream=None):
    """One recurrent step: x [batch, nheads, headdim], dt [batch, nheads], B and C
    [batch, ngroups, dstate], state [batch, nheads, dstate, headdim] fp32 (updated in
    place).  Returns y [batch, nheads, headdim] in x's dtype."""
    dev = x.device
    code = _DTYPE_CODE.get(x.dtype)
    if code is None:
        raise TypeError(f"x must be fp32 or bf16, got {x.dtype}")
    if x.dim() != 3 or B.dim() != 3:
        raise ValueError(f"x must be [batch, nheads, headdim] and B [batch, ngroups, dstate], "
                         f"got {tuple(x.shape)} and {tuple(B.shape)}")
    bz, h, p = x.shape
    g, n = B.shape[1], B.shape[2]
    dims = SsdDims(bz, 1, h, p, n, g)
    f32 = torch.float32
    _need(x, "x", device=dev)
    for t, name in ((B, "B"), (C, "C")):
        _shape(_need(t, name, x.dtype, dev), name, (bz, g, n))
    _shape(_need(dt, "dt", f32, dev), "dt", (bz, h))
    for t, name in ((A, "A"), (D, "D")):
        _shape(_need(t, name, f32, dev), name, (h,))
    _shape(_need(state, "state", f32, dev), "state", (bz, h, n, p))
    y = torch.empty_like(x) if y is None else y
    _out(y, "y", x.dtype, dev, x.shape)
    _check(library().ssd_decode_step(ctypes.byref(dims), code, _ptr(x),
                                     _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(state),
                                     _ptr(y), _stream(dev, stream)))
    return y


def ssd_bwd_workspace_size(dims, chunk_len):
    return int(library().ssd_bwd_workspace_size(ctypes.byref(dims), int(chunk_len)))


def ssd_bwd(x, dt, A, B, C, D, chunk_len, dy, init_state=None, d_final=None, want_d_init=True,
            out=None, workspace=None, fwd_workspace=None, stream=None):
    """Gradients through ssd_fwd (libssd.ssd_bwd): inputs as for ssd_fwd plus dy (x's shape
    and dtype) and d_final ([B,H,N,P] fp32 or None).  Returns a dict with dx, ddt, dA, dB,
    dC, dD and d_init (None when want_d_init is False).  `out` may hold preallocated output
    tensors under those names.  With fwd_workspace (the workspace of an ssd_fwd call on the
    same inputs) it calls libssd.ssd_bwd_saved, which reads the forward's intermediates
    instead of recomputing them."""
    dev = x.device
    f32 = torch.float32
    _need(x, "x", device=dev)
    code = _DTYPE_CODE.get(x.dtype)
    if code is None:
        raise TypeError(f"x must be fp32 or bf16, got {x.dtype}")
    for t, n in ((B, "B"), (C, "C"), (dy, "dy")):
        _need(t, n, x.dtype, dev)
    for t, n in ((dt, "dt"), (A, "A"), (D, "D")):
        _need(t, n, f32, dev)
    for t, n in ((init_state, "init_state"), (d_final, "d_final")):
        if t is not None:
            _need(t, n, f32, dev)
    d = dims_of(x, B)
    _layer_inputs(d, dt, A, C, D, init_state)
    fshape = (d.batch, d.nheads, d.dstate, d.headdim)
    _shape(dy, "dy", x.shape)
    _shape(d_final, "d_final", fshape)
    o = dict(out or {})
    o.setdefault("dx", torch.empty_like(x))
    o.setdefault("ddt", torch.empty_like(dt))
    o.setdefault("dA", torch.empty_like(A))
    o.setdefault("dB", torch.empty_like(B))
    o.setdefault("dC", torch.empty_like(C))
    o.setdefault("dD", torch.empty_like(D))
    if want_d_init:
        o.setdefault("d_init", torch.empty(fshape, dtype=f32, device=dev))
    else:
        o["d_init"] = None
    for k, like in (("dx", x), ("ddt", dt), ("dA", A), ("dB", B), ("dC", C), ("dD", D)):
        _out(o[k], k, like.dtype, dev, like.shape)
    _out(o["d_init"], "d_init", f32, dev, fshape)
    if workspace is None:
        ws = ssd_bwd_workspace_size(d, chunk_len)
        workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", device=dev)
    if fwd_workspace is not None:
        _need(fwd_workspace, "fwd_workspace", torch.uint8, dev)
        # the library takes no size for it: it must be a whole ssd_fwd workspace
        if _nbytes(fwd_workspace) < ssd_fwd_workspace_size(d, chunk_len):
            raise ValueError(f"fwd_workspace holds {_nbytes(fwd_workspace)} bytes, an ssd_fwd "
                             f"workspace {ssd_fwd_workspace_size(d, chunk_len)}")
        _check(library().ssd_bwd_saved(
            ctypes.byref(d), code, _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
            int(chunk_len), _ptr(init_state), _ptr(dy), _ptr(d_final), _ptr(fwd_workspace),
            _ptr(o["dx"]), _ptr(o["ddt"]), _ptr(o["dA"]), _ptr(o["dB"]), _ptr(o["dC"]),
            _ptr(o["dD"]), _ptr(o["d_init"]), _ptr(workspace), _nbytes(workspace),
            _stream(dev, stream)))
        return o
    _check(library().ssd_bwd(ctypes.byref(d), code, _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                             _ptr(D), int(chunk_len), _ptr(init_state), _ptr(dy), _ptr(d_final),
                             _ptr(o["dx"]), _ptr(o["ddt"]), _ptr(o["dA"]), _ptr(o["dB"]),
                             _ptr(o["dC"]), _ptr(o["dD"]), _ptr(o["d_init"]), _ptr(workspace),
                             _nbytes(workspace), _stream(dev, stream)))
    return o


# ---------------------------------------------------------------- the block around the layer
def _row_stride(t, name, dtype=None, device=None):
    """Elements between consecutive [B*T] rows of a [B, T, width] view whose last dim is
    contiguous and whose rows are evenly spaced (a column range of a wider tensor)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dim() != 3 or (t.shape[2] > 1 and t.stride(2) != 1):
        raise ValueError(f"{name} must be [B, T, width] with contiguous rows")
    rs = t.stride(1)
    if t.shape[0] > 1 and t.stride(0) != t.shape[1] * rs:
        raise ValueError(f"{name}: rows must be evenly spaced over batch and time")
    return rs


def ssd_block_prologue(xbc, conv_w, conv_b, dt_raw, dt_bias, nheads, headdim, dstate, ngroups,
                       x=None, B=None, C=None, dt=None, stream=None):
    """x, B, C, dt = prologue(xbc, dt_raw) on the GPU through libssd.ssd_block_prologue.

    xbc [B, T, H*P + 2*G*N] and dt_raw [B, T, H] in fp32 or bf16 (views with evenly spaced
    rows, e.g. column ranges of the projection output); conv_w [H*P+2GN, K], conv_b, dt_bias
    fp32 (biases may be None)."""
    dev = xbc.device
    code = _DTYPE_CODE.get(xbc.dtype)
    if code is None:
        raise TypeError(f"xbc must be fp32 or bf16, got {xbc.dtype}")
    xs = _row_stride(xbc, "xbc", device=dev)
    ds = _row_stride(dt_raw, "dt_raw", xbc.dtype, dev)
    _need(conv_w, "conv_w", torch.float32, dev)
    for t, n in ((conv_b, "conv_b"), (dt_bias, "dt_bias")):
        if t is not None:
            _need(t, n, torch.float32, dev)
    bz, T = xbc.shape[0], xbc.shape[1]
    d = SsdDims(bz, T, nheads, headdim, dstate, ngroups)
    cd = nheads * headdim + 2 * ngroups * dstate
    _shape(xbc, "xbc", (bz, T, cd))
    _shape(dt_raw, "dt_raw", (bz, T, nheads))
    if conv_w.dim() != 2 or conv_w.shape[0] != cd:
        raise ValueError(f"conv_w must be [{cd}, K], got {tuple(conv_w.shape)}")
    _shape(conv_b, "conv_b", (cd,))
    _shape(dt_bias, "dt_bias", (nheads,))
    x = torch.empty((bz, T, nheads, headdim), dtype=xbc.dtype, device=dev) if x is None else x
    B = torch.empty((bz, T, ngroups, dstate), dtype=xbc.dtype, device=dev) if B is None else B
    C = torch.empty((bz, T, ngroups, dstate), dtype=xbc.dtype, device=dev) if C is None else C
    dt = torch.empty((bz, T, nheads), dtype=torch.float32, device=dev) if dt is None else dt
    _out(x, "x", xbc.dtype, dev, (bz, T, nheads, headdim))
    _out(B, "B", xbc.dtype, dev, (bz, T, ngroups, dstate))
    _out(C, "C", xbc.dtype, dev, (bz, T, ngroups, dstate))
    _out(dt, "dt", torch.float32, dev, (bz, T, nheads))
    _check(library().ssd_block_prologue(ctypes.byref(d), code, _ptr(xbc), xs, _ptr(conv_w),
                                        _ptr(conv_b), int(conv_w.shape[1]), _ptr(dt_raw), ds,
                                        _ptr(dt_bias), _ptr(x), _ptr(B), _ptr(C), _ptr(dt),
                                        _stream(dev, stream)))
    return dict(x=x, B=B, C=C, dt=dt)


def ssd_block_epilogue(y, z, norm_w, norm_b, norm_groups, rms=False, eps=1e-5, dstate=16,
                       ngroups=1, out=None, stream=None):
    """out = norm(y * silu(z)) per token on the GPU through libssd.ssd_block_epilogue.

    y [B, T, H, P] contiguous; z [B, T, H*P] (a view with evenly spaced rows); norm_w,
    norm_b [H*P] fp32 (norm_b may be None).  dstate and ngroups only complete the layer's
    sizes for validation.  Returns out [B, T, H*P]."""
    dev = y.device
    code = _DTYPE_CODE.get(y.dtype)
    if code is None:
        raise TypeError(f"y must be fp32 or bf16, got {y.dtype}")
    _need(y, "y", device=dev)
    zs = _row_stride(z, "z", y.dtype, dev)
    _need(norm_w, "norm_w", torch.float32, dev)
    if norm_b is not None:
        _need(norm_b, "norm_b", torch.float32, dev)
    if y.dim() != 4:
        raise ValueError(f"y must be [B, T, H, P], got {tuple(y.shape)}")
    bz, T, H, P = y.shape
    d = SsdDims(bz, T, H, P, dstate, ngroups)
    _shape(z, "z", (bz, T, H * P))
    _shape(norm_w, "norm_w", (H * P,))
    _shape(norm_b, "norm_b", (H * P,))
    if out is None:
        out = torch.empty((bz, T, H * P), dtype=y.dtype, device=dev)
    _out(out, "out", y.dtype, dev, (bz, T, H * P))
    _check(library().ssd_block_epilogue(ctypes.byref(d), code, _ptr(y), _ptr(z), zs,
                                        _ptr(norm_w), _ptr(norm_b), int(norm_groups),
                                        int(bool(rms)), float(eps), _ptr(out),
                                        _stream(dev, stream)))
    return out


def ssd_block_fwd_workspace_size(dims, dtype, chunk_len):
    return int(library().ssd_block_fwd_workspace_size(ctypes.byref(dims), int(dtype),
                                                      int(chunk_len)))


def ssd_block_fwd_norm_in_scan(dims, dtype, chunk_len, norm_groups):
    return bool(library().ssd_block_fwd_norm_in_scan(ctypes.byref(dims), int(dtype),
                                                     int(chunk_len), int(norm_groups)))


def ssd_block_fwd(zxbcdt, conv_w, conv_b, dt_bias, A, D, chunk_len, norm_w, norm_b,
                  norm_groups, headdim, dstate, ngroups, rms=False, eps=1e-5, init_state=None,
                  out=None, final_state=None, workspace=None, want_final=True, stream=None):
    """out, final_state = block(zxbcdt) on the GPU through libssd.ssd_block_fwd.

    zxbcdt [B, T, 2*H*P + 2*G*N + H] contiguous ([z | x | B | C | dt_raw] per token), H from
    A.  Returns (out [B, T, H*P], final_state [B, H, N, P] or None)."""
    dev = zxbcdt.device
    code = _DTYPE_CODE.get(zxbcdt.dtype)
    if code is None:
        raise TypeError(f"zxbcdt must be fp32 or bf16, got {zxbcdt.dtype}")
    _need(zxbcdt, "zxbcdt", device=dev)
    f32 = torch.float32
    for t, n in ((conv_w, "conv_w"), (A, "A"), (D, "D"), (norm_w, "norm_w")):
        _need(t, n, f32, dev)
    for t, n in ((conv_b, "conv_b"), (dt_bias, "dt_bias"), (norm_b, "norm_b"),
                 (init_state, "init_state")):
        if t is not None:
            _need(t, n, f32, dev)
    if A.dim() != 1 or zxbcdt.dim() != 3:
        raise ValueError("A must be [H] and zxbcdt [B, T, width]")
    H = A.shape[0]
    bz, T = zxbcdt.shape[0], zxbcdt.shape[1]
    if zxbcdt.shape[2] != 2 * H * headdim + 2 * ngroups * dstate + H:
        raise ValueError("zxbcdt width must be 2*H*P + 2*G*N + H")
    d = SsdDims(bz, T, H, headdim, dstate, ngroups)
    cd = H * headdim + 2 * ngroups * dstate
    if conv_w.dim() != 2 or conv_w.shape[0] != cd:
        raise ValueError(f"conv_w must be [{cd}, K], got {tuple(conv_w.shape)}")
    _shape(conv_b, "conv_b", (cd,))
    for t, n in ((dt_bias, "dt_bias"), (D, "D")):
        _shape(t, n, (H,))
    for t, n in ((norm_w, "norm_w"), (norm_b, "norm_b")):
        _shape(t, n, (H * headdim,))
    fshape = (bz, H, dstate, headdim)
    _shape(init_state, "init_state", fshape)
    if out is None:
        out = torch.empty((bz, T, H * headdim), dtype=zxbcdt.dtype, device=dev)
    _out(out, "out", zxbcdt.dtype, dev, (bz, T, H * headdim))
    if final_state is None and want_final:
        final_state = torch.empty(fshape, dtype=f32, device=dev)
    _out(final_state, "final_state", f32, dev, fshape)
    if workspace is None:
        ws = ssd_block_fwd_workspace_size(d, code, chunk_len)
        workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", device=dev)
    _check(library().ssd_block_fwd(ctypes.byref(d), code, _ptr(zxbcdt), _ptr(conv_w),
                                   _ptr(conv_b), int(conv_w.shape[1]), _ptr(dt_bias), _ptr(A),
                                   _ptr(D), int(chunk_len), _ptr(init_state), _ptr(norm_w),
                                   _ptr(norm_b), int(norm_groups), int(bool(rms)), float(eps),
                                   _ptr(out), _ptr(final_state), _ptr(workspace),
                                   _nbytes(workspace), _stream(dev, stream)))
    return out, final_state


# ---------------------------------------------------------------- packed variable-length rows
def ssd_fwd_varlen_workspace_size(dims, chunk_len):
    return int(library().ssd_fwd_varlen_workspace_size(ctypes.byref(dims), int(chunk_len)))


def ssd_fwd_varlen(x, dt, A, B, C, D, chunk_len, cu_seqlens, y=None, final_states=None,
                   want_final=True, workspace=None, check_cu_seqlens=True, stream=None):
    """y, final_states = SSD over a packed row through libssd.ssd_fwd_varlen.

    x [1,T,H,P], B/C [1,T,G,N] in fp32 or bf16; dt [1,T,H], A, D [H] fp32; cu_seqlens int32
    [nseq+1] on the device (0 .. T).  Returns (y, final_states [nseq,H,N,P] fp32 or None).
    The library takes the sequence starts as given; with check_cu_seqlens (the default) they
    are copied to the host first and checked to rise from 0 to T (which waits for the
    stream; a caller that has checked them once can pass False)."""
    dev = x.device
    code = _DTYPE_CODE.get(x.dtype)
    if code is None:
        raise TypeError(f"x must be fp32 or bf16, got {x.dtype}")
    _need(x, "x", device=dev)
    for t, n in ((B, "B"), (C, "C")):
        _need(t, n, x.dtype, dev)
    for t, n in ((dt, "dt"), (A, "A"), (D, "D")):
        _need(t, n, torch.float32, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    if cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be one-dimensional")
    nseq = cu_seqlens.numel() - 1
    d = dims_of(x, B)
    _layer_inputs(d, dt, A, C, D)
    if check_cu_seqlens and d.batch == 1:
        cu = cu_seqlens.cpu()
        if nseq < 0 or int(cu[0]) != 0 or int(cu[-1]) != d.seqlen or \
                bool((cu[1:] < cu[:-1]).any()):
            raise ValueError(f"cu_seqlens must rise from 0 to T = {d.seqlen}")
    if y is None:
        y = torch.empty_like(x)
    _out(y, "y", x.dtype, dev, x.shape)
    fshape = (max(nseq, 0), d.nheads, d.dstate, d.headdim)
    if final_states is None and want_final:
        final_states = torch.empty(fshape, dtype=torch.float32, device=dev)
    _out(final_states, "final_states", torch.float32, dev, fshape)
    if workspace is None:
        ws = ssd_fwd_varlen_workspace_size(d, chunk_len)
        workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", device=dev)
    _check(library().ssd_fwd_varlen(ctypes.byref(d), code, _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                    _ptr(C), _ptr(D), int(chunk_len), _ptr(cu_seqlens), nseq,
                                    _ptr(y), _ptr(final_states), _ptr(workspace),
                                    _nbytes(workspace), _stream(dev, stream)))
    return y, final_states
