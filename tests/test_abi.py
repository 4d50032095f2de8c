"""The C-ABI library builds, loads and exports what include/ssd.h declares (CPU only).

Only validation paths are called here: every call below fails its argument checks before
any HIP call, so no GPU is needed.
"""
import ctypes
import os
import re

import pytest
import torch

from mamba_ssd_chunked_03_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libssd.so is not built (run __graft_entry__.build())")
    return binding.library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(binding.EXPORTED)
    for name in names:
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {binding.LIB_PATH}").read()
    for name in names:
        assert re.search(rf"\bT {name}\b", out), f"{name} not exported as a function"


def test_status_strings(lib):
    for code in range(7):
        s = binding.status_string(code)
        assert s.startswith("SSD_")
    assert binding.status_string(99) == "SSD_ERR_UNKNOWN"


def D(b=1, t=256, h=2, p=16, n=16, g=1):
    return binding.SsdDims(b, t, h, p, n, g)


def test_workspace_size(lib):
    d = D(4, 4096, 80, 64, 128, 1)
    ws = binding.ssd_fwd_workspace_size(d, 256)
    nC = 16
    chunk = 4 * 80 * nC * 256 * 4
    state = 4 * 80 * nC * 64 * 128 * 4
    # C B^T blocks: per (batch, group, chunk) the 72 causal (16-row tile, 32-step block)
    # pairs of a 256-step chunk, 64 lanes x 16 bytes each
    pairs = sum(t // 2 + 1 for t in range(256 // 16))
    assert pairs == 72
    gram = 4 * 1 * nC * pairs * 64 * 16
    assert ws == 2 * chunk + 2 * state + gram
    assert binding.ssd_chunk_gram_size(d, torch.bfloat16, 256) == gram
    assert binding.ssd_chunk_gram_size(d, torch.float32, 256) == 0
    assert binding.ssd_chunk_gram_size(D(1, 1000, 4, 64, 128, 2), torch.bfloat16, 64) == \
        1 * 2 * 16 * sum(t // 2 + 1 for t in range(4)) * 1024
    # ragged T rounds the chunk count up
    assert binding.ssd_fwd_workspace_size(D(1, 1000, 4, 64, 128, 1), 256) == \
        2 * (4 * 4 * 256 * 4) + 2 * (4 * 4 * 64 * 128 * 4) + 4 * pairs * 1024
    assert binding.ssd_fwd_workspace_size(D(1, 0, 2, 16, 16, 1), 64) == 0
    for bad, q in ((D(h=3, g=2), 64), (D(p=24), 64), (D(n=48), 64), (D(), 32), (D(b=-1), 64)):
        assert binding.ssd_fwd_workspace_size(bad, q) == 0


def _fwd(lib, d, dtype=0, q=64, ptrs=None, ws_bytes=1 << 30):
    p = dict(x=16, dt=16, A=16, B=16, C=16, D=16, init=None, y=16, final=None, ws=16)
    p.update(ptrs or {})
    v = {k: (None if val is None else ctypes.c_void_p(val)) for k, val in p.items()}
    return lib.ssd_fwd(ctypes.byref(d), dtype, v["x"], v["dt"], v["A"], v["B"], v["C"], v["D"], q,
                       v["init"], v["y"], v["final"], v["ws"], ws_bytes, None)


def test_validation_errors_before_any_launch(lib):
    assert _fwd(lib, D(h=3, g=2)) == 2                     # H % G
    assert _fwd(lib, D(t=-5)) == 2
    assert _fwd(lib, D(p=0)) == 2
    assert _fwd(lib, D(p=48)) == 3                         # unsupported head dim
    assert _fwd(lib, D(n=512)) == 3
    assert _fwd(lib, D(), q=100) == 3                      # unsupported chunk
    assert _fwd(lib, D(), dtype=7) == 3
    assert _fwd(lib, D(), ptrs=dict(x=None)) == 1
    assert _fwd(lib, D(), ptrs=dict(C=None)) == 1
    assert _fwd(lib, D(), ptrs=dict(x=0x1008)) == 4        # 8-byte aligned only
    assert _fwd(lib, D(), ptrs=dict(dt=0x1002)) == 4
    assert _fwd(lib, D(), ptrs=dict(ws=None)) == 5
    assert _fwd(lib, D(), ws_bytes=10) == 5
    assert _fwd(lib, D(b=1 << 20, t=1 << 20)) == 2          # index range
    # products that overflow int64, and sizes of exactly 2^31, are refused as shapes before
    # any pointer or workspace check
    assert _fwd(lib, D(b=1 << 20, t=1 << 30, h=1 << 16, p=16, n=16, g=1 << 16)) == 2
    assert _fwd(lib, D(b=1 << 31, t=1 << 31, h=1, p=16, n=16, g=1)) == 2
    assert _fwd(lib, D(b=1 << 31, t=1, h=1, p=16, n=16, g=1)) == 2
    assert _fwd(lib, D(b=1, t=1 << 31, h=1, p=16, n=16, g=1)) == 2
    assert _fwd(lib, D(b=(1 << 62), t=4, h=1, p=16, n=16, g=1)) == 2
    assert binding.ssd_fwd_workspace_size(D(b=1 << 20, t=1 << 30, h=1 << 16, p=16, n=16,
                                            g=1 << 16), 64) == 0
    # stage entry points validate the same way
    assert lib.ssd_chunk_cumsum(ctypes.byref(D(p=40)), 64, None, None, None, None, None) == 3
    assert lib.ssd_chunk_cumsum(ctypes.byref(D()), 64, None, None, None, None, None) == 1
    assert lib.ssd_chunk_state(ctypes.byref(D()), 1, 64, None, None, None, None, None, None,
                               None, None) == 1
    # a gram buffer needs C (bf16, a shape with a matrix-core scan)
    ok5 = [ctypes.c_void_p(256)] * 5
    assert lib.ssd_chunk_state(ctypes.byref(D(p=64, n=64)), 1, 64, *ok5, None,
                               ctypes.c_void_p(256), None) == 1
    assert lib.ssd_chunk_state(ctypes.byref(D(p=64, n=64)), 1, 64, *ok5, ctypes.c_void_p(256),
                               ctypes.c_void_p(264), None) == 4
    assert lib.ssd_state_passing(ctypes.byref(D()), 0, 64, ctypes.c_void_p(64),
                                 ctypes.c_void_p(64), None, ctypes.c_void_p(64), None,
                                 None) == 2   # aliasing
    assert lib.ssd_state_passing(ctypes.byref(D()), 5, 64, ctypes.c_void_p(64),
                                 ctypes.c_void_p(64), None, ctypes.c_void_p(128), None,
                                 None) == 3   # dtype
    assert lib.ssd_chunk_scan(ctypes.byref(D()), 1, 128, None, None, None, None, None, None,
                              None, None, None, None) == 1
    # bf16 scan needs its gram buffer; fp32 ignores it
    ok = [ctypes.c_void_p(256)] * 7
    mf = D(p=64, n=64)   # a shape with a matrix-core scan
    assert lib.ssd_chunk_scan(ctypes.byref(mf), 1, 64, *ok, None, ctypes.c_void_p(256),
                              None) == 1
    assert lib.ssd_chunk_scan(ctypes.byref(mf), 1, 64, *ok, ctypes.c_void_p(264),
                              ctypes.c_void_p(256), None) == 4
    assert lib.ssd_chunk_gram(ctypes.byref(mf), 1, 64, None, None, None, None) == 1
    assert lib.ssd_chunk_gram(ctypes.byref(mf), 1, 64, ctypes.c_void_p(8), ctypes.c_void_p(256),
                              ctypes.c_void_p(256), None) == 4
    assert lib.ssd_chunk_gram(ctypes.byref(D(p=40)), 1, 64, None, None, None, None) == 3
    # no gram buffer for fp32, dstate 16 or an empty sequence: nothing to do
    assert lib.ssd_chunk_gram(ctypes.byref(mf), 0, 64, None, None, None, None) == 0
    assert lib.ssd_chunk_gram(ctypes.byref(D()), 1, 64, None, None, None, None) == 0
    assert lib.ssd_chunk_gram(ctypes.byref(D(t=0, p=64, n=64)), 1, 64, None, None, None,
                              None) == 0
    assert lib.ssd_fwd(None, 0, None, None, None, None, None, None, 64, None, None, None, None,
                       0, None) == 1
    # the decode step: sizes checked as for ssd_fwd (seqlen ignored), then pointers
    assert lib.ssd_decode_step(ctypes.byref(D(t=0)), 1, None, None, None, None, None, None,
                               None, None, None) == 1
    assert lib.ssd_decode_step(ctypes.byref(D(p=48)), 1, *[ctypes.c_void_p(256)] * 8,
                               None) == 3
    assert lib.ssd_decode_step(ctypes.byref(D(h=3, g=2)), 1, *[ctypes.c_void_p(256)] * 8,
                               None) == 2
    assert lib.ssd_decode_step(ctypes.byref(D(b=0)), 1, None, None, None, None, None, None,
                               None, None, None) == 0
    assert lib.ssd_decode_step(ctypes.byref(D()), 1, *[ctypes.c_void_p(264)] * 8, None) == 4
    assert lib.ssd_decode_step(None, 1, None, None, None, None, None, None, None, None,
                               None) == 1


def test_noalloc_refuses_oversize_before_any_launch(lib):
    """ssd_fwd_noalloc checks the problem against its fixed array before touching the GPU:
    the long-context shape needs 2 x 671 MB of bf16 entry states and chunk states."""
    def call(d, dtype=1, q=256):
        p = [ctypes.c_void_p(256)] * 6
        return lib.ssd_fwd_noalloc(ctypes.byref(d), dtype, *p, q, None, ctypes.c_void_p(256),
                                   None, None)
    assert call(D(1, 65536, 80, 64, 128, 8)) == 5
    assert call(D(0, 65536, 80, 64, 128, 8)) == 0  # batch 0: nothing to do
    assert call(D(1, 65536, 80, 64, 128, 8), dtype=7) == 3
    assert call(D(h=3, g=2), q=64) == 2
    assert lib.ssd_fwd_noalloc(ctypes.byref(D()), 0, None, None, None, None, None, None, 64, None,
                               None, None, None) == 1


def test_size_limit_is_exact(lib):
    """Every tensor must hold fewer than 2^31 elements, with T rounded up to whole chunks.
    At H = 80, P = 64, N = 256, Q = 256, 1638 chunks put both x and the chunk states at
    2,146,959,360 elements: accepted (the call goes on to fail on the workspace size, after
    the shape checks); one more step makes a 1639th chunk and is refused as a shape."""
    assert 1638 * 256 * 80 * 64 < 1 << 31 <= 1639 * 256 * 80 * 64
    assert _fwd(lib, D(1, 1638 * 256, 80, 64, 256, 1), dtype=1, q=256, ws_bytes=10) == 5
    assert _fwd(lib, D(1, 1638 * 256 - 100, 80, 64, 256, 1), dtype=1, q=256, ws_bytes=10) == 5
    assert _fwd(lib, D(1, 1638 * 256 + 1, 80, 64, 256, 1), dtype=1, q=256, ws_bytes=10) == 2
    # the chunk states alone at the limit (Q = 64: four times the elements of x)
    assert 6553 * 80 * 16 * 256 < 1 << 31 <= 6554 * 80 * 16 * 256
    assert _fwd(lib, D(1, 6553 * 64, 80, 16, 256, 1), dtype=1, q=64, ws_bytes=10) == 5
    assert _fwd(lib, D(1, 6553 * 64 + 1, 80, 16, 256, 1), dtype=1, q=64, ws_bytes=10) == 2


def test_bwd_workspace_size(lib):
    d = D(4, 4096, 80, 64, 128, 1)
    nC = 16
    chunk = 4 * 80 * nC * 256 * 4
    state = 4 * 80 * nC * 64 * 128 * 4
    tiles = 4 * 80 * nC * (256 // 16) * 4
    per_chunk = 4 * 80 * nC * 4
    # dt_chunk, cs, chunk states (reused for the entry-state gradients), entry states, exit
    # gradients, dL/dcs, the explicit dL/ddt, the cross-block pair sums (Q/64 planes), two
    # per-tile shares and dA's per-chunk share
    assert binding.ssd_bwd_workspace_size(d, 256) == \
        4 * chunk + 3 * state + (256 // 64) * chunk + 2 * tiles + per_chunk
    # dstate 256 (headdim 64): the carried-state terms of the matrix-core path as well, (F B_j)
    # per step and head in bf16 and the dB, dC head sums in fp32
    d = D(2, 8192, 32, 64, 256, 1)
    nC = 32
    chunk = 2 * 32 * nC * 256 * 4
    state = 2 * 32 * nC * 64 * 256 * 4
    tiles = 2 * 32 * nC * (256 // 16) * 4
    per_chunk = 2 * 32 * nC * 4
    carried = 2 * 8192 * 32 * 64 * 2 + 2 * (2 * 8192 * 1 * 256 * 4)
    assert binding.ssd_bwd_workspace_size(d, 256) == \
        4 * chunk + 3 * state + (256 // 64) * chunk + 2 * tiles + per_chunk + carried
    assert binding.ssd_bwd_workspace_size(D(h=3, g=2), 64) == 0
    assert binding.ssd_bwd_workspace_size(D(t=0), 64) == 0


def _bwd(lib, d, dtype=0, q=64, ptrs=None, ws_bytes=1 << 30):
    names = ("x", "dt", "A", "B", "C", "D", "init", "dy", "dfin", "dx", "ddt", "dA", "dB", "dC",
             "dD", "dinit", "ws")
    p = {k: 256 for k in names}
    p.update(init=None, dfin=None, dinit=None)
    p.update(ptrs or {})
    v = {k: (None if val is None else ctypes.c_void_p(val)) for k, val in p.items()}
    return lib.ssd_bwd(ctypes.byref(d), dtype, v["x"], v["dt"], v["A"], v["B"], v["C"], v["D"], q,
                       v["init"], v["dy"], v["dfin"], v["dx"], v["ddt"], v["dA"], v["dB"],
                       v["dC"], v["dD"], v["dinit"], v["ws"], ws_bytes, None)


def test_bwd_validation_errors_before_any_launch(lib):
    assert _bwd(lib, D(h=3, g=2)) == 2
    assert _bwd(lib, D(p=48)) == 3
    assert _bwd(lib, D(), q=32) == 3
    assert _bwd(lib, D(), dtype=3) == 3
    for k in ("x", "dt", "A", "B", "C", "D", "dy", "dx", "ddt", "dB", "dC"):
        assert _bwd(lib, D(), ptrs={k: None}) == 1, k
    # dA and dD are written even for an empty problem, so they are always required
    assert _bwd(lib, D(b=0), ptrs=dict(dA=None)) == 1
    assert _bwd(lib, D(t=0), ptrs=dict(dD=None)) == 1
    assert _bwd(lib, D(), ptrs=dict(dy=264)) == 4
    assert _bwd(lib, D(), ptrs=dict(dB=264)) == 4
    assert _bwd(lib, D(), ptrs=dict(ddt=258)) == 4
    assert _bwd(lib, D(), ptrs=dict(dfin=258)) == 4
    assert _bwd(lib, D(), ptrs=dict(ws=None)) == 5
    assert _bwd(lib, D(), ws_bytes=100) == 5
    assert lib.ssd_bwd(None, 0, *[None] * 6, 64, *[None] * 11, 0, None) == 1


def test_block_fwd_workspace_size(lib):
    d = D(4, 4096, 80, 64, 128, 1)
    bt = 4 * 4096

    def r(v):
        return (v + 255) // 256 * 256
    # x, y, B, C (bf16), then ssd_fwd's workspace (the step sizes are made inside the
    # cumsum pass and never stored)
    fwd = binding.ssd_fwd_workspace_size(d, 256)
    assert binding.ssd_block_fwd_workspace_size(d, binding.SSD_BF16, 256) == \
        2 * r(bt * 80 * 64 * 2) + 2 * r(bt * 128 * 2) + r(fwd)
    assert binding.ssd_block_fwd_workspace_size(d, binding.SSD_F32, 256) == \
        2 * r(bt * 80 * 64 * 4) + 2 * r(bt * 128 * 4) + r(fwd)
    assert binding.ssd_block_fwd_workspace_size(D(h=3, g=2), 0, 64) == 0
    assert binding.ssd_block_fwd_workspace_size(d, 9, 256) == 0


def test_block_validation_errors_before_any_launch(lib):
    ok = ctypes.c_void_p(256)
    dm = D(p=16, n=16, h=2)          # Cd = 2*16 + 2*16 = 64, width 2*32 + 32 + 2 = 98

    def pro(d=dm, dtype=1, xs=64, k=4, ds=2, **p):
        a = dict(xbc=ok, w=ok, b=None, dt=ok, bias=None, x=ok, B=ok, C=ok, dto=ok)
        a.update({n: (None if v is None else ctypes.c_void_p(v)) for n, v in p.items()})
        return lib.ssd_block_prologue(ctypes.byref(d), dtype, a["xbc"], xs, a["w"], a["b"], k,
                                      a["dt"], ds, a["bias"], a["x"], a["B"], a["C"], a["dto"],
                                      None)
    assert pro(k=0) == 3 and pro(k=9) == 3 and pro(dtype=4) == 3
    assert pro(xs=63) == 2 and pro(ds=1) == 2
    assert pro(xbc=None) == 1 and pro(dto=None) == 1
    assert pro(x=264) == 4 and pro(dto=258) == 4 and pro(xbc=257) == 4   # element alignment
    assert pro(d=D(b=0)) == 0 and pro(d=D(t=0), xbc=None) == 0            # nothing to do
    assert pro(d=D(h=3, g=2)) == 2

    def epi(d=dm, dtype=1, zs=32, groups=1, rms=0, eps=1e-5, **p):
        a = dict(y=ok, z=ok, w=ok, b=None, out=ok)
        a.update({n: (None if v is None else ctypes.c_void_p(v)) for n, v in p.items()})
        return lib.ssd_block_epilogue(ctypes.byref(d), dtype, a["y"], a["z"], zs, a["w"], a["b"],
                                      groups, rms, ctypes.c_float(eps), a["out"], None)
    assert epi(groups=0) == 2 and epi(groups=3) == 2 and epi(zs=31) == 2
    assert epi(eps=-1.0) == 2 and epi(eps=float("nan")) == 2
    assert epi(y=None) == 1 and epi(w=None) == 1
    assert epi(out=264) == 4 and epi(z=257) == 4 and epi(w=258) == 4
    assert epi(d=D(t=0), y=None) == 0

    def blk(d=dm, dtype=1, k=4, q=64, groups=1, ws_bytes=1 << 30, **p):
        a = dict(zx=ok, w=ok, A=ok, Dp=ok, nw=ok, out=ok, ws=ok)
        a.update({n: (None if v is None else ctypes.c_void_p(v)) for n, v in p.items()})
        return lib.ssd_block_fwd(ctypes.byref(d), dtype, a["zx"], a["w"], None, k, None, a["A"],
                                 a["Dp"], q, None, a["nw"], None, groups, 0,
                                 ctypes.c_float(1e-5), a["out"], None, a["ws"], ws_bytes, None)
    assert blk(k=0) == 3 and blk(q=100) == 3 and blk(groups=5) == 2
    assert blk(zx=None) == 1 and blk(A=None) == 1
    assert blk(zx=264) == 4 and blk(ws=None) == 5 and blk(ws_bytes=100) == 5


def test_varlen_validation_errors_before_any_launch(lib):
    ok = ctypes.c_void_p(256)

    def call(d, dtype=1, q=64, nseq=2, ws_bytes=1 << 30, **p):
        a = dict(x=ok, dt=ok, A=ok, B=ok, C=ok, D=ok, cu=ok, y=ok, fin=None, ws=ok)
        a.update({n: (None if v is None else ctypes.c_void_p(v)) for n, v in p.items()})
        return lib.ssd_fwd_varlen(ctypes.byref(d), dtype, a["x"], a["dt"], a["A"], a["B"],
                                  a["C"], a["D"], q, a["cu"], nseq, a["y"], a["fin"], a["ws"],
                                  ws_bytes, None)
    assert call(D(b=2)) == 2 and call(D(), nseq=0) == 2          # batch 1, nseq >= 1
    assert call(D(), q=100) == 3 and call(D(), dtype=9) == 3
    assert call(D(), cu=None) == 1 and call(D(), x=None) == 1
    assert call(D(), cu=258) == 4 and call(D(), x=264) == 4
    assert call(D(), ws=None) == 5 and call(D(), ws_bytes=16) == 5
    d = D()
    assert binding.ssd_fwd_varlen_workspace_size(d, 64) == binding.ssd_fwd_workspace_size(d, 64)
    assert binding.ssd_fwd_varlen_workspace_size(D(b=2), 64) == 0


def test_bwd_saved_needs_the_forward_workspace(lib):
    ok = [ctypes.c_void_p(256)] * 6
    # fwd_workspace NULL is an error before anything else is read
    assert lib.ssd_bwd_saved(ctypes.byref(D()), 1, *ok, 64, None, ctypes.c_void_p(256), None,
                             None, *[ctypes.c_void_p(256)] * 7, ctypes.c_void_p(256), 1 << 30,
                             None) == 1
    assert lib.ssd_bwd_saved(ctypes.byref(D()), 1, *ok, 64, None, ctypes.c_void_p(256), None,
                             ctypes.c_void_p(264), *[ctypes.c_void_p(256)] * 7,
                             ctypes.c_void_p(256), 1 << 30, None) == 4


def test_block_norm_in_scan_query(lib):
    """ssd_block_fwd_norm_in_scan: the gate and the norm run in the chunk scan exactly where
    every norm group lies inside one head (S = H P / norm_groups a multiple of 16 dividing
    P), in bf16, at head sizes 32 and 64; answered from the sizes alone (no GPU here)."""
    q = binding.ssd_block_fwd_norm_in_scan
    bf, f32 = binding.SSD_BF16, binding.SSD_F32
    d = D(4, 4096, 80, 64, 128, 1)
    assert q(d, bf, 256, 80)            # S = 64 = P: one group per head
    assert q(d, bf, 256, 160)           # S = 32: two per head
    assert q(d, bf, 256, 320)           # S = 16: four per head
    assert not q(d, bf, 256, 640)       # S = 8: below a 16-channel p-tile
    assert not q(d, bf, 256, 1)         # one group over all heads (the model default)
    assert not q(d, bf, 256, 40)        # S = 128: a group spans two heads
    assert not q(d, bf, 256, 3)         # does not divide H P
    assert not q(d, f32, 256, 80)       # fp32 takes the VALU scan
    assert q(D(2, 200, 4, 32, 128, 1), bf, 64, 8)       # P = 32, S = 16
    assert not q(D(2, 200, 4, 16, 128, 1), bf, 64, 4)   # P = 16 has no gated scan
    assert not q(D(1, 256, 3, 64, 16, 1), bf, 64, 3)    # rows of 2*192 + 32 + 3 bf16: not 8 B
    assert not q(D(h=3, g=2), bf, 64, 3)                # invalid sizes
    assert not q(d, bf, 100, 80)                        # unsupported chunk length
    assert not q(d, 9, 256, 80)                         # unknown dtype
    # 64 rows of z span 2^31 bytes or more: the scan's 32-bit offsets would not reach them
    big = D(1, 64, 1 << 17, 64, 128, 1)                 # H P = 2^23: rows of over 2^25 bytes
    assert not q(big, bf, 64, 1 << 17)
