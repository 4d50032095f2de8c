"""The Python binding refuses tensors whose shapes do not match the layer's sizes (CPU only).

The C ABI receives bare pointers and sizes, so a buffer of the wrong size would be read or
written past its end on the GPU.  The binding checks every tensor's shape, dtype, device
and layout against the dims it reads off x and B, and refuses a mismatch before any call
into libssd.  Every call below fails that check, so no GPU is needed.
"""
import pytest
import torch

from mamba_ssd_chunked_03_amd import binding

BZ, T, H, P, N, G, Q = 2, 100, 4, 16, 32, 2, 64
f32, bf16 = torch.float32, torch.bfloat16


@pytest.fixture(scope="module", autouse=True)
def lib():
    return binding.library()


def layer(dtype=bf16):
    return dict(x=torch.zeros(BZ, T, H, P, dtype=dtype), dt=torch.zeros(BZ, T, H),
                A=torch.zeros(H), B=torch.zeros(BZ, T, G, N, dtype=dtype),
                C=torch.zeros(BZ, T, G, N, dtype=dtype), D=torch.zeros(H))


def fwd(**over):
    a = layer()
    kw = {k: over.pop(k) for k in list(over) if k not in a}
    a.update(over)
    return binding.ssd_fwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], Q, **kw)


@pytest.mark.parametrize("name,bad", [
    ("B", torch.zeros(BZ, T + 1, G, N, dtype=bf16)),      # another length
    ("C", torch.zeros(BZ, T, G, N + 16, dtype=bf16)),
    ("dt", torch.zeros(BZ, T, H + 1)),
    ("A", torch.zeros(H + 1)),
    ("D", torch.zeros(1)),
    ("x", torch.zeros(BZ, T, H * P, dtype=bf16)),         # not 4-D
])
def test_fwd_refuses_mismatched_inputs(name, bad):
    with pytest.raises(ValueError):
        fwd(**{name: bad})


def test_fwd_refuses_mismatched_outputs():
    with pytest.raises(ValueError, match="y"):
        fwd(y=torch.zeros(BZ, T - 1, H, P, dtype=bf16))
    with pytest.raises(TypeError, match="y"):
        fwd(y=torch.zeros(BZ, T, H, P, dtype=f32))
    with pytest.raises(ValueError, match="final_state"):
        fwd(final_state=torch.zeros(BZ, H, P, N))         # [N][P] transposed
    with pytest.raises(ValueError, match="init_state"):
        fwd(init_state=torch.zeros(BZ, H, N, P + 1))
    with pytest.raises(ValueError, match="contiguous"):
        fwd(y=torch.zeros(BZ, T, P, H, dtype=bf16).transpose(2, 3))


def test_bwd_refuses_mismatched_tensors():
    a = layer()
    args = (a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], Q)
    dy = torch.zeros(BZ, T, H, P, dtype=bf16)
    with pytest.raises(ValueError, match="dy"):
        binding.ssd_bwd(*args, torch.zeros(BZ, T, H, P // 2, dtype=bf16))
    with pytest.raises(ValueError, match="d_final"):
        binding.ssd_bwd(*args, dy, d_final=torch.zeros(BZ, H, N))
    with pytest.raises(ValueError, match="dB"):
        binding.ssd_bwd(*args, dy, out=dict(dB=torch.zeros(BZ, T, G, N - 1, dtype=bf16)))
    with pytest.raises(TypeError, match="ddt"):
        binding.ssd_bwd(*args, dy, out=dict(ddt=torch.zeros(BZ, T, H, dtype=bf16)))
    # the forward's workspace is passed without a size: it must be a whole one
    with pytest.raises(ValueError, match="fwd_workspace"):
        binding.ssd_bwd(*args, dy, fwd_workspace=torch.zeros(64, dtype=torch.uint8))


def test_stage_calls_refuse_mismatched_tensors():
    a = layer()
    dims = binding.dims_of(a["x"], a["B"])
    nC = binding.nchunks(T, Q)
    with pytest.raises(ValueError, match="dt"):
        binding.ssd_chunk_cumsum(dims, Q, torch.zeros(BZ, T, H + 1), a["A"])
    with pytest.raises(ValueError, match="cs"):
        binding.ssd_chunk_cumsum(dims, Q, a["dt"], a["A"], cs=torch.zeros(BZ, H, nC + 1, Q))
    chunk = torch.zeros(BZ, H, nC, Q)
    with pytest.raises(ValueError, match="states"):
        binding.ssd_chunk_state(dims, Q, a["x"], a["B"], chunk, chunk,
                                states=torch.zeros(BZ, H, nC, N, P, dtype=bf16))
    with pytest.raises(ValueError, match="entry_states"):
        binding.ssd_chunk_scan(dims, Q, a["x"], a["B"], a["C"], chunk, chunk, a["D"],
                               torch.zeros(BZ, H, nC - 1, P, N, dtype=bf16))
    ent = torch.zeros(BZ, H, nC, P, N, dtype=bf16)
    with pytest.raises(ValueError, match="gram"):
        binding.ssd_chunk_scan(dims, Q, a["x"], a["B"], a["C"], chunk, chunk, a["D"], ent,
                               gram=torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="final_state"):
        binding.ssd_state_passing(dims, Q, ent, chunk, final_state=torch.zeros(BZ, H, N))


def test_decode_refuses_mismatched_tensors():
    x = torch.zeros(BZ, H, P, dtype=bf16)
    Bm = torch.zeros(BZ, G, N, dtype=bf16)
    state = torch.zeros(BZ, H, N, P)
    dt, A, D = torch.zeros(BZ, H), torch.zeros(H), torch.zeros(H)
    with pytest.raises(ValueError, match="state"):
        binding.ssd_decode_step(x, dt, A, Bm, Bm, D, torch.zeros(BZ, H, P, N + 1))
    with pytest.raises(TypeError, match="dt"):
        binding.ssd_decode_step(x, dt.to(bf16), A, Bm, Bm, D, state)
    with pytest.raises(ValueError, match="C"):
        binding.ssd_decode_step(x, dt, A, Bm, torch.zeros(BZ, G + 1, N, dtype=bf16), D, state)


def test_varlen_checks_sequence_starts():
    a = {k: v[:1] if v.dim() > 1 else v for k, v in layer().items()}
    args = (a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], Q)
    for cu in ([0, 60, 40, T], [0, 50, T - 1], [5, 50, T], [0, 50, T + 1]):
        with pytest.raises(ValueError, match="cu_seqlens"):
            binding.ssd_fwd_varlen(*args, torch.tensor(cu, dtype=torch.int32))
    cu = torch.tensor([0, 50, T], dtype=torch.int32)
    with pytest.raises(ValueError, match="final_states"):
        binding.ssd_fwd_varlen(*args, cu, final_states=torch.zeros(3, H, N, P))


def test_block_calls_refuse_mismatched_tensors():
    cd = H * P + 2 * G * N
    zx = torch.zeros(BZ, T, 2 * H * P + 2 * G * N + H, dtype=bf16)
    xbc, dt_raw = zx[:, :, H * P:H * P + cd], zx[:, :, H * P + cd:]
    w = torch.zeros(cd, 4)
    with pytest.raises(ValueError, match="xbc"):
        binding.ssd_block_prologue(zx[:, :, :cd - 8], w, None, dt_raw, None, H, P, N, G)
    with pytest.raises(ValueError, match="conv_w"):
        binding.ssd_block_prologue(xbc, torch.zeros(cd - 1, 4), None, dt_raw, None, H, P, N, G)
    with pytest.raises(ValueError, match="dt_bias"):
        binding.ssd_block_prologue(xbc, w, None, dt_raw, torch.zeros(H + 1), H, P, N, G)
    y = torch.zeros(BZ, T, H, P, dtype=bf16)
    with pytest.raises(ValueError, match="norm_w"):
        binding.ssd_block_epilogue(y, zx[:, :, :H * P], torch.zeros(H * P - 1), None, 1)
    A, D = torch.zeros(H), torch.zeros(H)
    with pytest.raises(ValueError, match="norm_b"):
        binding.ssd_block_fwd(zx, w, None, None, A, D, Q, torch.zeros(H * P),
                              torch.zeros(H), 1, P, N, G)
    with pytest.raises(ValueError, match="out"):
        binding.ssd_block_fwd(zx, w, None, None, A, D, Q, torch.zeros(H * P), None, 1, P, N, G,
                              out=torch.zeros(BZ, T, H * P + 1, dtype=bf16))
