"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on the GPU.

Whole-tensor rel-L2 against the oracle on small cases (several chunks and ragged tails);
at the full model-shaped sizes and at the size limit, every (batch, head) sequence is
checked against the oracle, each on its own as well as the whole tensor.  Per-stage tests feed each
kernel oracle-made inputs so that a mistake is pinned to its stage.
"""
import numpy as np
import pytest
import torch

import oracle
from mamba_ssd_chunked_03_amd import binding
from mamba_ssd_chunked_03_amd.workloads import (LONG_CTX, MAMBA2_130M, MAMBA2_2P7B, NSWEEP, STRESS,
                                                TINY_FP32, Workload, generate, variants)
from parity import (TOL, assert_every_sequence, check_every_sequence, gpu_fwd, np64, oracle_fwd,
                    rel_l2, say, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    binding.library()
    torch.cuda.init()
    return torch.device("cuda:0")


SMALL = [TINY_FP32] + list(STRESS.values())


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_fwd_matches_oracle_small(w):
    say(f"[fwd small] {w.describe()}")
    cpu = generate(w)
    y, fin = gpu_fwd(to_device(cpu), w.chunk_len)
    y_ref, f_ref = oracle_fwd(cpu)
    ey, ef = rel_l2(np64(y), y_ref), rel_l2(np64(fin), f_ref)
    say(f"    rel_l2 y={ey:.3e} final={ef:.3e}")
    assert ey <= TOL[w.dtype]
    assert ef <= TOL[w.dtype]


MODEL = [MAMBA2_130M, MAMBA2_2P7B, *NSWEEP, LONG_CTX]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("w", MODEL, ids=[w.name for w in MODEL])
def test_fwd_matches_oracle_full_size(w):
    """Every (b, h) sequence of the model-shaped workloads, at full size in the launch
    configuration the bench times, against the oracle: the whole tensor and each
    sequence on its own within the bound (a single wrong tile shows in its sequence)."""
    say(f"[fwd full size] {w.describe()}")
    cpu = generate(w)
    y, fin = gpu_fwd(to_device(cpu), w.chunk_len)
    assert torch.isfinite(y.float()).all()
    assert_every_sequence(w, check_every_sequence(w, cpu, y, fin))


@pytest.mark.timeout(300)
@pytest.mark.parametrize("q", [64, 128], ids=["Q64", "Q128"])
def test_fwd_130m_shape_at_other_chunk_lengths(q):
    """The 130M-shaped layer at chunk lengths 64 and 128 (256 is the workload itself):
    the chunk length is the block decomposition's tunable block size and leaves the result
    unchanged, so every sequence must still match the oracle."""
    w = variants(MAMBA2_130M, name=f"mamba2_130m_q{q}", chunk_len=q)
    say(f"[fwd chunk length] {w.describe()}")
    cpu = generate(w)
    y, fin = gpu_fwd(to_device(cpu), w.chunk_len)
    assert_every_sequence(w, check_every_sequence(w, cpu, y, fin))


# The largest shapes the library accepts: tensors just under 2^31 elements (T rounded up to
# whole chunks), each with a ragged last chunk.  A 32-bit overflow of an element or byte
# offset anywhere on the path would show here.  The first puts x, y and the chunk states
# at the limit (4.3 GB each in bf16); the second the chunk states alone (Q = 64, N = 256:
# four times the elements of x).  Both shapes also run at small sizes below.
LIMIT = [
    Workload("limit_x_and_states", 1, 1638 * 256 - 100, 80, 64, 256, 1, 256, init_state=True),
    Workload("limit_states", 1, 819 * 64 - 37, 80, 128, 256, 1, 64, init_state=True),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("w", LIMIT, ids=[w.name for w in LIMIT])
def test_fwd_at_the_size_limit(w):
    say(f"[fwd size limit] {w.describe()}")
    padded = w.nchunks * w.chunk_len
    assert padded * w.nheads * w.headdim < 1 << 31
    assert w.nchunks * w.nheads * w.headdim * w.dstate < 1 << 31
    assert max(padded * w.nheads * w.headdim,
               w.nchunks * w.nheads * w.headdim * w.dstate) > 0.99 * (1 << 31)
    cpu = generate(w)
    y, fin = gpu_fwd(to_device(cpu), w.chunk_len)
    assert torch.isfinite(y).all()
    assert_every_sequence(w, check_every_sequence(w, cpu, y, fin))


def test_tiny_fp32_whole_output():
    """The fp32 workload compared on every output, at the fp32 bound."""
    w = TINY_FP32
    cpu = generate(w)
    y, fin = gpu_fwd(to_device(cpu), w.chunk_len)
    y_ref, f_ref = oracle_fwd(cpu)
    assert rel_l2(np64(y), y_ref) <= 1e-4
    assert rel_l2(np64(fin), f_ref) <= 1e-4
    # element-wise: no single output is far off either
    err = np.abs(np64(y) - y_ref).max() / np.abs(y_ref).max()
    assert err < 1e-4


# ------------------------------------------------------------------ stage by stage

STAGE_CASES = [STRESS["slow_decay_fp32"], STRESS["slow_decay"], STRESS["ragged_250_q64"],
               STRESS["ragged_1000"]]


def _dims(w):
    return binding.SsdDims(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups)


@pytest.mark.parametrize("w", STAGE_CASES, ids=[w.name for w in STAGE_CASES])
def test_stage_chunk_cumsum(w):
    say(f"[stage cumsum] {w.describe()}")
    cpu = generate(w)
    dv = to_device(cpu)
    dtc, cs = binding.ssd_chunk_cumsum(_dims(w), w.chunk_len, dv["dt"], dv["A"])
    torch.cuda.synchronize()
    ref = oracle.chunk_cumsum(np64(cpu["dt"]), np64(cpu["A"]), w.chunk_len)
    # dt copied exactly; zero past the end of the sequence
    Q, T = w.chunk_len, w.seqlen
    dt_pad = np.zeros((w.batch, w.nchunks * Q, w.nheads))
    dt_pad[:, :T] = np64(cpu["dt"])
    dt_ref = dt_pad.reshape(w.batch, w.nchunks, Q, w.nheads).transpose(0, 3, 1, 2)
    np.testing.assert_array_equal(np64(dtc), dt_ref)
    # fp32 prefix sums: error relative to the running sum of |dt*A| (all terms share a sign)
    mag = np.abs(ref).max()
    assert np.abs(np64(cs) - ref).max() <= 2e-6 * max(mag, 1e-30)


@pytest.mark.parametrize("w", STAGE_CASES, ids=[w.name for w in STAGE_CASES])
def test_stage_chunk_state(w):
    say(f"[stage chunk_state] {w.describe()}")
    cpu = generate(w)
    dv = to_device(cpu)
    d = _dims(w)
    dtc, cs = binding.ssd_chunk_cumsum(d, w.chunk_len, dv["dt"], dv["A"])
    S = binding.ssd_chunk_state(d, w.chunk_len, dv["x"], dv["B"], dtc, cs)
    torch.cuda.synchronize()
    c = {k: np64(v) for k, v in cpu.items()}
    ref = oracle.chunk_states(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], w.chunk_len)
    e = rel_l2(np64(S).swapaxes(-1, -2), ref)
    say(f"    rel_l2 S={e:.3e}")
    assert e <= (1e-5 if w.dtype == "fp32" else TOL[w.dtype])


@pytest.mark.parametrize("w", STAGE_CASES, ids=[w.name for w in STAGE_CASES])
def test_stage_state_passing(w):
    """Fed the oracle's chunk states and log decays (rounded to fp32), the scan must give
    the oracle's entry states and final state."""
    say(f"[stage state_passing] {w.describe()}")
    cpu = generate(w)
    c = {k: np64(v) for k, v in cpu.items()}
    S = oracle.chunk_states(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], w.chunk_len)
    cs = oracle.chunk_cumsum(c["dt"], c["A"], w.chunk_len)
    ent_ref, fin_ref = oracle.entry_states(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"],
                                           w.chunk_len, init_state=c["init_state"])
    dev = "cuda"
    # chunk states are stored in the input dtype
    S_d = torch.from_numpy(S.swapaxes(-1, -2).copy()).float().to(cpu["x"].dtype).to(dev)
    cs_d = torch.from_numpy(cs).float().to(dev)
    init = None if cpu["init_state"] is None else cpu["init_state"].to(dev)
    ent, fin = binding.ssd_state_passing(_dims(w), w.chunk_len, S_d, cs_d, init_state=init)
    torch.cuda.synchronize()
    e1 = rel_l2(np64(ent).swapaxes(-1, -2), ent_ref)
    e2 = rel_l2(np64(fin), fin_ref)
    say(f"    rel_l2 entry={e1:.3e} final={e2:.3e}")
    # carried in fp32; chunk states in and entry states out in the input dtype (with bf16,
    # one rounding of each chunk state and one of each entry state)
    assert e1 <= (1e-5 if w.dtype == "fp32" else 6e-3)
    assert e2 <= (1e-5 if w.dtype == "fp32" else 4e-3)


@pytest.mark.parametrize("w", STAGE_CASES, ids=[w.name for w in STAGE_CASES])
def test_stage_chunk_scan(w):
    """Fed the oracle's log decays and entry states, the chunk scan must give the
    oracle's y."""
    say(f"[stage chunk_scan] {w.describe()}")
    cpu = generate(w)
    c = {k: np64(v) for k, v in cpu.items()}
    cs = oracle.chunk_cumsum(c["dt"], c["A"], w.chunk_len)
    ent, _ = oracle.entry_states(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], w.chunk_len,
                                 init_state=c["init_state"])
    y_ref, _ = oracle_fwd(cpu)
    dv = to_device(cpu)
    d = _dims(w)
    dtc, _ = binding.ssd_chunk_cumsum(d, w.chunk_len, dv["dt"], dv["A"])
    cs_d = torch.from_numpy(cs).float().cuda()
    ent_d = torch.from_numpy(ent.swapaxes(-1, -2).copy()).to(cpu["x"].dtype).cuda()
    gram = binding.ssd_chunk_gram(d, w.chunk_len, dv["B"], dv["C"])
    y = binding.ssd_chunk_scan(d, w.chunk_len, dv["x"], dv["B"], dv["C"], dtc, cs_d, dv["D"], ent_d,
                               gram=gram)
    torch.cuda.synchronize()
    e = rel_l2(np64(y), y_ref)
    say(f"    rel_l2 y={e:.3e}")
    assert e <= TOL[w.dtype]


# ------------------------------------------------------------------ invariants

def test_chunk_length_does_not_change_the_result():
    base = variants(STRESS["slow_decay"], seqlen=1000)
    cpu = generate(base)
    y_ref, f_ref = oracle_fwd(cpu)
    dv = to_device(cpu)
    outs = []
    for q in (64, 128, 256):
        say(f"[chunk invariance] Q={q}")
        y, fin = gpu_fwd(dv, q)
        assert rel_l2(np64(y), y_ref) <= TOL["bf16"]
        assert rel_l2(np64(fin), f_ref) <= TOL["bf16"]
        outs.append(np64(y))
    assert rel_l2(outs[0], outs[2]) <= TOL["bf16"]


def test_deterministic_run_to_run():
    w = STRESS["slow_decay"]
    dv = to_device(generate(w))
    say("[determinism]")
    y1, f1 = gpu_fwd(dv, w.chunk_len)
    y2, f2 = gpu_fwd(dv, w.chunk_len)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


def _at_4_byte_offset(t):
    """A copy of t whose storage starts 4 bytes past a 16-byte boundary."""
    buf = torch.empty(t.numel() + 4, dtype=t.dtype, device=t.device)
    out = buf[1:1 + t.numel()].view(t.shape)
    out.copy_(t)
    assert out.data_ptr() % 16 == 4
    return out


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_states_at_4_byte_offsets_match_aligned(dtype):
    """init_state and final_state need only 4-byte alignment.  The state kernel moves them
    in 16-byte runs through LDS when they are 16-byte aligned and element by element
    otherwise; both give the same bits, forward and backward (d_final, d_init)."""
    w = variants(STRESS["slow_decay"], dtype=dtype)
    dv = to_device(generate(w))
    say(f"[state alignment] {dtype}")
    args = (dv["x"], dv["dt"], dv["A"], dv["B"], dv["C"], dv["D"], w.chunk_len)
    y0, f0 = binding.ssd_fwd(*args, init_state=dv["init_state"])
    fin = _at_4_byte_offset(torch.zeros_like(f0))
    y1, f1 = binding.ssd_fwd(*args, init_state=_at_4_byte_offset(dv["init_state"]),
                             final_state=fin)
    assert torch.equal(y0, y1) and torch.equal(f0, f1)
    g = torch.Generator(device="cpu").manual_seed(5)
    dy = torch.randn(dv["x"].shape, generator=g).to(dv["x"])
    dfin = torch.randn(f0.shape, generator=g).to(f0)
    o0 = binding.ssd_bwd(*args, dy, init_state=dv["init_state"], d_final=dfin)
    dinit = _at_4_byte_offset(torch.zeros_like(o0["d_init"]))
    o1 = binding.ssd_bwd(*args, dy, init_state=_at_4_byte_offset(dv["init_state"]),
                         d_final=_at_4_byte_offset(dfin), out={"d_init": dinit})
    for k in o0:
        assert torch.equal(o0[k], o1[k]), k


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_split_run_resumes_from_final_state(dtype):
    """Two segments, the second starting from the first's final state, reproduce one
    run over the whole sequence (the state hand-off of sequence parallelism)."""
    w = variants(STRESS["slow_decay"], dtype=dtype, seqlen=768, batch=1)
    cpu = generate(w)
    dv = to_device(cpu)
    say(f"[split run] {dtype}")
    y_full, f_full = gpu_fwd(dv, w.chunk_len)
    T1 = 300   # not a chunk multiple
    first = {k: (v[:, :T1].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in dv.items()}
    ya, fa = gpu_fwd(first, w.chunk_len)
    second = {k: (v[:, T1:].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in dv.items()}
    second["init_state"] = fa
    yb, fb = gpu_fwd(second, w.chunk_len)
    y_ref, f_ref = oracle_fwd(cpu)
    y_split = np.concatenate([np64(ya), np64(yb)], axis=1)
    assert rel_l2(y_split, y_ref) <= TOL[dtype]
    assert rel_l2(np64(fb), f_ref) <= TOL[dtype]
    assert rel_l2(y_split, np64(y_full)) <= TOL[dtype]


def test_empty_sequence_and_empty_batch():
    say("[empty]")
    w = Workload("t0", 2, 0, 2, 32, 32, 1, 64, init_state=True)
    cpu = generate(w)
    dv = to_device(cpu)
    y, fin = gpu_fwd(dv, 64)
    assert y.numel() == 0
    assert torch.equal(fin, dv["init_state"])
    dv["init_state"] = None
    y, fin = gpu_fwd(dv, 64)
    assert torch.count_nonzero(fin) == 0
    w = Workload("b0", 0, 64, 2, 32, 32, 1, 64)
    dv = to_device(generate(w))
    y, fin = gpu_fwd(dv, 64)
    assert y.numel() == 0 and fin.numel() == 0


def test_bad_arguments_raise():
    w = TINY_FP32
    dv = to_device(generate(w))
    with pytest.raises(binding.SsdError) as ei:
        binding.ssd_fwd(dv["x"], dv["dt"], dv["A"], dv["B"], dv["C"], dv["D"], 96)
    assert ei.value.code == 3
    with pytest.raises(TypeError):
        binding.ssd_fwd(dv["x"], dv["dt"].double(), dv["A"], dv["B"], dv["C"], dv["D"], 64)


# ------------------------------------------------------------------ MFMA instantiations

SWEEP = [  # (headdim P, dstate N, chunk Q, groups)
    (16, 64, 64, 1), (32, 32, 128, 2), (64, 256, 256, 1), (128, 128, 128, 2),
    (128, 256, 64, 1), (16, 256, 128, 2), (64, 64, 256, 2), (128, 32, 256, 1),
    (32, 128, 64, 1), (64, 128, 128, 1), (128, 64, 256, 2), (16, 16, 64, 1),
    (16, 128, 256, 2),
]


@pytest.mark.parametrize("shape", SWEEP, ids=[f"P{p}_N{n}_Q{q}_G{g}" for p, n, q, g in SWEEP])
def test_shape_sweep_matches_oracle(shape):
    """Every kernel instantiation family (and the VALU fallback for N=16), with a ragged
    tail, slow decay and an init state."""
    P, N, Q, G = shape
    w = Workload(f"sweep_P{P}_N{N}_Q{Q}", 1, 2 * Q + 37, 2, P, N, G, Q, init_state=True,
                 log_neg_a_range=(np.log(0.005), np.log(0.05)))
    say(f"[sweep] {w.describe()}")
    cpu = generate(w)
    y, fin = gpu_fwd(to_device(cpu), Q)
    y_ref, f_ref = oracle_fwd(cpu)
    ey, ef = rel_l2(np64(y), y_ref), rel_l2(np64(fin), f_ref)
    say(f"    rel_l2 y={ey:.3e} final={ef:.3e}")
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"]


# ------------------------------------------------------------------ persistent pipelines

PIPE = [  # (batch, seqlen, heads, headdim P, dstate N, groups, chunk Q)
    (2, 16384, 8, 64, 128, 4, 256),   # 4 items per workgroup, crossing units
    (1, 32768, 4, 32, 128, 2, 128),
    (2, 16384, 4, 128, 128, 2, 256),  # single-buffered scan
    (1, 8192, 6, 16, 128, 3, 64),
    (2, 16384, 8, 64, 256, 4, 256),   # N = 256: B in two column slices, crossing units
    (1, 8192, 6, 32, 256, 3, 128),
]


@pytest.mark.parametrize("shape", PIPE, ids=[f"B{b}_T{t}_H{h}_P{p}_N{n}_G{g}_Q{q}"
                                             for b, t, h, p, n, g, q in PIPE])
def test_pipelined_runs_match_oracle(shape):
    """Enough (unit, head) items that each persistent workgroup walks several of them,
    across unit boundaries, so the prefetched copies and the register-resident per-unit
    operands are all exercised; slow decay keeps every carried state visible."""
    Bz, T, H, P, N, G, Q = shape
    w = Workload(f"pipe_{Bz}_{T}_{H}_{P}_{N}_{G}_{Q}", Bz, T, H, P, N, G, Q, init_state=True,
                 log_neg_a_range=(np.log(0.005), np.log(0.05)))
    say(f"[pipeline] {w.describe()}")
    cpu = generate(w)
    y, fin = gpu_fwd(to_device(cpu), Q)
    y_ref, f_ref = oracle_fwd(cpu)
    ey, ef = rel_l2(np64(y), y_ref), rel_l2(np64(fin), f_ref)
    say(f"    rel_l2 y={ey:.3e} final={ef:.3e}")
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"]


GRAM_CASES = [  # (batch, seqlen, heads, headdim P, dstate N, groups, chunk Q)
    (2, 4096 + 77, 6, 64, 128, 3, 256),   # blocks written by the states kernel itself
    (1, 8192, 16, 32, 128, 2, 256),       # several units per workgroup
    (1, 1000, 4, 64, 64, 2, 128),         # separate launch after the states kernel
    (2, 2048 + 100, 6, 64, 256, 2, 256),  # N = 256: summed over the two B column slices
]


@pytest.mark.parametrize("shape", GRAM_CASES, ids=[f"B{b}_T{t}_H{h}_P{p}_N{n}_G{g}_Q{q}"
                                                   for b, t, h, p, n, g, q in GRAM_CASES])
def test_chunk_state_fills_the_same_gram_blocks(shape):
    """ssd_chunk_state given a gram buffer writes exactly what ssd_chunk_gram writes."""
    Bz, T, H, P, N, G, Q = shape
    w = Workload(f"gram_{Bz}_{T}_{H}_{P}_{N}_{G}_{Q}", Bz, T, H, P, N, G, Q)
    say(f"[gram via chunk_state] {w.describe()}")
    dv = to_device(generate(w))
    d = _dims(w)
    dtc, cs = binding.ssd_chunk_cumsum(d, Q, dv["dt"], dv["A"])
    ref = binding.ssd_chunk_gram(d, Q, dv["B"], dv["C"])
    assert ref.numel() > 0
    got = torch.full_like(ref, 0x5A)
    binding.ssd_chunk_state(d, Q, dv["x"], dv["B"], dtc, cs, C=dv["C"], gram=got)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


# ------------------------------------------------------------------ ssd_fwd = its stages

STAGED = [  # (batch, seqlen, heads, headdim P, dstate N, groups, chunk Q)
    (2, 4096 + 77, 6, 64, 128, 3, 256),   # ragged last chunk, C B^T written by the same pass
    (1, 8192, 16, 32, 128, 2, 128),
    (2, 3000, 8, 64, 64, 2, 64),
    (1, 5000, 4, 32, 256, 1, 256),
    (1, 5000, 4, 64, 256, 1, 256),
]


@pytest.mark.parametrize("shape", STAGED, ids=[f"B{b}_T{t}_H{h}_P{p}_N{n}_G{g}_Q{q}"
                                               for b, t, h, p, n, g, q in STAGED])
def test_fwd_equals_its_stages(shape):
    """ssd_fwd leaves in its workspace exactly the dt_chunk and cs of ssd_chunk_cumsum, and
    gives exactly the y and final state of the stage-by-stage calls (with the C B^T blocks
    from their own launch)."""
    Bz, T, H, P, N, G, Q = shape
    w = Workload(f"staged_{Bz}_{T}_{H}_{P}_{N}_{G}_{Q}", Bz, T, H, P, N, G, Q, init_state=True)
    say(f"[fwd = stages] {w.describe()}")
    dv = to_device(generate(w))
    d = _dims(w)
    ws = torch.zeros(binding.ssd_fwd_workspace_size(d, Q), dtype=torch.uint8, device="cuda")
    y, fin = binding.ssd_fwd(dv["x"], dv["dt"], dv["A"], dv["B"], dv["C"], dv["D"], Q,
                             init_state=dv["init_state"], workspace=ws)
    dtc, cs = binding.ssd_chunk_cumsum(d, Q, dv["dt"], dv["A"])
    S = binding.ssd_chunk_state(d, Q, dv["x"], dv["B"], dtc, cs)
    E, f2 = binding.ssd_state_passing(d, Q, S, cs, init_state=dv["init_state"])
    gram = binding.ssd_chunk_gram(d, Q, dv["B"], dv["C"])
    y2 = binding.ssd_chunk_scan(d, Q, dv["x"], dv["B"], dv["C"], dtc, cs, dv["D"], E, gram=gram)
    torch.cuda.synchronize()
    # the workspace begins with dt_chunk, then cs, each rounded up to 256 bytes
    n = dtc.numel()
    off = (n * 4 + 255) // 256 * 256
    assert torch.equal(ws[:n * 4].view(torch.float32), dtc.reshape(-1))
    assert torch.equal(ws[off:off + n * 4].view(torch.float32), cs.reshape(-1))
    assert torch.equal(y, y2)
    assert torch.equal(fin, f2)
