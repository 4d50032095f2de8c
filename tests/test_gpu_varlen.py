"""Parity of packed variable-length rows (ssd_fwd_varlen through the C ABI) with the fp64
oracle (oracle/varlen.py: every sequence through the recurrence on its own), on the GPU.

y and the per-sequence final states are compared whole-tensor by rel-L2 at the layer's
bounds (1e-4 fp32, 2e-2 bf16).  Cases:
- starts inside chunks, on chunk boundaries, several in one chunk, and empty sequences;
- a single sequence, which must equal ssd_fwd bit for bit;
- every kernel path (fp32 VALU, bf16 MFMA at Q = 64 / 256, N = 64 / 128, G > 1);
- a model-shaped packed row at full size.
"""
import numpy as np
import pytest
import torch

from mamba_ssd_chunked_03_amd import binding
from mamba_ssd_chunked_03_amd.workloads import Workload, generate
from oracle.varlen import ssd_varlen_ref
from parity import TOL, np64, per_seq_rel_l2, rel_l2, say, seq_errors

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    binding.library()
    torch.cuda.init()
    return torch.device("cuda:0")


def _run(w, cu):
    cpu = generate(w)
    d = {k: (None if v is None else v.to("cuda")) for k, v in cpu.items()}
    cut = torch.tensor(cu, dtype=torch.int32, device="cuda")
    y, fin = binding.ssd_fwd_varlen(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"],
                                    w.chunk_len, cut)
    torch.cuda.synchronize()
    c = {k: np64(v) for k, v in cpu.items()}
    ry, rf = ssd_varlen_ref(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], cu)
    return y, fin, ry, rf


def _check(w, y, fin, ry, rf, cu):
    """Whole tensors, and every (sequence, head) on its own: y over the sequence's steps,
    its final state."""
    tol = TOL[w.dtype]
    yg, fg = np64(y), np64(fin)
    ey, ef = rel_l2(yg, ry), rel_l2(fg, rf)
    # A sequence of one or a few steps has y = k x per head for a scalar k = dt C.B + D
    # (one step), which can cancel to near zero: its own norm is then no scale for the
    # rounding of the two terms.  Each (sequence, head) is measured against its own norm,
    # or a quarter of the typical norm of that many outputs where its own is smaller.
    ms = np.mean(ry ** 2, axis=(0, 1, 3))  # per head
    sy = []
    for s in range(len(cu) - 1):
        if cu[s + 1] > cu[s]:
            err2, ref2 = seq_errors(yg[:, cu[s]:cu[s + 1]], ry[:, cu[s]:cu[s + 1]], (0, 1, 3))
            floor = (0.25 ** 2) * ms * (cu[s + 1] - cu[s]) * ry.shape[3]
            sy.append(per_seq_rel_l2(err2, np.maximum(ref2, floor)).max())
    err2, ref2 = seq_errors(fg, rf, (2, 3))
    sf = per_seq_rel_l2(err2, ref2)
    wy, wf = max(sy), sf.max()
    say(f"    whole y={ey:.2e} final={ef:.2e}; worst (sequence, head) y={wy:.2e} "
        f"final={wf:.2e}")
    assert ey <= tol, f"y: {ey:.3e}"
    assert ef <= tol, f"final states: {ef:.3e}"
    assert wy <= tol, f"y of one (sequence, head): {wy:.3e}"
    assert wf <= tol, f"final state of one (sequence, head): {wf:.3e}"


LN = np.log
CASES = [
    # fp32, Q = 64: starts inside chunks, at a chunk boundary (64), two in one chunk
    (Workload("vl_fp32", 1, 300, 2, 16, 16, 1, 64, dtype="fp32",
              log_neg_a_range=(LN(0.01), LN(0.1))), [0, 37, 64, 90, 100, 230, 300]),
    (Workload("vl_fp32_g2", 1, 200, 4, 32, 32, 2, 64, dtype="fp32",
              log_neg_a_range=(LN(0.01), LN(0.1))), [0, 1, 2, 130, 130, 200]),
    # bf16 MFMA Q = 256, N = 128, P = 64
    (Workload("vl_bf16_q256", 1, 1000, 4, 64, 128, 1, 256,
              log_neg_a_range=(LN(0.005), LN(0.05))), [0, 100, 256, 257, 600, 1000]),
    # bf16 MFMA Q = 64, N = 64, several starts per chunk
    (Workload("vl_bf16_q64", 1, 500, 4, 64, 64, 2, 64,
              log_neg_a_range=(LN(0.01), LN(0.1))),
     [0, 5, 9, 20, 33, 40, 63, 64, 65, 128, 200, 201, 202, 203, 350, 500]),
    # bf16, Q = 128, empty sequences at the ends
    (Workload("vl_bf16_q128", 1, 384, 2, 64, 128, 1, 128,
              log_neg_a_range=(LN(0.01), LN(0.1))), [0, 0, 128, 300, 384, 384]),
]


@pytest.mark.parametrize("w,cu", CASES, ids=[c[0].name for c in CASES])
def test_varlen_matches_oracle(w, cu):
    say(f"[varlen] {w.describe()} cu={cu}")
    y, fin, ry, rf = _run(w, cu)
    _check(w, y, fin, ry, rf, cu)


def test_single_sequence_equals_ssd_fwd():
    w = Workload("vl_one", 1, 700, 4, 64, 128, 1, 256, log_neg_a_range=(LN(0.005), LN(0.05)))
    cpu = generate(w)
    d = {k: (None if v is None else v.to("cuda")) for k, v in cpu.items()}
    cut = torch.tensor([0, 700], dtype=torch.int32, device="cuda")
    y, fin = binding.ssd_fwd_varlen(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], 256, cut)
    y2, f2 = binding.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], 256)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    # the final state goes through the stored (rounded) entry state of the last chunk
    assert rel_l2(np64(fin[0]), np64(f2[0])) <= TOL[w.dtype]


def test_varlen_full_size_packed_row():
    """The 2.7B layer's 16384 tokens as one packed row of seeded sequence lengths (64 to
    4096 steps), compared whole-tensor."""
    rng = np.random.default_rng(11)
    T = 16384
    cuts = [0]
    while cuts[-1] < T:
        cuts.append(min(T, cuts[-1] + int(rng.integers(64, 4097))))
    w = Workload("vl_2p7b_packed", 1, T, 80, 64, 128, 1, 256)
    say(f"[varlen full] {w.describe()} {len(cuts) - 1} sequences")
    y, fin, ry, rf = _run(w, cuts)
    _check(w, y, fin, ry, rf, cuts)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_dense_packing_of_short_sequences(dtype):
    """Sequences of 1 to 4 steps packed at chunk length 256, about 100 starts per chunk.
    Every start lowers the running log-decay sum by the gap, so the sums reach about
    -120 k inside a chunk with k starts, and each decay carries a relative error of about
    ulp(120 k): the documented precision limit of dense packing.  The bound checked here is
    that limit (2e-3 in fp32); bf16 keeps the layer's own bar."""
    rng = np.random.default_rng(5)
    T = 1024
    cuts = [0]
    while cuts[-1] < T:
        cuts.append(min(T, cuts[-1] + int(rng.integers(1, 5))))
    w = Workload(f"vl_dense_{dtype}", 1, T, 4, 64, 64, 1, 256, dtype=dtype,
                 log_neg_a_range=(LN(0.01), LN(0.1)))
    say(f"[varlen dense] {w.describe()} {len(cuts) - 1} sequences")
    y, fin, ry, rf = _run(w, cuts)
    ey, ef = rel_l2(np64(y), ry), rel_l2(np64(fin), rf)
    say(f"    whole y={ey:.2e} final={ef:.2e}")
    bound = 2e-3 if dtype == "fp32" else TOL["bf16"]
    assert ey <= bound and ef <= bound
