"""ssd_fwd_noalloc (through the C ABI): the forward with its stage buffers in the library's
fixed device array, for callers that cannot allocate.  Two calls in a row, the second on
a smaller input, each checked against ssd_fwd (with a workspace of its own) bit for bit and
against the oracle at the forward's bar; then the full bench-sized layer, and the size
limit."""
import numpy as np
import pytest
import torch

from mamba_ssd_chunked_03_amd import binding
from mamba_ssd_chunked_03_amd.workloads import MAMBA2_2P7B, Workload, generate
from parity import TOL, np64, oracle_fwd, rel_l2, say, to_device

pytestmark = pytest.mark.gpu

LN = np.log
CASES = [  # the second smaller than the first, as a caller reusing the array would do
    Workload("noalloc_big", 2, 2048 + 77, 8, 64, 128, 2, 256, init_state=True,
             log_neg_a_range=(LN(0.005), LN(0.05))),
    Workload("noalloc_small", 1, 300, 4, 64, 64, 1, 64, init_state=True,
             log_neg_a_range=(LN(0.01), LN(0.1))),
]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    binding.library()
    torch.cuda.init()


def _both(w):
    cpu = generate(w)
    d = to_device(cpu)
    args = (d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], w.chunk_len)
    y1, f1 = binding.ssd_fwd(*args, init_state=d["init_state"])
    y2, f2 = binding.ssd_fwd_noalloc(*args, init_state=d["init_state"])
    torch.cuda.synchronize()
    return cpu, y1, f1, y2, f2


def test_noalloc_equals_ssd_fwd_on_two_calls_the_second_smaller():
    for w in CASES + [Workload("noalloc_fp32", 1, 200, 2, 32, 32, 1, 64, dtype="fp32",
                               init_state=True, log_neg_a_range=(LN(0.01), LN(0.1)))]:
        say(f"[noalloc] {w.describe()}")
        cpu, y1, f1, y2, f2 = _both(w)
        assert torch.equal(y1, y2) and torch.equal(f1, f2)
        y_ref, f_ref = oracle_fwd(cpu)
        ey, ef = rel_l2(np64(y2), y_ref), rel_l2(np64(f2), f_ref)
        say(f"    rel_l2 y={ey:.3e} final={ef:.3e}")
        assert ey <= TOL[w.dtype] and ef <= TOL[w.dtype]


def test_noalloc_at_the_bench_workload():
    """The 2.7B-shaped layer fits the array (183 MB of stage buffers): bit-identical to
    ssd_fwd."""
    w = MAMBA2_2P7B
    say(f"[noalloc] {w.describe()}")
    _, y1, f1, y2, f2 = _both(w)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


def test_noalloc_refuses_a_problem_larger_than_the_array():
    w = Workload("noalloc_too_big", 1, 65536, 80, 64, 128, 8, 256)  # 671 MB of entry states
    d = to_device(generate(w))
    with pytest.raises(binding.SsdError) as ei:
        binding.ssd_fwd_noalloc(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], 256)
    assert ei.value.code == 5
