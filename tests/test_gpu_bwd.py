"""Parity of the backward (ssd_bwd through the C ABI) with the fp64 oracle, on the GPU.

Every gradient (dx, ddt, dA, dB, dC, dD, d_init) is compared by rel-L2 with the oracle's
reverse-mode differentiation of the token recurrence, on the same seeded inputs and
upstream gradients, at the forward's bounds: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs
(fp32 accumulation).  Each is checked whole-tensor, and all but the per-head sums dA and
dD per slice as well: per (b, h) sequence, per (b, g) for dB and dC.
"""
import numpy as np
import pytest
import torch

import oracle
from mamba_ssd_chunked_03_amd import binding
from mamba_ssd_chunked_03_amd.workloads import (STRESS, TINY_FP32, WORKLOADS, Workload,
                                                generate, generate_grads, variants)
from parity import TOL, np64, per_seq_rel_l2, rel_l2, say, seq_errors, to_device

pytestmark = pytest.mark.gpu

GRADS = ("dx", "ddt", "dA", "dB", "dC", "dD", "d_init")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    binding.library()
    torch.cuda.init()
    return torch.device("cuda:0")


def gpu_bwd(w, cpu, up):
    d = to_device(cpu)
    u = to_device(up)
    g = binding.ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], w.chunk_len, u["dy"],
                        init_state=d["init_state"], d_final=u["d_final"])
    torch.cuda.synchronize()
    return g


def oracle_bwd(cpu, up):
    c = {k: np64(v) for k, v in cpu.items()}
    return oracle.ssd_bwd_ref(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"], np64(up["dy"]),
                              init_state=c["init_state"], d_final=np64(up["d_final"]))


# Per-slice checks next to the whole-tensor one: the axes summed over for one slice of each
# gradient (per (b, h) sequence; per (b, g) for the group gradients dB and dC).  dA and dD
# hold one value per head, each a sum over every batch element and step of terms of both
# signs, so a single head's value has no scale of its own: they are bounded as whole
# vectors, and each head's error against the vector's rms is only logged.
SLICE_AXES = {"dx": (1, 3), "ddt": (1,), "dB": (1, 3), "dC": (1, 3), "d_init": (2, 3)}


def compare(w, g, ref):
    tol = TOL[w.dtype]
    whole, worst = {}, {}
    for k in GRADS:
        u = np64(g[k])
        whole[k] = rel_l2(u, ref[k])
        if k in SLICE_AXES:
            err2, ref2 = seq_errors(u, ref[k], SLICE_AXES[k])
            sl = per_seq_rel_l2(err2, ref2)
            i = np.unravel_index(np.argmax(sl), sl.shape)
            worst[k] = (float(sl[i]), tuple(int(v) for v in i))
        else:
            r = np.asarray(ref[k], dtype=np.float64)
            rms = np.sqrt(np.mean(r ** 2))
            e = np.abs(u - r) / (rms if rms > 0 else 1.0)
            worst[k] = (float(e.max()), (int(np.argmax(e)),))
    say("    whole " + " ".join(f"{k}={v:.2e}" for k, v in whole.items()))
    say("    worst slice " + " ".join(f"{k}={v:.2e}@{i}" for k, (v, i) in worst.items()))
    for k, v in whole.items():
        assert v <= tol, f"{k}: rel_l2 {v:.3e} > {tol}"
    for k, (v, i) in worst.items():
        if k in SLICE_AXES:
            assert v <= tol, f"{k} at {i}: rel_l2 {v:.3e} > {tol}"


CASES = [
    TINY_FP32,
    variants(TINY_FP32, name="tiny_fp32_init", init_state=True,
             log_neg_a_range=(np.log(0.01), np.log(0.1))),
    STRESS["slow_decay_fp32"],
    STRESS["ragged_250_q64"],
    STRESS["short_t17"],
    STRESS["short_t1"],
    STRESS["a_zero"],
    STRESS["dt_zero"],
    STRESS["groups_half"],
    STRESS["slow_decay"],
    Workload("bwd_ragged_q128_fp32", 2, 300, 3, 64, 32, 1, 128, dtype="fp32", init_state=True,
             log_neg_a_range=(np.log(0.01), np.log(0.1))),
    Workload("bwd_g2_q256", 1, 700, 4, 64, 128, 2, 256, init_state=True,
             log_neg_a_range=(np.log(0.005), np.log(0.05))),
    # N = 256: the recomputed states and the state gradients run the pipelined states
    # kernel with B (C) in two column slices, two items per workgroup across units; the
    # in-chunk part runs the carried-state kernel and then the in-chunk kernel
    Workload("bwd_n256_pipe", 2, 8192, 8, 64, 256, 2, 256, init_state=True,
             log_neg_a_range=(np.log(0.005), np.log(0.05))),
    # N = 256 at the other chunk lengths, each with a ragged last chunk (44 and 60 rows:
    # row blocks past the end, and a block cut inside)
    Workload("bwd_n256_q64", 1, 300, 4, 64, 256, 2, 64, init_state=True,
             log_neg_a_range=(np.log(0.01), np.log(0.1))),
    Workload("bwd_n256_q128", 2, 700, 6, 64, 256, 3, 128, init_state=True,
             log_neg_a_range=(np.log(0.005), np.log(0.05))),
    # headdim 32 on the matrix cores (ragged_250_q64 and short_t17 above are too): B and C
    # through LDS in 64- and 32-column slices for C B^T, W staged past the exchange area
    Workload("bwd_p32_q256", 2, 1000, 8, 32, 128, 2, 256, init_state=True,
             log_neg_a_range=(np.log(0.005), np.log(0.05))),
    Workload("bwd_p32_n64_q256", 1, 600, 4, 32, 64, 1, 256, init_state=True,
             log_neg_a_range=(np.log(0.01), np.log(0.1))),
    Workload("bwd_p32_q128", 1, 500, 4, 32, 128, 1, 128, init_state=True,
             log_neg_a_range=(np.log(0.005), np.log(0.05))),
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_bwd_matches_oracle_small(w):
    say(f"[bwd small] {w.describe()}")
    cpu = generate(w)
    up = generate_grads(w)
    g = gpu_bwd(w, cpu, up)
    compare(w, g, oracle_bwd(cpu, up))


def test_bwd_without_final_gradient_or_init():
    """d_final = None is a zero final-state gradient; init_state = None a zero init."""
    w = variants(STRESS["ragged_250_q64"], name="bwd_no_final", init_state=False)
    cpu = generate(w)
    up = generate_grads(w, with_final=False)
    g = gpu_bwd(w, cpu, up)
    compare(w, g, oracle_bwd(cpu, up))


def test_bwd_empty_sequence():
    """T = 0: no step gradients; dA = dD = 0 and d_init = d_final."""
    w = Workload("bwd_empty", 2, 0, 4, 32, 64, 2, 64, init_state=True)
    cpu = generate(w)
    up = generate_grads(w)
    d = to_device(cpu)
    u = to_device(up)
    g = binding.ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], 64, u["dy"],
                        init_state=d["init_state"], d_final=u["d_final"],
                        out=dict(dA=torch.full((4,), 7.0, device="cuda"),
                                 dD=torch.full((4,), 7.0, device="cuda")))
    torch.cuda.synchronize()
    assert torch.equal(g["dA"].cpu(), torch.zeros(4))
    assert torch.equal(g["dD"].cpu(), torch.zeros(4))
    assert torch.equal(g["d_init"].cpu(), up["d_final"])


def test_bwd_is_deterministic():
    w = STRESS["groups_half"]
    cpu = generate(w)
    up = generate_grads(w)
    a = gpu_bwd(w, cpu, up)
    b = gpu_bwd(w, cpu, up)
    for k in GRADS:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["mamba2_2p7b", "mamba2_130m", "nsweep_n64", "nsweep_n128",
                                  "nsweep_n256", "long_ctx_65k"])
def test_bwd_full_size_workloads(name):
    """The model-shaped backward workloads at full size, with the launch configuration that
    bench.py --bwd times (bf16, Q = 256; the MFMA in-chunk kernel, preceded at N = 256 by
    the carried-state kernel), compared with the oracle's reverse-mode pass over every
    (b, h) sequence.  long_ctx_65k adds eight groups of ten heads, an initial state and 256
    chunks per sequence."""
    w = WORKLOADS[name]
    say(f"[bwd full] {w.describe()}")
    cpu = generate(w)
    up = generate_grads(w)
    g = gpu_bwd(w, cpu, up)
    compare(w, g, oracle_bwd(cpu, up))


SAVED_CASES = ["slow_decay", "tiny_fp32", "bwd_g2_q256", "bwd_n256_q128", "bwd_p32_q256"]


@pytest.mark.parametrize("w", [{c.name: c for c in CASES}[n] for n in SAVED_CASES],
                         ids=SAVED_CASES)
def test_bwd_saved_equals_recompute(w):
    """ssd_bwd_saved (the forward's intermediates read from its workspace) gives the same
    bits as ssd_bwd (which recomputes them)."""
    cpu = generate(w)
    up = generate_grads(w)
    d = to_device(cpu)
    u = to_device(up)
    dims = binding.dims_of(d["x"], d["B"])
    fws = torch.empty(max(1, binding.ssd_fwd_workspace_size(dims, w.chunk_len)),
                      dtype=torch.uint8, device="cuda")
    binding.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], w.chunk_len,
                    init_state=d["init_state"], workspace=fws)
    a = binding.ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], w.chunk_len, u["dy"],
                        init_state=d["init_state"], d_final=u["d_final"])
    b = binding.ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], w.chunk_len, u["dy"],
                        init_state=d["init_state"], d_final=u["d_final"], fwd_workspace=fws)
    torch.cuda.synchronize()
    for k in GRADS:
        assert torch.equal(a[k], b[k]), k
