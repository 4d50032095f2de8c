"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle on the same
inputs (upcast to fp64, which is exact for fp32 and bf16), and compare."""
import sys

import numpy as np
import torch

import oracle
from mamba_ssd_chunked_03_amd import binding
from mamba_ssd_chunked_03_amd.workloads import head_slice

# Tolerances on rel-L2 = ||gpu - oracle||_2 / ||oracle||_2 over a whole tensor, as stated
# for the SSD forward: 1e-4 with fp32 inputs, 2e-2 with bf16 inputs (fp32 accumulation).
TOL = {"fp32": 1e-4, "bf16": 2e-2}


def say(*msg):
    print(*msg, file=sys.stderr, flush=True)


def np64(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def rel_l2(u, ref):
    u = np.asarray(u, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert u.shape == ref.shape, (u.shape, ref.shape)
    assert np.isfinite(u).all(), "non-finite values in the GPU result"
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((u - ref).ravel())
    return num / den if den > 0 else num


def to_device(inputs, device="cuda"):
    return {k: (None if v is None else v.to(device)) for k, v in inputs.items()}


def gpu_fwd(dev_inputs, chunk_len):
    d = dev_inputs
    y, fin = binding.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], chunk_len,
                             init_state=d["init_state"])
    torch.cuda.synchronize()
    return y, fin


def oracle_fwd(cpu_inputs, nthreads=0):
    c = {k: np64(v) for k, v in cpu_inputs.items()}
    y, fin, _ = oracle.ssd_ref(c["x"], c["dt"], c["A"], c["B"], c["C"], c["D"],
                               init_state=c["init_state"], nthreads=nthreads)
    return y, fin


def sampled_pairs(w, count=4):
    """(batch, head) pairs spread over the workload, always including the first and last."""
    pairs = {(0, 0), (w.batch - 1, w.nheads - 1)}
    rng = np.random.default_rng(1234)
    while len(pairs) < min(count, w.batch * w.nheads):
        pairs.add((int(rng.integers(w.batch)), int(rng.integers(w.nheads))))
    return sorted(pairs)


def check_sampled(w, cpu_inputs, y_gpu, fin_gpu, count=4):
    """Compare whole (b, h) sequences of the GPU output with the oracle run on just that
    sequence.  Returns the worst rel-L2 of y and of the final state."""
    worst_y = worst_f = 0.0
    for b, h in sampled_pairs(w, count):
        sl = head_slice(cpu_inputs, w, b, h)
        y_ref, f_ref = oracle_fwd(sl)
        ey = rel_l2(np64(y_gpu[b:b + 1, :, h:h + 1, :]), y_ref)
        worst_y = max(worst_y, ey)
        if fin_gpu is not None:
            ef = rel_l2(np64(fin_gpu[b:b + 1, h:h + 1]), f_ref)
            worst_f = max(worst_f, ef)
    return worst_y, worst_f
