"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle on the same
inputs (upcast to fp64, which is exact for fp32 and bf16), and compare."""
import sys

import numpy as np
import torch

import oracle
from mamba_ssd_chunked_03_amd import binding

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


def seq_errors(u, ref, axes):
    """Squared error and squared reference norm summed over `axes`: one entry per
    remaining index (per sequence, when the remaining axes are batch and head)."""
    u = np.asarray(u, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert u.shape == ref.shape, (u.shape, ref.shape)
    assert np.isfinite(u).all(), "non-finite values in the GPU result"
    return ((u - ref) ** 2).sum(axis=axes), (ref ** 2).sum(axis=axes)


def per_seq_rel_l2(err2, ref2):
    """rel-L2 of each slice from its summed squared error and reference norm (the absolute
    error where the reference is all zeros)."""
    err2 = np.asarray(err2, dtype=np.float64)
    ref2 = np.asarray(ref2, dtype=np.float64)
    return np.where(ref2 > 0, np.sqrt(err2 / np.where(ref2 > 0, ref2, 1.0)), np.sqrt(err2))


class SeqReport:
    """Whole-tensor and per-(b, h) rel-L2 of y and of the final state, accumulated over
    blocks of sequences."""

    def __init__(self, batch, nheads):
        self.ey = np.zeros((batch, nheads))
        self.ry = np.zeros((batch, nheads))
        self.ef = np.zeros((batch, nheads))
        self.rf = np.zeros((batch, nheads))

    def add(self, b, h0, y_gpu, y_ref, f_gpu, f_ref):
        h1 = h0 + y_ref.shape[2]
        e, r = seq_errors(y_gpu, y_ref, (0, 1, 3))
        self.ey[b, h0:h1], self.ry[b, h0:h1] = e, r
        if f_gpu is not None:
            e, r = seq_errors(f_gpu, f_ref, (0, 2, 3))
            self.ef[b, h0:h1], self.rf[b, h0:h1] = e, r

    def whole(self):
        f = lambda e, r: np.sqrt(e.sum() / r.sum()) if r.sum() > 0 else np.sqrt(e.sum())
        return f(self.ey, self.ry), f(self.ef, self.rf)

    def worst(self):
        """(worst y rel-L2, its (b, h)), (worst final-state rel-L2, its (b, h))."""
        sy, sf = per_seq_rel_l2(self.ey, self.ry), per_seq_rel_l2(self.ef, self.rf)
        iy = np.unravel_index(np.argmax(sy), sy.shape)
        jf = np.unravel_index(np.argmax(sf), sf.shape)
        return (float(sy[iy]), tuple(int(i) for i in iy)), (float(sf[jf]), tuple(int(i) for i in jf))


def check_every_sequence(w, cpu_inputs, y_gpu, fin_gpu, heads_per_call=16):
    """Compare every (b, h) sequence of the GPU output with the oracle.  The oracle runs
    over all of them, a block of heads of one group at a time (which bounds host memory at
    the largest sizes); each sequence's rel-L2 is recorded next to the whole-tensor one.
    Returns the SeqReport."""
    hpg = w.nheads // w.ngroups
    step = max(1, min(heads_per_call, hpg))
    rep = SeqReport(w.batch, w.nheads)
    init = cpu_inputs["init_state"]
    for b in range(w.batch):
        for g in range(w.ngroups):
            for h0 in range(g * hpg, (g + 1) * hpg, step):
                h1 = min(h0 + step, (g + 1) * hpg)
                sl = dict(x=cpu_inputs["x"][b:b + 1, :, h0:h1], dt=cpu_inputs["dt"][b:b + 1, :, h0:h1],
                          A=cpu_inputs["A"][h0:h1], B=cpu_inputs["B"][b:b + 1, :, g:g + 1],
                          C=cpu_inputs["C"][b:b + 1, :, g:g + 1], D=cpu_inputs["D"][h0:h1],
                          init_state=None if init is None else init[b:b + 1, h0:h1])
                y_ref, f_ref = oracle_fwd(sl)
                fg = None if fin_gpu is None else np64(fin_gpu[b:b + 1, h0:h1])
                rep.add(b, h0, np64(y_gpu[b:b + 1, :, h0:h1, :]), y_ref, fg, f_ref)
    return rep


def assert_every_sequence(w, rep, tol=None, label="fwd"):
    """Whole-tensor and per-sequence bounds, with the worst sequence logged."""
    tol = TOL[w.dtype] if tol is None else tol
    wy, wf = rep.whole()
    (sy, iy), (sf, jf) = rep.worst()
    say(f"    [{label}] whole rel_l2 y={wy:.3e} final={wf:.3e}; worst sequence y={sy:.3e} "
        f"at (b,h)={iy}, final={sf:.3e} at (b,h)={jf}")
    assert wy <= tol and wf <= tol, (wy, wf)
    assert sy <= tol, f"y of sequence (b,h)={iy}: rel_l2 {sy:.3e} > {tol}"
    assert sf <= tol, f"final state of sequence (b,h)={jf}: rel_l2 {sf:.3e} > {tol}"
