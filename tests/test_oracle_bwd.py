"""Pins for the fp64 backward oracle (CPU only).

oracle.ssd_bwd_ref differentiates the token recurrence by hand, step by step in reverse.
Nothing here trusts that derivation: it is compared with
  * central finite differences of the forward oracle (itself pinned in test_oracle.py),
  * torch autograd through an independent implementation of the quadratic (dual) form
    y = (L o C B^T)(dt x) + ..., written below from the same definition,
  * closed forms for the constant-decay scalar case,
  * consistency of the per-chunk boundary gradients with gradients of suffix runs,
and a mutation test plants plausible mistakes in the backward's source and checks that
the pins catch every one of them.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import oracle
from oracle import build as oracle_build

INPUTS = ("x", "dt", "A", "B", "C", "D", "init_state")
GRAD_OF = {"x": "dx", "dt": "ddt", "A": "dA", "B": "dB", "C": "dC", "D": "dD",
           "init_state": "d_init"}


def _rand_case(rng, bsz, T, H, P, N, G, with_init=True, a_range=(0.05, 2.0)):
    x = rng.standard_normal((bsz, T, H, P))
    dt = np.log1p(np.exp(rng.standard_normal((bsz, T, H)) - 1.0))
    A = -rng.uniform(*a_range, size=H)
    B = rng.standard_normal((bsz, T, G, N)) / np.sqrt(N)
    C = rng.standard_normal((bsz, T, G, N)) / np.sqrt(N)
    D = rng.standard_normal(H)
    init = rng.standard_normal((bsz, H, N, P)) * 0.3 if with_init else None
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=D, init_state=init)


def _loss(inp, Wy, Wf, lib=None):
    y, f, _ = oracle.ssd_ref(**inp, lib=lib)
    return float((y * Wy).sum() + (f * Wf).sum())


def _fd_grads(inp, Wy, Wf, eps=1e-6, sample=None, rng=None, lib=None):
    """Central differences of L = <y, Wy> + <final, Wf> for every (or a sample of the)
    entries of every input.  Returns {input name: (flat indices, derivative values)}."""
    out = {}
    for k in INPUTS:
        v = inp[k]
        if v is None:
            continue
        n = v.size
        idx = np.arange(n) if sample is None or n <= sample else rng.choice(n, sample, replace=False)
        vals = []
        for i in idx:
            plus, minus = v.copy().ravel(), v.copy().ravel()
            plus[i] += eps
            minus[i] -= eps
            lp = _loss(dict(inp, **{k: plus.reshape(v.shape)}), Wy, Wf, lib)
            lm = _loss(dict(inp, **{k: minus.reshape(v.shape)}), Wy, Wf, lib)
            vals.append((lp - lm) / (2 * eps))
        out[k] = (idx, np.array(vals))
    return out


def _check_against_fd(inp, d_final_given=True, sample=None, seed=0, lib=None, tol=2e-7):
    rng = np.random.default_rng(seed)
    bsz, T, H, P = inp["x"].shape
    N = inp["B"].shape[3]
    Wy = rng.standard_normal((bsz, T, H, P))
    Wf = rng.standard_normal((bsz, H, N, P)) if d_final_given else np.zeros((bsz, H, N, P))
    g = oracle.ssd_bwd_ref(**inp, dy=Wy, d_final=Wf if d_final_given else None, lib=lib)
    fd = _fd_grads(inp, Wy, Wf, sample=sample, rng=rng, lib=lib)
    worst = 0.0
    for k, (idx, vals) in fd.items():
        got = g[GRAD_OF[k]].ravel()[idx]
        scale = max(1.0, np.abs(vals).max())
        worst = max(worst, np.abs(got - vals).max() / scale)
    return worst


# ---------------------------------------------------------------- finite differences

FD_CASES = [
    # (batch, T, H, P, N, G, init, d_final)
    (1, 1, 1, 1, 1, 1, False, False),
    (1, 4, 1, 1, 2, 1, True, True),
    (2, 7, 2, 3, 2, 1, True, True),
    (1, 9, 4, 2, 3, 2, True, False),
    (2, 6, 3, 2, 2, 3, False, True),
]


@pytest.mark.parametrize("case", FD_CASES)
def test_gradients_match_finite_differences(case):
    bsz, T, H, P, N, G, wi, wf = case
    inp = _rand_case(np.random.default_rng(200 + T * 3 + H), bsz, T, H, P, N, G, wi)
    assert _check_against_fd(inp, d_final_given=wf, seed=T) < 2e-7


def test_gradients_across_recompute_segments():
    """T longer than the oracle's recompute segment (64 steps): sampled entries."""
    inp = _rand_case(np.random.default_rng(201), 1, 150, 2, 2, 2, 1, True, a_range=(0.01, 0.1))
    assert _check_against_fd(inp, sample=25, seed=5) < 2e-7


# ---------------------------------------------------------------- autograd of the dual form

def _torch_quadratic(x, dt, A, B, C, D, init):
    """y and final state by the quadratic form, differentiable (torch fp64, CPU).

    L[t, s] = exp(cs_t - cs_s) for s <= t (cs the inclusive prefix sum of dt*A), the
    masked-and-decayed C B^T acting on dt-scaled inputs, plus the decayed init state read
    by C and the D skip; final = sum_s exp(cs_T-1 - cs_s) dt_s B_s x_s^T + exp(cs_T-1) init.
    """
    bsz, T, H, P = x.shape
    G = B.shape[2]
    hpg = H // G
    Bh = B.repeat_interleave(hpg, dim=2)                      # [b, T, H, N]
    Ch = C.repeat_interleave(hpg, dim=2)
    cs = torch.cumsum(dt * A, dim=1)                          # [b, T, H]
    seg = cs[:, :, None, :] - cs[:, None, :, :]               # [b, t, s, H]
    causal = torch.tril(torch.ones(T, T, dtype=torch.bool))[None, :, :, None]
    L = torch.exp(torch.where(causal, seg, torch.full_like(seg, -torch.inf)))
    CB = torch.einsum("bthn,bshn->btsh", Ch, Bh)
    u = dt[..., None] * x
    y = torch.einsum("btsh,bshp->bthp", L * CB, u) + D[None, None, :, None] * x
    wlast = torch.exp(cs[:, -1:, :] - cs)                     # [b, T, H]
    final = torch.einsum("bsh,bshn,bshp->bhnp", wlast, Bh, u)
    if init is not None:
        y = y + torch.exp(cs)[..., None] * torch.einsum("bthn,bhnp->bthp", Ch, init)
        final = final + torch.exp(cs[:, -1])[..., None, None] * init
    return y, final


AG_CASES = [
    (1, 16, 2, 3, 4, 1, True),
    (2, 23, 4, 2, 3, 2, True),
    (1, 31, 3, 4, 2, 3, False),
    (1, 70, 2, 2, 3, 1, True),
]


@pytest.mark.parametrize("case", AG_CASES)
def test_gradients_match_autograd_of_quadratic_form(case):
    bsz, T, H, P, N, G, wi = case
    rng = np.random.default_rng(300 + T)
    inp = _rand_case(rng, bsz, T, H, P, N, G, wi)
    dy = rng.standard_normal((bsz, T, H, P))
    dfin = rng.standard_normal((bsz, H, N, P))
    g = oracle.ssd_bwd_ref(**inp, dy=dy, d_final=dfin)
    tens = {k: (None if v is None else torch.tensor(v, dtype=torch.float64, requires_grad=True))
            for k, v in inp.items()}
    y, fin = _torch_quadratic(*(tens[k] for k in INPUTS))
    ((y * torch.tensor(dy)).sum() + (fin * torch.tensor(dfin)).sum()).backward()
    for k in INPUTS:
        if tens[k] is None:
            continue
        ref = tens[k].grad.numpy()
        got = g[GRAD_OF[k]]
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-11 * max(1.0, np.abs(ref).max()),
                                   err_msg=k)


# ---------------------------------------------------------------- closed forms

def test_constant_decay_closed_forms():
    """N = P = 1, x = B = C = 1, D = 0, constant step d and A, a zero init state, and the
    loss L = y_{T-1} = d * sum_{m<T} a^m with a = exp(d A).  Then
      dL/dx_s = d a^(T-1-s),  dL/dA = d^2 sum_m m a^m,
      sum_t dL/ddt_t = d/dd [d sum_m exp(m d A)] = sum_m a^m (1 + m d A),
    and the init-state gradient is C a^T = a^T."""
    T, d, Av = 40, 0.3, -0.25
    one = np.ones((1, T, 1, 1))
    dy = np.zeros((1, T, 1, 1))
    dy[0, -1] = 1.0
    g = oracle.ssd_bwd_ref(one, np.full((1, T, 1), d), np.array([Av]), one, one, np.zeros(1),
                           dy=dy, init_state=np.zeros((1, 1, 1, 1)))
    a = np.exp(d * Av)
    m = np.arange(T)
    np.testing.assert_allclose(g["dx"].reshape(T), d * a ** (T - 1 - m), rtol=1e-13)
    np.testing.assert_allclose(g["dA"][0], d * d * np.sum(m * a ** m), rtol=1e-12)
    np.testing.assert_allclose(g["ddt"].sum(), np.sum(a ** m * (1 + m * d * Av)), rtol=1e-12)
    np.testing.assert_allclose(g["d_init"].reshape(()), a ** T, rtol=1e-13)
    np.testing.assert_allclose(g["dD"][0], 1.0, rtol=0, atol=0)   # <x_{T-1}, dy_{T-1}>


def test_no_decay_gradients():
    """A = 0 (a = 1): y_t = C_t^T (init + sum_{s<=t} dt_s B_s x_s^T) + D x_t, so with
    Lam_s = sum_{t>=s} C_t dy_t^T + d_final (a reverse cumulative sum):
    dx_s = D dy_s + dt_s Lam_s^T B_s and ddt_s = B_s^T Lam_s x_s exactly."""
    rng = np.random.default_rng(17)
    inp = _rand_case(rng, 1, 21, 1, 3, 4, 1, True)
    inp["A"] = np.zeros(1)
    dy = rng.standard_normal(inp["x"].shape)
    dfin = rng.standard_normal((1, 1, 4, 3))
    g = oracle.ssd_bwd_ref(**inp, dy=dy, d_final=dfin)
    outer = np.einsum("tn,tp->tnp", inp["C"][0, :, 0], dy[0, :, 0])
    Lam = np.cumsum(outer[::-1], axis=0)[::-1] + dfin[0, 0]
    x, dt, B = inp["x"][0, :, 0], inp["dt"][0, :, 0], inp["B"][0, :, 0]
    dx = inp["D"][0] * dy[0, :, 0] + dt[:, None] * np.einsum("tn,tnp->tp", B, Lam)
    np.testing.assert_allclose(g["dx"][0, :, 0], dx, rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["ddt"][0, :, 0], np.einsum("tn,tnp,tp->t", B, Lam, x),
                               rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["d_init"][0, 0], Lam[0], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- chunk-level records

def test_boundary_grads_are_suffix_init_gradients():
    """boundary_grads[c] = dL/d(state after chunk c) through the later steps: the init
    gradient of the run over the steps after chunk c, started from that state."""
    rng = np.random.default_rng(18)
    inp = _rand_case(rng, 2, 29, 2, 3, 2, 1, True, a_range=(0.01, 0.2))
    dy = rng.standard_normal(inp["x"].shape)
    dfin = rng.standard_normal((2, 2, 2, 3))
    Q = 8
    g = oracle.ssd_bwd_ref(**inp, dy=dy, d_final=dfin, chunk_len=Q)
    bg = g["boundary_grads"]
    assert bg.shape == (2, 2, 4, 2, 3)
    np.testing.assert_array_equal(bg[:, :, -1], dfin)
    _, _, bound = oracle.ssd_ref(**inp, chunk_len=Q)
    for c in range(3):
        s0 = (c + 1) * Q
        suf = {k: (v[:, s0:] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
        suf["init_state"] = bound[:, :, c]
        gs = oracle.ssd_bwd_ref(**suf, dy=dy[:, s0:], d_final=dfin)
        np.testing.assert_allclose(bg[:, :, c], gs["d_init"], rtol=0, atol=1e-13)


def test_group_gradients_sum_head_shares():
    """G = 1 versus G = H with B and C replicated: the shared B/C gradient is the sum of
    the per-group ones, and every other gradient is unchanged."""
    rng = np.random.default_rng(19)
    inp = _rand_case(rng, 1, 17, 3, 2, 4, 1, True)
    dy = rng.standard_normal(inp["x"].shape)
    g1 = oracle.ssd_bwd_ref(**inp, dy=dy)
    rep = dict(inp, B=np.repeat(inp["B"], 3, axis=2), C=np.repeat(inp["C"], 3, axis=2))
    g3 = oracle.ssd_bwd_ref(**rep, dy=dy)
    np.testing.assert_allclose(g1["dB"][:, :, 0], g3["dB"].sum(axis=2), rtol=0, atol=1e-13)
    np.testing.assert_allclose(g1["dC"][:, :, 0], g3["dC"].sum(axis=2), rtol=0, atol=1e-13)
    for k in ("dx", "ddt", "dA", "dD", "d_init"):
        np.testing.assert_allclose(g1[k], g3[k], rtol=0, atol=1e-13, err_msg=k)


def test_gradients_linear_in_upstream_and_thread_independent():
    rng = np.random.default_rng(20)
    inp = _rand_case(rng, 2, 19, 2, 2, 3, 1, True)
    d1, d2 = rng.standard_normal(inp["x"].shape), rng.standard_normal(inp["x"].shape)
    f1, f2 = rng.standard_normal((2, 2, 3, 2)), rng.standard_normal((2, 2, 3, 2))
    ga = oracle.ssd_bwd_ref(**inp, dy=d1, d_final=f1, nthreads=1)
    gb = oracle.ssd_bwd_ref(**inp, dy=d2, d_final=f2, nthreads=3)
    gc = oracle.ssd_bwd_ref(**inp, dy=0.5 * d1 - 2 * d2, d_final=0.5 * f1 - 2 * f2, nthreads=4)
    for k in ("dx", "ddt", "dA", "dB", "dC", "dD", "d_init"):
        np.testing.assert_allclose(gc[k], 0.5 * ga[k] - 2 * gb[k], rtol=0, atol=1e-12, err_msg=k)
    ga2 = oracle.ssd_bwd_ref(**inp, dy=d1, d_final=f1, nthreads=5)
    for k in ("dx", "ddt", "dA", "dB", "dC", "dD", "d_init"):
        np.testing.assert_array_equal(ga[k], ga2[k])


def test_bwd_error_codes():
    rng = np.random.default_rng(21)
    inp = _rand_case(rng, 1, 4, 2, 2, 2, 1, False)
    with pytest.raises(ValueError):
        oracle.ssd_bwd_ref(**inp, dy=np.zeros((1, 4, 2, 3)))
    with pytest.raises(ValueError):
        oracle.ssd_bwd_ref(**inp, dy=np.zeros((1, 4, 2, 2)), d_final=np.zeros((1, 2, 2, 3)))


# ---------------------------------------------------------------- the pins have teeth

BWD_MUTANTS = {
    "ddt_without_decay_term": ("j->ddt[(b * T + t) * H + h] = direct + Ah * a * q;",
                               "j->ddt[(b * T + t) * H + h] = direct;"),
    "dA_without_dt": ("dA_acc += dtt * a * q;", "dA_acc += a * q;"),
    "dx_without_skip": ("dxt[p] = Dh * dyt[p] + dtt * acc;", "dxt[p] = dtt * acc;"),
    "dB_without_dt": ("dBt[n] = dtt * u;", "dBt[n] = u;"),
    "dC_from_previous_state": ("acc += S_t[n * P + p] * dyt[p];",
                               "acc += S_prev[n * P + p] * dyt[p];"),
    "q_with_current_state": ("q += S_prev[k] * Lam[k];", "q += S_t[k] * Lam[k];"),
    "lam_transposed": ("acc += Bt[n] * Lam[n * P + p];",
                       "acc += Bt[n] * Lam[(p * N + n) % (N * P)];"),
    "recompute_wrong_decay": ("step_state(nxt, exp(DTT(t) * Ah),", "step_state(nxt, exp(DTT(t) * Ah * 0.5),"),
    "checkpoint_off_by_one": ("if (t % kSeg == 0)", "if (t % kSeg == 1)"),
    "ignore_d_final": ("if (j->d_final)\n        memcpy(Lam", "if (0)\n        memcpy(Lam"),
    "boundary_record_shifted": ("t % j->chunk_len == j->chunk_len - 1", "t % j->chunk_len == 0"),
    "no_decay_of_lam": ("Lam[k] *= a;", "Lam[k] *= 1.0;"),
}


def _bwd_pins_pass(lib):
    ok = True
    rng = np.random.default_rng(77)
    inp = _rand_case(rng, 1, 6, 2, 2, 2, 1, True)
    ok &= _check_against_fd(inp, d_final_given=True, seed=1, lib=lib) < 2e-7
    long_case = _rand_case(rng, 1, 70, 1, 1, 2, 1, True, a_range=(0.01, 0.1))
    ok &= _check_against_fd(long_case, d_final_given=True, sample=12, seed=2, lib=lib) < 2e-7
    # the boundary record against the suffix-run init gradient
    c = _rand_case(rng, 1, 12, 1, 2, 2, 1, True, a_range=(0.01, 0.2))
    dy = rng.standard_normal(c["x"].shape)
    dfin = rng.standard_normal((1, 1, 2, 2))
    g = oracle.ssd_bwd_ref(**c, dy=dy, d_final=dfin, chunk_len=4, lib=lib)
    _, _, bound = oracle.ssd_ref(**c, chunk_len=4, lib=lib)
    suf = {k: (v[:, 4:] if k in ("x", "dt", "B", "C") else v) for k, v in c.items()}
    suf["init_state"] = bound[:, :, 0]
    gs = oracle.ssd_bwd_ref(**suf, dy=dy[:, 4:], d_final=dfin, lib=lib)
    ok &= np.allclose(g["boundary_grads"][:, :, 0], gs["d_init"], atol=1e-12)
    return bool(ok)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_bwd_pins_reject_planted_mistakes():
    src = open(oracle_build.SOURCE).read()
    assert _bwd_pins_pass(oracle.library())
    with tempfile.TemporaryDirectory() as tmp:
        shutil.copy(os.path.join(os.path.dirname(oracle_build.SOURCE), "ssd_oracle.h"), tmp)
        for name, (old, new) in BWD_MUTANTS.items():
            assert src.count(old) == 1, f"mutation site for {name} not unique"
            path = os.path.join(tmp, f"m_{name}.c")
            with open(path, "w") as f:
                f.write(src.replace(old, new))
            out = os.path.join(tmp, f"m_{name}.so")
            subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-I", tmp, path, "-o", out,
                            "-lm", "-lpthread"], check=True, capture_output=True)
            lib = oracle.load_library(out)
            assert not _bwd_pins_pass(lib), f"no pin catches the planted mistake '{name}'"


def test_chunk_entry_grads_compose_to_boundary_grads():
    """The reverse inter-chunk carry: with Z_c the entry-state gradient through chunk c's
    own outputs and F_c the boundary gradient after chunk c,
    F_{c-1} = Z_c + exp(sum of dt*A over chunk c) F_c, and d_init = Z_0 + exp(..) F_0."""
    rng = np.random.default_rng(22)
    inp = _rand_case(rng, 1, 27, 2, 3, 2, 1, True, a_range=(0.01, 0.2))
    dy = rng.standard_normal(inp["x"].shape)
    dfin = rng.standard_normal((1, 2, 2, 3))
    Q = 8
    Z = oracle.chunk_entry_grads(**inp, dy=dy, chunk_len=Q)
    g = oracle.ssd_bwd_ref(**inp, dy=dy, d_final=dfin, chunk_len=Q)
    F = g["boundary_grads"]
    cs = oracle.chunk_cumsum(inp["dt"], inp["A"], Q)
    for c in range(4):
        carried = Z[:, :, c] + np.exp(cs[:, :, c, -1])[..., None, None] * F[:, :, c]
        want = F[:, :, c - 1] if c > 0 else g["d_init"]
        np.testing.assert_allclose(carried, want, rtol=0, atol=1e-12)
    # and Z_c is the chunk's exp(cs)-weighted C^T dy contraction (stage-2 mirror)
    C, x = inp["C"], inp["x"]
    for c in range(4):
        sl = slice(c * Q, min(27, (c + 1) * Q))
        w = np.exp(cs[:, :, c, : sl.stop - sl.start])            # [b, h, steps]
        zc = np.einsum("bht,btn,bthp->bhnp", w, C[:, sl, 0], dy[:, sl])
        np.testing.assert_allclose(Z[:, :, c], zc, rtol=0, atol=1e-12)
