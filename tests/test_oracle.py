"""Pins for the fp64 oracle (CPU only).

The oracle is the token-by-token recurrence.  Every check here compares it with
something it does not contain: numbers printed on the pages, the independent quadratic
(dual) form, closed forms for special cases, and invariants of a linear causal map.
A mutation test at the end plants plausible mistakes in the oracle's source and checks
that at least one pin catches each of them.
"""
import os
import re
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from oracle import build as oracle_build
from oracle.quadratic import one_ss_mask, ssd_quadratic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "four_token_example.txt")


def _read_golden():
    vals = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split(None, 1)
            rows = [[float(v) for v in r.split()] for r in rest.split("|")]
            vals[key] = np.array(rows if len(rows) > 1 else rows[0])
    return vals


def _example_as_ssd():
    """The page's example in this API's terms: A=-1 and dt_t = -ln a_t give
    exp(dt_t*A) = a_t; x'_t = x_t / dt_t makes the scaled input dt_t*x'_t equal x_t."""
    g = _read_golden()
    a, x = g["a"], g["x"]
    dt = -np.log(a)
    inputs = dict(x=(x / dt).reshape(1, 4, 1, 1), dt=dt.reshape(1, 4, 1), A=np.array([-1.0]),
                  B=g["B"].reshape(1, 4, 1, 2), C=g["C"].reshape(1, 4, 1, 2), D=np.array([0.0]))
    return g, inputs


def _rand_case(rng, bsz, T, H, P, N, G, with_init, a_range=(0.05, 2.0)):
    x = rng.standard_normal((bsz, T, H, P))
    dt = np.log1p(np.exp(rng.standard_normal((bsz, T, H)) - 1.0))
    A = -rng.uniform(*a_range, size=H)
    B = rng.standard_normal((bsz, T, G, N)) / np.sqrt(N)
    C = rng.standard_normal((bsz, T, G, N)) / np.sqrt(N)
    D = rng.standard_normal(H)
    init = rng.standard_normal((bsz, H, N, P)) * 0.3 if with_init else None
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=D, init_state=init)


# ---------------------------------------------------------------- printed example

def test_worked_example_recurrence_matches_printed_output():
    g, inp = _example_as_ssd()
    y, final, _ = oracle.ssd_ref(**inp)
    np.testing.assert_allclose(y.reshape(4), g["y_recurrence"], rtol=0, atol=1e-12)
    # the state after the last token, worked out by hand from the same recurrence:
    # h3 = 0.7 * [3.4, 4.6] + [1, -1] * 4
    np.testing.assert_allclose(final.reshape(2), [6.38, -0.78], rtol=0, atol=1e-12)


def test_worked_example_mask_and_matrix_form():
    g, inp = _example_as_ssd()
    L = one_ss_mask(g["a"])
    np.testing.assert_allclose(L, g["L"], rtol=0, atol=1e-12)
    # in terms of this API the mask is built from exp(dt*A)
    L2 = one_ss_mask(np.exp(inp["dt"].reshape(4) * -1.0))
    np.testing.assert_allclose(L2, g["L"], rtol=0, atol=1e-12)
    y, _ = ssd_quadratic(**inp)
    np.testing.assert_allclose(y.reshape(4), g["y_matrix"], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- dual forms agree

CASES = [
    # (batch, T, H, P, N, G, init)
    (1, 1, 1, 1, 1, 1, False),
    (1, 5, 1, 3, 2, 1, True),
    (2, 37, 2, 4, 3, 1, True),
    (1, 24, 4, 2, 8, 2, True),
    (2, 16, 4, 3, 5, 4, False),
    (1, 64, 3, 8, 8, 3, True),
]


@pytest.mark.parametrize("case", CASES)
def test_recurrence_equals_quadratic_form(case):
    bsz, T, H, P, N, G, with_init = case
    rng = np.random.default_rng(1000 + T * 7 + N)
    inp = _rand_case(rng, bsz, T, H, P, N, G, with_init)
    y_r, f_r, _ = oracle.ssd_ref(**inp)
    y_q, f_q = ssd_quadratic(**inp)
    scale = max(1.0, np.abs(y_q).max())
    np.testing.assert_allclose(y_r, y_q, rtol=0, atol=1e-12 * scale)
    np.testing.assert_allclose(f_r, f_q, rtol=0, atol=1e-12 * max(1.0, np.abs(f_q).max()))


# ---------------------------------------------------------------- closed forms

def test_no_decay_is_causal_linear_attention():
    """A = 0 gives a = 1: the state is init + a running sum of dt B x^T (cumsum)."""
    rng = np.random.default_rng(3)
    inp = _rand_case(rng, 2, 33, 2, 3, 4, 1, True)
    inp["A"] = np.zeros(2)
    y, final, _ = oracle.ssd_ref(**inp)
    x, dt, B, C, D, s0 = (inp[k] for k in ("x", "dt", "B", "C", "D", "init_state"))
    outer = np.einsum("btn,bthp->bthnp", B[:, :, 0], dt[..., None] * x)
    S = np.cumsum(outer, axis=1) + s0[:, None]
    y_cf = np.einsum("btn,bthnp->bthp", C[:, :, 0], S) + D[None, None, :, None] * x
    np.testing.assert_allclose(y, y_cf, rtol=0, atol=1e-12)
    np.testing.assert_allclose(final, S[:, -1], rtol=0, atol=1e-12)


def test_zero_step_keeps_init_state():
    """dt = 0: no decay and no input, so y_t = C_t^T init + D x_t and final = init."""
    rng = np.random.default_rng(4)
    inp = _rand_case(rng, 1, 20, 2, 3, 4, 2, True)
    inp["dt"] = np.zeros_like(inp["dt"])
    y, final, _ = oracle.ssd_ref(**inp)
    x, C, D, s0 = inp["x"], inp["C"], inp["D"], inp["init_state"]
    y_cf = np.einsum("btn,bhnp->bthp", C[:, :, 0], s0) + D[None, None, :, None] * x
    y_cf[:, :, 1] = np.einsum("btn,bnp->btp", C[:, :, 1], s0[:, 1]) + D[1] * x[:, :, 1]
    np.testing.assert_allclose(y, y_cf, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(final, s0)
    # a tiny step moves the result by O(dt)
    inp["dt"] = np.full_like(inp["dt"], 1e-9)
    y2, f2, _ = oracle.ssd_ref(**inp)
    assert 0 < np.abs(y2 - y).max() < 1e-7
    assert 0 < np.abs(f2 - final).max() < 1e-7


def test_single_input_gives_cumulative_product():
    """N = P = 1, B = C = 1, D = 0, and input only at t = 0 with dt_0 x_0 = 1:
    y_t = a_1 a_2 ... a_t (the 1-SS 'cumprod' case)."""
    T = 12
    rng = np.random.default_rng(5)
    dt = rng.uniform(0.1, 1.0, size=(1, T, 1))
    A = np.array([-0.7])
    x = np.zeros((1, T, 1, 1))
    x[0, 0, 0, 0] = 1.0 / dt[0, 0, 0]
    one = np.ones((1, T, 1, 1))
    y, _, _ = oracle.ssd_ref(x, dt, A, one, one, np.zeros(1))
    a = np.exp(dt[0, :, 0] * A[0])
    expect = np.array([np.prod(a[1:t + 1]) for t in range(T)])
    np.testing.assert_allclose(y.reshape(T), expect, rtol=1e-13, atol=0)


def test_unit_decay_gives_cumulative_sum():
    """a = 1 with N = P = 1 and B = C = 1: y = cumsum(dt * x)."""
    T = 40
    rng = np.random.default_rng(6)
    dt = rng.uniform(0.0, 1.0, size=(1, T, 1))
    x = rng.standard_normal((1, T, 1, 1))
    one = np.ones((1, T, 1, 1))
    y, _, _ = oracle.ssd_ref(x, dt, np.zeros(1), one, one, np.zeros(1))
    np.testing.assert_allclose(y.reshape(T), np.cumsum(dt.reshape(T) * x.reshape(T)),
                               rtol=1e-13, atol=1e-14)


def test_constant_decay_gives_geometric_series():
    """Constant dt and A (a RetNet-style fixed decay gamma = exp(dt*A)) with x = B = C = 1:
    y_t = dt * (1 - gamma^(t+1)) / (1 - gamma)."""
    T, dtv, Av = 50, 0.3, -0.4
    one = np.ones((1, T, 1, 1))
    y, final, _ = oracle.ssd_ref(one, np.full((1, T, 1), dtv), np.array([Av]), one, one,
                                 np.zeros(1))
    gam = np.exp(dtv * Av)
    t = np.arange(T)
    np.testing.assert_allclose(y.reshape(T), dtv * (1 - gam ** (t + 1)) / (1 - gam), rtol=1e-13)
    np.testing.assert_allclose(final.reshape(()), dtv * (1 - gam ** T) / (1 - gam), rtol=1e-13)


# ---------------------------------------------------------------- invariants

def test_linear_in_input_and_init_state():
    rng = np.random.default_rng(7)
    i1 = _rand_case(rng, 1, 30, 2, 3, 4, 1, True)
    i2 = dict(i1, x=rng.standard_normal(i1["x"].shape),
              init_state=rng.standard_normal(i1["init_state"].shape))
    al, be = 0.7, -1.9
    y1, f1, _ = oracle.ssd_ref(**i1)
    y2, f2, _ = oracle.ssd_ref(**i2)
    i3 = dict(i1, x=al * i1["x"] + be * i2["x"],
              init_state=al * i1["init_state"] + be * i2["init_state"])
    y3, f3, _ = oracle.ssd_ref(**i3)
    np.testing.assert_allclose(y3, al * y1 + be * y2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(f3, al * f1 + be * f2, rtol=0, atol=1e-12)


def test_causal():
    rng = np.random.default_rng(8)
    inp = _rand_case(rng, 1, 30, 2, 3, 4, 1, True)
    y0, _, _ = oracle.ssd_ref(**inp)
    t0 = 17
    for key in ("x", "dt", "B", "C"):
        pert = dict(inp)
        arr = inp[key].copy()
        arr[:, t0] += 0.5
        pert[key] = arr
        y1, _, _ = oracle.ssd_ref(**pert)
        np.testing.assert_array_equal(y1[:, :t0], y0[:, :t0])
        assert np.abs(y1[:, t0] - y0[:, t0]).max() > 1e-6


def test_groups_replicated_equal_single_group():
    rng = np.random.default_rng(9)
    inp = _rand_case(rng, 2, 25, 4, 3, 5, 1, True)
    y1, f1, _ = oracle.ssd_ref(**inp)
    rep = dict(inp, B=np.repeat(inp["B"], 4, axis=2), C=np.repeat(inp["C"], 4, axis=2))
    y4, f4, _ = oracle.ssd_ref(**rep)
    np.testing.assert_array_equal(y1, y4)
    np.testing.assert_array_equal(f1, f4)
    # heads 0,1 -> group 0 and 2,3 -> group 1 when G = 2
    two = dict(inp, B=np.concatenate([inp["B"], rng.standard_normal(inp["B"].shape)], axis=2),
               C=np.concatenate([inp["C"], rng.standard_normal(inp["C"].shape)], axis=2))
    y2, _, _ = oracle.ssd_ref(**two)
    np.testing.assert_array_equal(y2[:, :, :2], y1[:, :, :2])
    assert np.abs(y2[:, :, 2:] - y1[:, :, 2:]).max() > 1e-3


def test_split_run_equals_full_run():
    """Resume from a state: run [0, T1), then [T1, T) starting from its final state."""
    rng = np.random.default_rng(10)
    inp = _rand_case(rng, 2, 41, 2, 3, 4, 2, True, a_range=(0.01, 0.1))
    y, f, _ = oracle.ssd_ref(**inp)
    T1 = 19
    first = {k: (v[:, :T1] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    ya, fa, _ = oracle.ssd_ref(**first)
    second = {k: (v[:, T1:] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    second["init_state"] = fa
    yb, fb, _ = oracle.ssd_ref(**second)
    np.testing.assert_allclose(np.concatenate([ya, yb], axis=1), y, rtol=0, atol=1e-13)
    np.testing.assert_allclose(fb, f, rtol=0, atol=1e-13)


def test_batch_and_head_permutation_equivariance():
    rng = np.random.default_rng(11)
    inp = _rand_case(rng, 3, 15, 3, 2, 3, 3, True)
    y, f, _ = oracle.ssd_ref(**inp)
    pb = np.array([2, 0, 1])
    perm = {k: (v[pb] if k in ("x", "dt", "B", "C", "init_state") else v) for k, v in inp.items()}
    yp, fp, _ = oracle.ssd_ref(**perm)
    np.testing.assert_array_equal(yp, y[pb])
    np.testing.assert_array_equal(fp, f[pb])
    ph = np.array([1, 2, 0])   # G == H, so heads and groups permute together
    perm = dict(inp, x=inp["x"][:, :, ph], dt=inp["dt"][:, :, ph], A=inp["A"][ph],
                D=inp["D"][ph], B=inp["B"][:, :, ph], C=inp["C"][:, :, ph],
                init_state=inp["init_state"][:, ph])
    yp, fp, _ = oracle.ssd_ref(**perm)
    np.testing.assert_array_equal(yp, y[:, :, ph])
    np.testing.assert_array_equal(fp, f[:, ph])


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(12)
    inp = _rand_case(rng, 2, 40, 3, 4, 5, 1, True)
    a = oracle.ssd_ref(**inp, chunk_len=16, nthreads=1)
    b = oracle.ssd_ref(**inp, chunk_len=16, nthreads=5)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


# ---------------------------------------------------------------- chunk-level helpers

def test_boundary_states_are_prefix_final_states():
    rng = np.random.default_rng(13)
    inp = _rand_case(rng, 1, 23, 2, 2, 3, 1, True, a_range=(0.01, 0.2))
    Q = 8
    _, _, bound = oracle.ssd_ref(**inp, chunk_len=Q)
    assert bound.shape[2] == 3
    for c, end in enumerate((8, 16, 23)):
        pre = {k: (v[:, :end] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
        _, fq = ssd_quadratic(**pre)
        np.testing.assert_allclose(bound[:, :, c], fq, rtol=0, atol=1e-13)


def test_chunk_cumsum_is_chunk_local_prefix_sum():
    rng = np.random.default_rng(14)
    dt = rng.uniform(0, 1, size=(2, 21, 3))
    A = -rng.uniform(0.1, 2, size=3)
    cs = oracle.chunk_cumsum(dt, A, 8)
    assert cs.shape == (2, 3, 3, 8)
    for b in range(2):
        for h in range(3):
            for c in range(3):
                run = 0.0
                for i in range(8):
                    t = c * 8 + i
                    if t < 21:
                        run += dt[b, t, h] * A[h]
                    assert cs[b, h, c, i] == pytest.approx(run, abs=1e-14)


def test_chunk_and_entry_states_compose_to_the_final_state():
    """Stages 2 and 3: entry_{c+1} = exp(sum of dt*A over chunk c) * entry_c + S_c,
    with S_c from the chunk alone (zero start), checked against the quadratic form."""
    rng = np.random.default_rng(15)
    inp = _rand_case(rng, 1, 29, 2, 3, 4, 1, True, a_range=(0.01, 0.2))
    Q = 8
    S = oracle.chunk_states(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], Q)
    ent, final = oracle.entry_states(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                                     inp["D"], Q, init_state=inp["init_state"])
    cs = oracle.chunk_cumsum(inp["dt"], inp["A"], Q)
    for c in range(S.shape[2]):
        sl = slice(c * Q, min(29, (c + 1) * Q))
        part = {k: (v[:, sl] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
        part["init_state"] = None
        _, fq = ssd_quadratic(**part)
        np.testing.assert_allclose(S[:, :, c], fq, rtol=0, atol=1e-13)
        nxt = np.exp(cs[:, :, c, -1])[..., None, None] * ent[:, :, c] + S[:, :, c]
        if c + 1 < S.shape[2]:
            np.testing.assert_allclose(ent[:, :, c + 1], nxt, rtol=0, atol=1e-13)
        else:
            np.testing.assert_allclose(final, nxt, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(ent[:, :, 0], inp["init_state"])


def test_error_codes():
    rng = np.random.default_rng(16)
    inp = _rand_case(rng, 1, 4, 3, 2, 2, 1, False)
    with pytest.raises(ValueError):
        oracle.ssd_ref(**dict(inp, A=np.zeros(2)))
    bad = dict(inp, B=np.zeros((1, 4, 2, 2)), C=np.zeros((1, 4, 2, 2)))   # 3 heads, 2 groups
    with pytest.raises(RuntimeError):
        oracle.ssd_ref(**bad)


# ---------------------------------------------------------------- the pins have teeth

MUTANTS = {
    "drop_skip": ("yt[p] = acc + j->D[h] * xt[p];", "yt[p] = acc;"),
    "decay_sign": ("exp(dt * j->A[h])", "exp(-dt * j->A[h])"),
    "no_input_scale": ("const double wb = dt * Bt[n];", "const double wb = Bt[n];"),
    "read_with_B": ("acc += Ct[n] * S[n * P + p];", "acc += Bt[n] * S[n * P + p];"),
    "transposed_read": ("acc += Ct[n] * S[n * P + p];", "acc += Ct[n] * S[(p * N + n) % (N * P)];"),
    "decay_after_input": ("Sn[p] = a * Sn[p] + wb * xt[p];", "Sn[p] = a * (Sn[p] + wb * xt[p]);"),
    "wrong_group": ("const int64_t g = h / heads_per_group;", "const int64_t g = h % G;"),
    "ignore_init": ("if (j->init_state)\n        memcpy", "if (0)\n        memcpy"),
    "boundary_off_by_one": ("(t + 1) % j->chunk_len == 0", "t % j->chunk_len == 0"),
    "skip_first_step": ("for (int64_t t = 0; t < T; ++t) {", "for (int64_t t = 1; t < T; ++t) {"),
}


def _pins_pass(lib):
    """A fast subset of the pins, run against a given build of the oracle."""
    ok = True
    g, inp = _example_as_ssd()
    y, _, _ = oracle.ssd_ref(**inp, lib=lib)
    ok &= np.allclose(y.reshape(4), g["y_recurrence"], atol=1e-12)
    rng = np.random.default_rng(99)
    for case in ((1, 24, 4, 2, 8, 2, True), (1, 19, 3, 3, 5, 3, True)):
        bsz, T, H, P, N, G, wi = case
        c = _rand_case(rng, bsz, T, H, P, N, G, wi)
        y_r, f_r, bnd = oracle.ssd_ref(**c, chunk_len=8, lib=lib)
        y_q, f_q = ssd_quadratic(**c)
        ok &= np.allclose(y_r, y_q, atol=1e-11) and np.allclose(f_r, f_q, atol=1e-11)
        pre = {k: (v[:, :8] if k in ("x", "dt", "B", "C") else v) for k, v in c.items()}
        _, f8 = ssd_quadratic(**pre)
        ok &= np.allclose(bnd[:, :, 0], f8, atol=1e-11)
    return bool(ok)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_pins_reject_planted_mistakes():
    src = open(oracle_build.SOURCE).read()
    assert _pins_pass(oracle.library())
    with tempfile.TemporaryDirectory() as tmp:
        shutil.copy(os.path.join(os.path.dirname(oracle_build.SOURCE), "ssd_oracle.h"), tmp)
        for name, (old, new) in MUTANTS.items():
            assert src.count(old) == 1, f"mutation site for {name} not unique"
            path = os.path.join(tmp, f"m_{name}.c")
            with open(path, "w") as f:
                f.write(src.replace(old, new))
            out = os.path.join(tmp, f"m_{name}.so")
            subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-I", tmp, path, "-o", out,
                            "-lm", "-lpthread"], check=True, capture_output=True)
            lib = oracle.load_library(out)
            assert not _pins_pass(lib), f"no pin catches the planted mistake '{name}'"
