"""Pins of the block oracle (oracle/block.py) against things other than itself.

- numpy's convolution routine for the causal depthwise conv;
- an impulse response that fixes the tap order;
- causality;
- torch's group_norm and rms_norm (fp64) for the per-token normalisation;
- closed forms and identities of softplus and SiLU;
- special cases: a zero gate gives the shift, and a normalised group has zero mean and unit
  variance;
- the slicing of the projection output checked with channel-tagged inputs;
- the whole block against the independent quadratic form of the SSD layer.

Planted mistakes in a copy of the oracle's source must each fail one of these pins.
"""
import math
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import block as ob
from oracle.quadratic import ssd_quadratic

RNG = np.random.default_rng(123)


# ------------------------------------------------------------------ the pins, per module
def pin_conv_numpy(m):
    """Causal conv equals numpy.convolve with the taps reversed (first T outputs)."""
    for K in (1, 2, 3, 4, 7):
        u = RNG.standard_normal((2, 13, 5))
        w = RNG.standard_normal((5, K))
        b = RNG.standard_normal(5)
        out = m.causal_conv1d(u, w, b)
        for bb in range(2):
            for c in range(5):
                ref = np.convolve(u[bb, :, c], w[c, ::-1])[:13] + b[c]
                if not np.allclose(out[bb, :, c], ref, rtol=1e-13, atol=1e-13):
                    return False
    return True


def pin_conv_impulse(m):
    """A unit impulse at t0 produces w[c, K-1-s] at t0 + s (the current step takes the last
    tap), the bias elsewhere."""
    K, T, t0 = 4, 12, 5
    w = RNG.standard_normal((3, K))
    b = RNG.standard_normal(3)
    u = np.zeros((1, T, 3))
    u[0, t0, 1] = 1.0
    out = m.causal_conv1d(u, w, b)
    exp = np.tile(b, (1, T, 1))
    for s in range(K):
        exp[0, t0 + s, 1] += w[1, K - 1 - s]
    return np.allclose(out, exp, rtol=0, atol=1e-15)


def pin_conv_causal(m):
    """Changing the input from step t1 on leaves every earlier output unchanged."""
    u = RNG.standard_normal((1, 20, 4))
    w = RNG.standard_normal((4, 4))
    a = m.causal_conv1d(u, w, None)
    u2 = u.copy()
    u2[:, 9:] += 1.0
    b2 = m.causal_conv1d(u2, w, None)
    return np.array_equal(a[:, :9], b2[:, :9]) and not np.allclose(a[:, 9:], b2[:, 9:])


def pin_silu(m):
    v = np.linspace(-30, 30, 601)
    s = m.silu(v)
    sig = 0.5 * (1 + np.tanh(v / 2))  # the logistic function written through tanh
    return (m.silu(0.0) == 0.0 and np.allclose(s - m.silu(-v), v, rtol=1e-13, atol=1e-12)
            and np.allclose(s, v * sig, rtol=1e-12, atol=1e-14)
            and m.silu(800.0) == 800.0 and abs(m.silu(-800.0)) == 0.0)


def pin_softplus(m):
    v = np.linspace(-40, 40, 801)
    s = m.softplus(v)
    return (abs(m.softplus(0.0) - math.log(2.0)) < 1e-15
            and np.allclose(s - m.softplus(-v), v, rtol=1e-13, atol=1e-12)
            and np.allclose(s, np.logaddexp(0.0, v), rtol=1e-14, atol=1e-300)
            and m.softplus(1000.0) == 1000.0 and np.all(s > 0))


def _torch_gate_norm(y, z, w, b, groups, rms, eps):
    yt, zt = torch.from_numpy(y), torch.from_numpy(z)
    v = yt * torch.nn.functional.silu(zt)
    Bz, T, Dc = v.shape
    flat = v.reshape(Bz * T, Dc, 1)
    if rms:
        n = torch.nn.functional.rms_norm(flat.reshape(Bz * T, groups, Dc // groups),
                                         (Dc // groups,), eps=eps)
        return (n.reshape(Bz, T, Dc) * torch.from_numpy(w)).numpy()
    n = torch.nn.functional.group_norm(flat, groups, torch.from_numpy(w), torch.from_numpy(b),
                                       eps=eps)
    return n.reshape(Bz, T, Dc).numpy()


def pin_norm_torch(m):
    """Group and RMS normalisation per token equal torch's, in fp64."""
    for groups, rms, eps in ((1, False, 1e-5), (4, False, 1e-5), (12, False, 1e-3),
                             (1, True, 1e-5), (3, True, 1e-6)):
        y = RNG.standard_normal((2, 5, 48))
        z = RNG.standard_normal((2, 5, 48))
        w = 1 + 0.1 * RNG.standard_normal(48)
        b = 0.1 * RNG.standard_normal(48)
        out = m.gate_norm(y, z, w, b, groups, rms=rms, eps=eps)
        ref = _torch_gate_norm(y, z, w, b, groups, rms, eps)
        if not np.allclose(out, ref, rtol=1e-12, atol=1e-12):
            return False
    return True


def pin_norm_special(m):
    """A zero gate gives the shift; with unit scale and no shift each group of a token has
    mean 0 and variance var / (var + eps); scaling y by c > 0 scales var by c^2."""
    y = RNG.standard_normal((1, 3, 32))
    b = RNG.standard_normal(32)
    ok = np.allclose(m.gate_norm(y, np.zeros_like(y), np.ones(32), b, 4), b, atol=1e-15)
    z = RNG.standard_normal((1, 3, 32))
    eps = 1e-5
    out = m.gate_norm(y, z, np.ones(32), np.zeros(32), 4, eps=eps).reshape(1, 3, 4, 8)
    v = (y * z / (1 + np.exp(-z))).reshape(1, 3, 4, 8)
    var = v.var(axis=3)
    ok &= np.allclose(out.mean(axis=3), 0, atol=1e-13)
    ok &= np.allclose(out.var(axis=3), var / (var + eps), rtol=1e-12)
    return bool(ok)


def pin_prologue_slices(m):
    """Identity taps (only the current step, weight 1, no bias) leave silu(xbc): x, B and C
    are the right channel ranges; dt = softplus(dt_raw + bias)."""
    H, P, N, G, T = 2, 3, 4, 1, 6
    cd = H * P + 2 * G * N
    xbc = RNG.standard_normal((1, T, cd))
    w = np.zeros((cd, 3))
    w[:, 2] = 1.0
    dt_raw = RNG.standard_normal((1, T, H))
    bias = np.array([0.3, -1.2])
    p = m.block_prologue(xbc, w, None, dt_raw, bias, H, P, N, G)
    s = xbc / (1 + np.exp(-xbc))
    sp = np.log(1 + np.exp(dt_raw + bias))
    return (np.allclose(p["x"].reshape(1, T, H * P), s[:, :, :H * P], atol=1e-15)
            and np.allclose(p["B"].reshape(1, T, N), s[:, :, H * P:H * P + N], atol=1e-15)
            and np.allclose(p["C"].reshape(1, T, N), s[:, :, H * P + N:], atol=1e-15)
            and np.allclose(p["dt"], sp, rtol=1e-14))


def pin_block_quadratic(m):
    """The block equals its parts composed by hand, with the SSD layer computed by the
    quadratic form instead of the recurrence, on a channel-tagged projection output."""
    H, P, N, G, T, K = 2, 4, 3, 1, 9, 3
    d = H * P
    cd = d + 2 * G * N
    zx = RNG.standard_normal((2, T, 2 * d + 2 * G * N + H))
    cw = RNG.standard_normal((cd, K)) * 0.5
    cb = RNG.standard_normal(cd) * 0.1
    dtb = np.array([-1.0, -2.0])
    A = np.array([-0.5, -2.0])
    D = np.array([0.7, -0.3])
    nw = 1 + 0.1 * RNG.standard_normal(d)
    nb = 0.1 * RNG.standard_normal(d)
    init = RNG.standard_normal((2, H, N, P)) * 0.3
    out, fin = m.block_fwd(zx, cw, cb, dtb, A, D, nw, nb, H, P, N, G, 2, init_state=init)
    # by hand
    z = zx[:, :, :d]
    xbc = zx[:, :, d:d + cd]
    dtr = zx[:, :, d + cd:]
    conv = np.zeros((2, T, cd)) + cb
    for t in range(T):
        for s in range(K):
            if t - s >= 0:
                conv[:, t] += cw[:, K - 1 - s] * xbc[:, t - s]
    v = conv / (1 + np.exp(-conv))
    x = v[:, :, :d].reshape(2, T, H, P)
    Bm = v[:, :, d:d + N].reshape(2, T, 1, N)
    Cm = v[:, :, d + N:].reshape(2, T, 1, N)
    dt = np.log1p(np.exp(dtr + dtb))
    y, fq = ssd_quadratic(x, dt, A, Bm, Cm, D, init_state=init)
    g = y.reshape(2, T, d) * (z / (1 + np.exp(-z)))
    gg = g.reshape(2, T, 2, d // 2)
    n = (gg - gg.mean(3, keepdims=True)) / np.sqrt(gg.var(3, keepdims=True) + 1e-5)
    ref = n.reshape(2, T, d) * nw + nb
    return (np.allclose(out, ref, rtol=1e-9, atol=1e-9)
            and np.allclose(fin, fq, rtol=1e-9, atol=1e-9))


PINS = [pin_conv_numpy, pin_conv_impulse, pin_conv_causal, pin_silu, pin_softplus,
        pin_norm_torch, pin_norm_special, pin_prologue_slices, pin_block_quadratic]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_block_oracle_pin(pin):
    assert pin(ob)


# ------------------------------------------------------------------ planted mistakes
MUTANTS = [
    ("back = K - 1 - k", "back = k"),                                      # taps reversed
    ("out += np.asarray(b, dtype=np.float64)", "out -= np.asarray(b, dtype=np.float64)"),
    ("out[:, back:, :] += w[:, k] * u[:, :T - back, :]",
     "out[:, back:, :] += w[:, k] * u[:, back:, :]"),                       # not causal
    ("return v / (1.0 + np.exp(-v))", "return 1.0 / (1.0 + np.exp(-v))"),  # sigmoid
    ("np.log1p(np.exp(-np.abs(v)))", "np.log1p(np.exp(-v))"),
    ("dtr = dtr + np.asarray(dt_bias", "dtr = dtr - np.asarray(dt_bias"),
    ("B=v[:, :, d:d + gn]", "B=v[:, :, d + gn:d + 2 * gn]"),                # B, C swapped
    ("n = (vg - mu) / np.sqrt(var + eps)", "n = vg / np.sqrt(var + eps)"),
    ("n = (vg - mu) / np.sqrt(var + eps)", "n = (vg - mu) / np.sqrt(var) "),
    ("var = np.mean((vg - mu) ** 2", "var = np.mean((vg) ** 2"),
    ("* silu(z.reshape(Bz, T, -1)))", "* z.reshape(Bz, T, -1))"),          # ungated
    ("out = out + np.asarray(bias", "out = out - np.asarray(bias"),
    ("n = vg / np.sqrt(ms + eps)", "n = vg / np.sqrt(ms + eps) * 0.5"),
    ("zx[:, :, 2 * d + 2 * gn:2 * d + 2 * gn + nheads]",
     "zx[:, :, 2 * d + gn:2 * d + gn + nheads]"),                          # dt slice
    ("zx[:, :, d:2 * d + 2 * gn]", "zx[:, :, d - 1:2 * d + 2 * gn - 1]"),   # xBC slice
]


def _mutant(src, old, new):
    assert src.count(old) >= 1, old
    mod = types.ModuleType("oracle._block_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new, 1), "block_mutant.py", "exec"), mod.__dict__)
    return mod


def test_block_pins_reject_planted_mistakes():
    src = open(ob.__file__).read()
    survivors = []
    for old, new in MUTANTS:
        m = _mutant(src, old, new)
        caught = False
        for pin in PINS:
            try:
                with np.errstate(all="ignore"):
                    if not pin(m):
                        caught = True
                        break
            except Exception:
                caught = True
                break
        if not caught:
            survivors.append(new)
    assert not survivors, f"planted mistakes not caught: {survivors}"


def test_block_oracle_uses_the_layer_oracle():
    """block_fwd's SSD step is the recurrence oracle: with an identity projection path the
    final state equals ssd_ref's on the prologue's outputs."""
    H, P, N, G, T = 2, 4, 3, 1, 7
    d = H * P
    cd = d + 2 * G * N
    zx = RNG.standard_normal((1, T, 2 * d + 2 * G * N + H))
    cw = RNG.standard_normal((cd, 2))
    A, D = np.array([-1.0, -0.2]), np.array([0.1, 0.2])
    _, fin = ob.block_fwd(zx, cw, None, None, A, D, np.ones(d), None, H, P, N, G, 1)
    z, xbc, dtr = ob.split_projection(zx, H, P, N, G)
    p = ob.block_prologue(xbc, cw, None, dtr, None, H, P, N, G)
    _, f2, _ = oracle.ssd_ref(p["x"], p["dt"], A, p["B"], p["C"], D)
    assert np.array_equal(fin, f2)
