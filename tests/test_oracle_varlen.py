"""Pins of the packed variable-length oracle (oracle/varlen.py).

- the sequence-by-sequence oracle equals a plain step loop that resets the state at every
  sequence start;
- one sequence equals the layer's oracle;
- sequences are independent: changing one leaves the others' outputs bit-identical;
- empty sequences have zero final states, and malformed cu_seqlens are rejected.
"""
import numpy as np
import pytest

import oracle
from oracle.varlen import ssd_varlen_loop, ssd_varlen_ref

RNG = np.random.default_rng(5)


def _inputs(T, H=2, P=3, N=4, G=1):
    x = RNG.standard_normal((1, T, H, P))
    dt = np.log1p(np.exp(RNG.standard_normal((1, T, H)) - 1))
    A = -np.exp(RNG.uniform(np.log(0.05), np.log(2.0), H))
    B = RNG.standard_normal((1, T, G, N)) / 2
    C = RNG.standard_normal((1, T, G, N)) / 2
    D = RNG.standard_normal(H)
    return x, dt, A, B, C, D


@pytest.mark.parametrize("cu", [[0, 7, 19, 20, 31], [0, 31], [0, 1, 2, 3, 31], [0, 10, 10, 31]])
def test_varlen_equals_reset_loop(cu):
    args = _inputs(31, H=4, G=2)
    y, f = ssd_varlen_ref(*args, cu)
    y2, f2 = ssd_varlen_loop(*args, cu)
    assert np.allclose(y, y2, rtol=1e-12, atol=1e-12)
    assert np.allclose(f, f2, rtol=1e-12, atol=1e-12)


def test_single_sequence_is_the_layer():
    args = _inputs(40)
    y, f = ssd_varlen_ref(*args, [0, 40])
    y2, f2, _ = oracle.ssd_ref(*args)
    assert np.array_equal(y, y2) and np.array_equal(f[0], f2[0])


def test_sequences_are_independent():
    x, dt, A, B, C, D = _inputs(30)
    cu = [0, 9, 21, 30]
    y, f = ssd_varlen_ref(x, dt, A, B, C, D, cu)
    x2 = x.copy()
    x2[:, 9:21] += 1.0     # change only the second sequence
    y2, f2 = ssd_varlen_ref(x2, dt, A, B, C, D, cu)
    assert np.array_equal(y[:, :9], y2[:, :9]) and np.array_equal(y[:, 21:], y2[:, 21:])
    assert np.array_equal(f[0], f2[0]) and np.array_equal(f[2], f2[2])
    assert not np.allclose(y[:, 9:21], y2[:, 9:21])


def test_empty_sequences_and_bad_offsets():
    args = _inputs(12)
    y, f = ssd_varlen_ref(*args, [0, 0, 12, 12])
    assert np.all(f[0] == 0) and np.all(f[2] == 0)
    for bad in ([1, 12], [0, 11], [0, 8, 5, 12], [0]):
        with pytest.raises(ValueError):
            ssd_varlen_ref(*args, bad)
