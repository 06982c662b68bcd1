"""The CPU oracle against what the pages and plain mathematics fix (CPU only)."""
import numpy as np
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


def _matrix_form(q, k, v, scale, causal):
    """The eager attention code of 'Kimi K3 - Softmax over keys' in matrix form, in
    float64: an explicit additive mask of 0 / -inf, softmax along the key axis, then
    the product with V.  A second, independent formulation for tiny shapes."""
    Tq, Tk = q.shape[0], k.shape[0]
    S = (q @ k.T) * scale
    if causal:
        t = np.arange(Tq)[:, None] + (Tk - Tq)
        s = np.arange(Tk)[None, :]
        S = S + np.where(s <= t, 0.0, -np.inf)
    S = S - S.max(axis=1, keepdims=True)
    E = np.exp(S)
    return (E / E.sum(axis=1, keepdims=True)) @ v


@pytest.mark.parametrize("seed", range(6))
def test_oracle_matches_matrix_form(seed):
    r = np.random.default_rng(100 + seed)
    Tk = int(r.integers(1, 40))
    Tq = int(r.integers(1, Tk + 1))
    D = int(r.integers(1, 20))
    q, k, v = r.standard_normal((Tq, D)), r.standard_normal((Tk, D)), r.standard_normal((Tk, D))
    for causal in (True, False):
        out = oracle.attend_head(q, k, v, 0.37, causal)
        assert np.max(np.abs(out - _matrix_form(q, k, v, 0.37, causal))) <= 1e-12


def test_attend_layouts_agree():
    r = np.random.default_rng(7)
    B, T, H, D = 2, 13, 3, 4
    Q, K, V = (r.standard_normal((B, T, H, D)) for _ in range(3))
    a = oracle.attend(Q, K, V, 0.5, True, layout="bthd")
    b = oracle.attend(Q.transpose(0, 2, 1, 3), K.transpose(0, 2, 1, 3), V.transpose(0, 2, 1, 3), 0.5,
                      True, layout="bhtd")
    assert np.array_equal(a, b.transpose(0, 2, 1, 3))


def test_oracle_rejects_bad_arguments():
    q = np.zeros((3, 4))
    with pytest.raises(ValueError):
        oracle.attend_head(np.zeros((5, 4)), q, q, 1.0, True)  # more queries than keys
    with pytest.raises(ValueError):
        oracle.attend_head(q, q, q, 1.0, True, rows=[3])
    with pytest.raises(ValueError):
        oracle.gated_mla_layer(np.zeros((1, 2, 6)), *([np.zeros((6, 6))] * 6), num_heads=4)
