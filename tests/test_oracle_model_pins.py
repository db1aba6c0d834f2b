"""Pins for the layer oracle (oracle/model.py): projections, SwiGLU, RMSNorm and the
whole-model decode step, each against something independent of its code -- brute-force
sums on tiny inputs, scipy's sigmoid, closed forms and exact invariances.

Definitions from the page "Samba: Simple Hybrid State Space Models for Efficient
Unlimited Context Language Modeling" (paper-graph-ui summary): "SwiGLU Formulation",
"The layer arrangement pattern" (RMSNorm before and a residual skip after each layer)."""
import numpy as np
import scipy.special

from oracle import model


def brute_linear(x, w_t):
    M, K = x.shape
    N = w_t.shape[0]
    out = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            s = 0.0
            for k in range(K):
                s += float(x[m, k]) * float(w_t[n, k])
            out[m, n] = s
    return out


def test_linear_is_the_brute_force_sum():
    rng = np.random.default_rng(1)
    x, w = rng.standard_normal((3, 5)), rng.standard_normal((4, 5))
    np.testing.assert_allclose(model.linear(x, w), brute_linear(x, w), rtol=1e-13, atol=1e-13)


def test_linear_orientation_one_hot():
    """A one-hot input row selects column k of every output row's weights: out[n] = w_t[n, k]."""
    rng = np.random.default_rng(2)
    w = rng.standard_normal((6, 4))
    x = np.zeros((1, 4))
    x[0, 2] = 1.0
    np.testing.assert_array_equal(model.linear(x, w)[0], w[:, 2])


def test_swiglu_brute_force():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 6))
    w1, w2 = rng.standard_normal((3, 6)), rng.standard_normal((3, 6))
    g, a = brute_linear(x, w1), brute_linear(x, w2)
    ref = g * a * scipy.special.expit(a)
    np.testing.assert_allclose(model.swiglu(x, w1, w2), ref, rtol=1e-12, atol=1e-13)


def test_swiglu_gate_is_the_second_factor():
    """Zero W2 makes SiLU(x W2) = 0 whatever W1; zero W1 makes the output 0 whatever W2."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 5))
    w = rng.standard_normal((3, 5))
    np.testing.assert_array_equal(model.swiglu(x, w, np.zeros_like(w)), 0.0)
    np.testing.assert_array_equal(model.swiglu(x, np.zeros_like(w), w), 0.0)
