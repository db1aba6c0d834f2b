"""fp64 CPU oracle for the layers around the scan: projections, SwiGLU MLP, RMSNorm.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by ``tests/`` and
``bench.py``'s CPU baseline, never by the product package.  numpy in float64; a matrix
product is the library primitive ``@`` applied to the definition as written on the page
"Samba: Simple Hybrid State Space Models for Efficient Unlimited Context Language
Modeling" (paper-graph-ui summary):
- a projection X W with W in R^{d_in x d_out} ("Input Projection and Short Convolution",
  "Gated Output", the attention projections); weights here are stored one row per output
  feature, W^T [d_out, d_in], so the product is ``x @ w_t.T``;
- "SwiGLU Formulation": SwiGLU(x) = (x W1) * SiLU(x W2), followed by W3.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def silu(v):
    v = _f64(v)
    return v / (1.0 + np.exp(-v))


def linear(x, w_t):
    """x [M, d_in] times W = w_t.T: one output feature per row of w_t [d_out, d_in]."""
    return _f64(x) @ _f64(w_t).T


def swiglu(x, w1_t, w2_t):
    """(x W1) * SiLU(x W2), the intermediate activation of the SwiGLU MLP."""
    return linear(x, w1_t) * silu(linear(x, w2_t))
