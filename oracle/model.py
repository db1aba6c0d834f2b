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


def rmsnorm(x, w, eps):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * w (page 1, "The layer
    arrangement pattern": every layer is preceded by RMSNorm)."""
    x = _f64(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * _f64(w)


def _split_heads(a, heads, dh):
    return a.reshape(a.shape[:-1] + (heads, dh))


def mamba_weights(cfg, ly):
    """W_in^T, W_g^T, W_r^T, W_b^T, W_c^T from the stacked matrices of a Mamba layer."""
    de, dr, N = cfg["d_inner"], cfg["dt_rank"], cfg["d_state"]
    wig, wx = ly["w_in_gate"], ly["w_xproj"]
    return wig[:de], wig[de:], wx[:dr], wx[dr:dr + N], wx[dr + N:]


def qkv_weights(cfg, ly):
    """W_q^T, W_k^T, W_v^T from the stacked matrix of an attention layer."""
    hq, hk = cfg["n_heads"] * cfg["head_dim"], cfg["n_kv_heads"] * cfg["head_dim"]
    w = ly["w_qkv"]
    return w[:hq], w[hq:hq + hk], w[hq + hk:]


class DecodeState:
    """Decode state of a stack, float64: per Mamba layer h [S, d_inner, N] and the conv
    history [S, 3, d_inner] (oldest first); per SWA layer every key and value of every
    sequence so far (un-rotated), so that attention can be taken over any window."""

    def __init__(self, cfg, layers, nseq):
        self.h, self.hist, self.k, self.v = {}, {}, {}, {}
        for i, ly in enumerate(layers):
            if ly["kind"] == "mamba":
                self.h[i] = np.zeros((nseq, cfg["d_inner"], cfg["d_state"]))
                self.hist[i] = np.zeros((nseq, 3, cfg["d_inner"]))
            elif ly["kind"] == "swa":
                self.k[i] = [np.zeros((0, cfg["n_kv_heads"], cfg["head_dim"])) for _ in range(nseq)]
                self.v[i] = [np.zeros((0, cfg["n_kv_heads"], cfg["head_dim"])) for _ in range(nseq)]


def cached_key(k, p, base, act):
    """The key that, rotated by RoPE at position p, equals act(RoPE(k, p)): how a key kept in
    a cache after rotation, in the activation precision ``act``, enters attention (the
    rotation by -p is exact in float64 up to rounding of the order 1e-16)."""
    import oracle
    out = np.empty_like(_f64(k))
    for h in range(k.shape[0]):
        out[h] = oracle.rope(act(oracle.rope(k[h], p, base)), -p, base)
    return out


def decode_step(cfg, layers, final_norm_w, hidden, state, pos, act=None):
    """One generation step of the stack for S sequences: for each layer hidden +=
    Layer(RMSNorm(hidden)); returns (hidden, RMSNorm(hidden) with final_norm_w), both
    float64 [S, d_model].  ``state`` is updated; ``pos`` (int array [S]) is the new tokens'
    positions (SWA keys are appended at pos; sequences with pos < 0 get no attention output)
    and is NOT modified.  Layers follow page 1: "The Mamba Layer" (H = X W_in, U =
    SiLU(conv(H)), Delta = softplus(U W_r W_q + b), B = U W_b, C = U W_c, the S6 update,
    (Y * SiLU(X W_g)) W_out), "The Sliding Window Attention (SWA) Layer", "SwiGLU
    Formulation"; the Mamba core is the oracle's decode step.

    ``act`` (default: none) is applied to every activation a layer hands to the next
    operation (the normed input, x, z, u, the Delta factors, B, C, Y, q, k, v, the attention
    output, the SwiGLU product) and to the keys kept for later steps after their rotation
    (see cached_key): passing a rounding to bfloat16 gives the same definition evaluated with
    bfloat16 activations between operations, still in float64 arithmetic."""
    import oracle
    rounded = act is not None
    if act is None:
        act = lambda a: a  # noqa: E731
    hidden = _f64(hidden).copy()
    S = hidden.shape[0]
    eps = cfg["norm_eps"]
    H, Hk, dh, w = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["window"]
    for i, ly in enumerate(layers):
        hn = act(rmsnorm(hidden, ly["norm_w"], eps))
        if ly["kind"] == "mamba":
            w_in, w_g, w_r, w_b, w_c = mamba_weights(cfg, ly)
            x, z = act(linear(hn, w_in)), act(linear(hn, w_g))
            u, _ = oracle.conv_silu(x[:, None, :], ly["conv_w"], ly["conv_b"], conv0=state.hist[i])
            u = act(u[:, 0, :])
            dt = act(linear(act(linear(u, w_r)), ly["w_dt_up"]))
            Bm, Cm = act(linear(u, w_b)), act(linear(u, w_c))
            y = act(oracle.decode_step(x, dt, Bm, Cm, z, ly["A"], ly["D"], ly["dt_bias"], ly["conv_w"],
                                       ly["conv_b"], state.h[i], state.hist[i]))
            hidden += linear(y, ly["w_out"])
        elif ly["kind"] == "swa":
            w_q, w_k, w_v = qkv_weights(cfg, ly)
            q = _split_heads(act(linear(hn, w_q)), H, dh)
            k = _split_heads(act(linear(hn, w_k)), Hk, dh)
            v = _split_heads(act(linear(hn, w_v)), Hk, dh)
            o = np.zeros((S, H, dh))
            for s in range(S):
                p = int(pos[s])
                if p < 0:
                    continue
                assert state.k[i][s].shape[0] == p, "key history must hold exactly positions 0..pos-1"
                ks = cached_key(k[s], p, cfg["rope_base"], act) if rounded else k[s]
                state.k[i][s] = np.concatenate([state.k[i][s], ks[None]])
                state.v[i][s] = np.concatenate([state.v[i][s], v[s][None]])
                qs = np.zeros((1, p + 1, H, dh))
                qs[0, p] = q[s]
                o[s] = oracle.swa(qs, state.k[i][s][None], state.v[i][s][None], window=w, base=cfg["rope_base"],
                                  rows=[p])[0, p]
            hidden += linear(act(o.reshape(S, H * dh)), ly["w_o"])
        else:
            dff = cfg["d_ff"]
            m = act(swiglu(hn, ly["w12"][:dff], ly["w12"][dff:]))
            hidden += linear(m, ly["w3"])
    return hidden, rmsnorm(hidden, final_norm_w, eps)


def prefill(cfg, layers, final_norm_w, emb):
    """The same stack over whole sequences (emb [S, L, d_model], zero initial state), in
    sequence form: the Mamba core through the oracle's prefill and conv, attention through
    the oracle's sliding-window attention.  Returns (hidden, out) [S, L, d_model]."""
    import oracle
    hidden = _f64(emb).copy()
    S, L, dm = hidden.shape
    eps = cfg["norm_eps"]
    H, Hk, dh = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    for ly in layers:
        hn = rmsnorm(hidden, ly["norm_w"], eps).reshape(S * L, dm)
        if ly["kind"] == "mamba":
            de = cfg["d_inner"]
            w_in, w_g, w_r, w_b, w_c = mamba_weights(cfg, ly)
            x = linear(hn, w_in).reshape(S, L, de)
            z = linear(hn, w_g).reshape(S, L, de)
            u, _ = oracle.conv_silu(x, ly["conv_w"], ly["conv_b"])
            u2 = u.reshape(S * L, de)
            dt = linear(linear(u2, w_r), ly["w_dt_up"]).reshape(S, L, de)
            Bm = linear(u2, w_b).reshape(S, L, -1)
            Cm = linear(u2, w_c).reshape(S, L, -1)
            y, _, _ = oracle.prefill(x, dt, Bm, Cm, z, ly["A"], ly["D"], ly["dt_bias"], ly["conv_w"], ly["conv_b"])
            hidden += linear(y.reshape(S * L, de), ly["w_out"]).reshape(S, L, dm)
        elif ly["kind"] == "swa":
            w_q, w_k, w_v = qkv_weights(cfg, ly)
            q = linear(hn, w_q).reshape(S, L, H, dh)
            k = linear(hn, w_k).reshape(S, L, Hk, dh)
            v = linear(hn, w_v).reshape(S, L, Hk, dh)
            o = oracle.swa(q, k, v, window=cfg["window"], base=cfg["rope_base"])
            hidden += linear(o.reshape(S * L, H * dh), ly["w_o"]).reshape(S, L, dm)
        else:
            dff = cfg["d_ff"]
            m = swiglu(hn, ly["w12"][:dff], ly["w12"][dff:])
            hidden += linear(m, ly["w3"]).reshape(S, L, dm)
    return hidden, rmsnorm(hidden, final_norm_w, eps)
