"""Wiring pins for the layer oracle (oracle/model.py), independent of its sequence form.

Each test builds a one-layer stack whose weights are zeros, scaled identities or one-hot
rows, so that the layer collapses to a closed form that can be written down by hand: a
channel whose conv output is exactly SiLU(0) = 0, a softplus of exactly 0 (ln 2), a gate of
SiLU(0) = 0, attention over keys with all-zero scores (a plain average of the values).  The
special cases are chosen so that a plausible wiring mistake -- x instead of u feeding W_r,
W_b or W_c, the gate taken from u or from the un-normed stream, the conv history holding u,
keys averaged instead of values, a layer reading the un-normed stream -- gives a different
number.  tests/test_oracle_model_mutants.py plants each of those mistakes in a copy of the
oracle and checks that one of these pins fails.

Definitions from the page "Samba: Simple Hybrid State Space Models for Efficient Unlimited
Context Language Modeling" (paper-graph-ui summary): "The Mamba Layer" (H = X W_in,
U = SiLU(conv(H)), Delta = softplus(U W_r W_q + b), B = U W_b, C = U W_c, the S6 update,
(Y * SiLU(X W_g)) W_out), "The Sliding Window Attention (SWA) Layer" and "Window
Specification", "SwiGLU Formulation", "The layer arrangement pattern" (RMSNorm before, a
residual skip after every layer).
"""
import math

import numpy as np
from scipy.special import expit

from oracle import model

LN2 = math.log(2.0)


def silu(v):
    return np.asarray(v, dtype=np.float64) * expit(v)


def cfg(dm=4, de=4, N=1, dr=1, H=1, Hk=1, dh=64, window=1, dff=4):
    return dict(d_model=dm, d_inner=de, d_state=N, dt_rank=dr, d_ff=dff, n_heads=H, n_kv_heads=Hk, head_dim=dh,
                window=window, rope_base=10000.0, norm_eps=0.0)


def mamba_layer(c, w_in, w_g, w_r, w_b, w_c, w_q, w_out, conv_w, conv_b, A=None, D=None, dt_bias=None):
    de, N = c["d_inner"], c["d_state"]
    return dict(kind="mamba", norm_w=np.ones(c["d_model"]), w_in_gate=np.concatenate([w_in, w_g]),
                w_xproj=np.concatenate([w_r, w_b, w_c]), w_dt_up=w_q, w_out=w_out,
                A=np.full((de, N), -1.0) if A is None else A, D=np.zeros(de) if D is None else D,
                dt_bias=np.zeros(de) if dt_bias is None else dt_bias, conv_w=conv_w, conv_b=conv_b)


def onehot_rows(n_rows, n_cols, cols):
    w = np.zeros((n_rows, n_cols))
    for r, k in enumerate(cols):
        w[r, k] = 1.0
    return w


def step(c, layers, hidden, pos=None, state=None):
    S = hidden.shape[0]
    st = model.DecodeState(c, layers, S) if state is None else state
    p = np.zeros(S, int) if pos is None else pos
    h, _ = model.decode_step(c, layers, np.ones(c["d_model"]), hidden, st, p)
    return h, st


# A hidden row whose RMS is not 1 (so the normed input differs from the stream) and whose
# entries are all different (so a transposed or permuted read changes the result).
HID = np.array([[0.5, -1.5, 2.0, 3.0]])
HN = HID / np.sqrt(np.mean(HID * HID))


def test_B_is_a_projection_of_u_not_x():
    """W_b selects channel 0, whose conv input is cancelled by its bias: u_0 = SiLU(0) = 0
    while x_0 = 0.7 hn_0 != 0.  So B = 0, the state stays 0 and y = D u exactly; the layer
    adds W_out (D u SiLU(z)) with W_out = I."""
    c = cfg()
    x = 0.7 * HN[0]
    conv_b = np.array([-x[0], 0.3, -0.2, 0.1])
    D = np.array([1.5, -0.5, 2.0, 0.25])
    ly = mamba_layer(c, 0.7 * np.eye(4), np.eye(4), np.ones((1, 4)), onehot_rows(1, 4, [0]), onehot_rows(1, 4, [1]),
                     np.full((4, 1), 0.4), np.eye(4), np.tile([0.0, 0.0, 0.0, 1.0], (4, 1)), conv_b, D=D)
    u = silu(x + conv_b)
    assert u[0] == 0.0
    h, _ = step(c, [ly], HID.copy())
    np.testing.assert_allclose(h[0], HID[0] + D * u * silu(HN[0]), rtol=1e-13, atol=1e-15)


def test_C_is_a_projection_of_u_not_x():
    """W_c selects the channel with u = 0 (x != 0): C = 0, so y = D u whatever the state."""
    c = cfg()
    x = 0.7 * HN[0]
    conv_b = np.array([0.2, -x[1], -0.2, 0.1])
    D = np.array([1.5, -0.5, 2.0, 0.25])
    ly = mamba_layer(c, 0.7 * np.eye(4), np.eye(4), np.ones((1, 4)), onehot_rows(1, 4, [2]), onehot_rows(1, 4, [1]),
                     np.full((4, 1), 0.4), np.eye(4), np.tile([0.0, 0.0, 0.0, 1.0], (4, 1)), conv_b, D=D)
    u = silu(x + conv_b)
    assert u[1] == 0.0 and u[2] != 0.0
    h, _ = step(c, [ly], HID.copy())
    np.testing.assert_allclose(h[0], HID[0] + D * u * silu(HN[0]), rtol=1e-13, atol=1e-15)


def test_delta_path_reads_u_and_the_bias():
    """W_r selects the channel with u = 0 (x != 0) and the Delta bias is 0, so Delta =
    softplus(0) = ln 2 on every channel.  From a zero state h = ln 2 B u with B = u_2,
    C = u_3 (one-hot W_b, W_c) and D = 0: out_d = ln 2 u_2 u_3 u_d SiLU(z_d)."""
    c = cfg()
    x = 0.7 * HN[0]
    conv_b = np.array([-x[0], 0.3, 0.5, -0.4])
    ly = mamba_layer(c, 0.7 * np.eye(4), np.eye(4), onehot_rows(1, 4, [0]), onehot_rows(1, 4, [2]),
                     onehot_rows(1, 4, [3]), np.full((4, 1), 3.0), np.eye(4), np.tile([0.0, 0.0, 0.0, 1.0], (4, 1)),
                     conv_b)
    u = silu(x + conv_b)
    assert u[0] == 0.0
    h, _ = step(c, [ly], HID.copy())
    np.testing.assert_allclose(h[0], HID[0] + LN2 * u[2] * u[3] * u * silu(HN[0]), rtol=1e-13, atol=1e-15)
    # a nonzero bias b moves Delta to softplus(b) = log(1 + e^b): with b = log(e - 1), Delta = 1
    ly["dt_bias"] = np.full(4, math.log(math.e - 1.0))
    h, _ = step(c, [ly], HID.copy())
    np.testing.assert_allclose(h[0], HID[0] + u[2] * u[3] * u * silu(HN[0]), rtol=1e-13, atol=1e-15)


def test_gate_reads_the_normed_input():
    """W_g = a permutation: z_d = hn_{perm(d)}, the normed stream (RMS of HID != 1), not u
    and not the raw stream."""
    c = cfg()
    x = 0.7 * HN[0]
    conv_b = np.array([-x[0], 0.3, -0.2, 0.1])
    D = np.array([1.5, -0.5, 2.0, 0.25])
    perm = [2, 0, 3, 1]
    ly = mamba_layer(c, 0.7 * np.eye(4), onehot_rows(4, 4, perm), np.ones((1, 4)), onehot_rows(1, 4, [0]),
                     onehot_rows(1, 4, [1]), np.full((4, 1), 0.4), np.eye(4), np.tile([0.0, 0.0, 0.0, 1.0], (4, 1)),
                     conv_b, D=D)
    u = silu(x + conv_b)
    h, _ = step(c, [ly], HID.copy())
    np.testing.assert_allclose(h[0], HID[0] + D * u * silu(HN[0][perm]), rtol=1e-13, atol=1e-15)


def test_conv_history_holds_the_pre_conv_input():
    """Taps (0, 0, k, 1): the second token's conv sees the first token's x (not its u):
    u2 = SiLU(x2 + k x1 + b).  W_b = 0 makes B = 0, which keeps the state at 0 and y = D u,
    so the output shows u1 and u2 directly."""
    c = cfg()
    kap = 0.8
    D = np.array([1.0, 2.0, -1.0, 0.5])
    ly = mamba_layer(c, 0.7 * np.eye(4), np.eye(4), np.ones((1, 4)), np.zeros((1, 4)), np.ones((1, 4)),
                     np.full((4, 1), 0.4), np.eye(4), np.tile([0.0, 0.0, kap, 1.0], (4, 1)), np.full(4, 0.1), D=D)
    h1, st = step(c, [ly], HID.copy())
    x1 = 0.7 * HN[0]
    np.testing.assert_allclose(h1[0], HID[0] + D * silu(x1 + 0.1) * silu(HN[0]), rtol=1e-13, atol=1e-15)
    hid2 = np.array([[-1.0, 0.25, 0.5, 2.0]])
    hn2 = hid2 / np.sqrt(np.mean(hid2 * hid2))
    h2, _ = step(c, [ly], hid2.copy(), state=st)
    x2 = 0.7 * hn2[0]
    np.testing.assert_allclose(h2[0], hid2[0] + D * silu(x2 + kap * x1 + 0.1) * silu(hn2[0]), rtol=1e-13,
                               atol=1e-15)


def test_state_is_carried_between_steps():
    """A = 0 (Abar = 1): after two tokens the state is the plain sum of the inputs,
    h = Delta_1 B_1 u_1 + Delta_2 B_2 u_2, with B = u_1 (one-hot W_b) and Delta =
    softplus(3 u_0) (W_r selects channel 0, W_q = 3, bias 0); the conv history then holds the
    last three pre-conv inputs, oldest first.  W_g = 0 (gate SiLU(0) = 0) keeps the stream
    unchanged; the state itself is compared."""
    c = cfg()
    ly = mamba_layer(c, 0.7 * np.eye(4), np.zeros((4, 4)), onehot_rows(1, 4, [0]), onehot_rows(1, 4, [1]),
                     onehot_rows(1, 4, [2]), np.full((4, 1), 3.0), np.eye(4), np.tile([0.0, 0.0, 0.0, 1.0], (4, 1)),
                     np.zeros(4), A=np.zeros((4, 1)))
    st = model.DecodeState(c, [ly], 1)
    hids = [HID.copy(), np.array([[-1.0, 0.25, 0.5, 2.0]])]
    u_hist = []
    for hid in hids:
        hn = hid / np.sqrt(np.mean(hid * hid))
        x = 0.7 * hn[0]
        u = silu(x)
        u_hist.append(u)
        model.decode_step(c, [ly], np.ones(4), hid, st, np.zeros(1, int))
    expect = np.zeros(4)
    for u in u_hist:
        delta = np.logaddexp(0.0, 3.0 * u[0])
        expect = expect + delta * u[1] * u
    np.testing.assert_allclose(st.h[0][0, :, 0], expect, rtol=1e-13, atol=1e-15)
    # conv history: the last inputs x, oldest first (zeros before the first token)
    x0 = 0.7 * (hids[0] / np.sqrt(np.mean(hids[0] ** 2)))[0]
    x1 = 0.7 * (hids[1] / np.sqrt(np.mean(hids[1] ** 2)))[0]
    np.testing.assert_allclose(st.hist[0][0], np.stack([np.zeros(4), x0, x1]), rtol=1e-15, atol=0)


def test_attention_with_zero_scores_averages_the_values_in_the_window():
    """W_q = 0 makes every score 0, so the softmax is uniform over the keys the window
    admits: positions t-1 .. t for window 1.  The layer then adds W_o mean(v) with v = hn W_v
    (W_v = 2 I, W_k = -I, W_o = I): the output is an average of values, never of keys, over
    exactly window + 1 positions."""
    c = cfg(dm=64, dh=64, window=1)
    rng = np.random.default_rng(7)
    ly = dict(kind="swa", norm_w=np.ones(64),
              w_qkv=np.concatenate([np.zeros((64, 64)), -np.eye(64), 2.0 * np.eye(64)]), w_o=np.eye(64))
    st = model.DecodeState(c, [ly], 1)
    hids = [rng.standard_normal((1, 64)) * (1.0 + t) for t in range(4)]
    vs = []
    for t, hid in enumerate(hids):
        hn = hid / np.sqrt(np.mean(hid * hid))
        vs.append(2.0 * hn[0])
        h, _ = model.decode_step(c, [ly], np.ones(64), hid, st, np.array([t]))
        lo = max(0, t - 1)
        np.testing.assert_allclose(h[0], hid[0] + np.mean(vs[lo:t + 1], axis=0), rtol=1e-12, atol=1e-13)


def test_inactive_sequence_gets_no_attention_output():
    """pos < 0: the attention layer adds nothing (W_o . 0)."""
    c = cfg(dm=64, dh=64, window=1)
    ly = dict(kind="swa", norm_w=np.ones(64),
              w_qkv=np.concatenate([np.zeros((64, 64)), -np.eye(64), 2.0 * np.eye(64)]), w_o=np.eye(64))
    st = model.DecodeState(c, [ly], 2)
    hid = np.random.default_rng(8).standard_normal((2, 64))
    h, _ = model.decode_step(c, [ly], np.ones(64), hid, st, np.array([0, -1]))
    np.testing.assert_array_equal(h[1], hid[1])
    np.testing.assert_allclose(h[0], hid[0] + 2.0 * hid[0] / np.sqrt(np.mean(hid[0] ** 2)), rtol=1e-13)


def test_mlp_reads_the_normed_input():
    """W1 = a I, W2 = b I, W3 = I: the layer adds a hn SiLU(b hn) with hn the normed stream."""
    c = cfg()
    a, b = 0.5, -1.25
    ly = dict(kind="mlp", norm_w=np.ones(4), w12=np.concatenate([a * np.eye(4), b * np.eye(4)]), w3=np.eye(4))
    st = model.DecodeState(c, [ly], 1)
    h, o = model.decode_step(c, [ly], np.ones(4), HID.copy(), st, np.zeros(1, int))
    np.testing.assert_allclose(h[0], HID[0] + a * HN[0] * silu(b * HN[0]), rtol=1e-13)
    # the step's second output is the final RMSNorm of the stream (weight 1)
    np.testing.assert_allclose(o[0], h[0] / np.sqrt(np.mean(h[0] ** 2)), rtol=1e-13)


def test_layers_apply_in_order_on_the_residual_stream():
    """Two MLP layers with W3 = I: the second reads the RMSNorm of the stream the first left
    (not the input), so the result is g(g(h)) with g(v) = v + a n(v) SiLU(b n(v))."""
    c = cfg()
    a, b = 0.5, -1.25
    ly = dict(kind="mlp", norm_w=np.ones(4), w12=np.concatenate([a * np.eye(4), b * np.eye(4)]), w3=np.eye(4))
    st = model.DecodeState(c, [ly, ly], 1)
    h, _ = model.decode_step(c, [ly, ly], np.ones(4), HID.copy(), st, np.zeros(1, int))

    def g(v):
        n = v / np.sqrt(np.mean(v * v))
        return v + a * n * silu(b * n)

    np.testing.assert_allclose(h[0], g(g(HID[0])), rtol=1e-13)
