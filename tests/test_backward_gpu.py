"""GPU parity of the backward entry point (gradients for training) against the fp64
oracle's gradients, through the C ABI.  The oracle's gradients are themselves pinned by
finite differences of the forward oracle (test_oracle_pins)."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_samba_amd as ss
from selective_state_space_samba_amd import synth
from tests.helpers import TOL, host, rel_err, tdev, tf32

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOKEN_GRADS = ("dx", "ddt", "dz", "dB", "dC")
PARAM_GRADS = ("dA", "dD", "ddt_bias", "dconv_w", "dconv_b")


def make(seed, lead, nseq, D, N, io, random_A=False, gate=True, state=True):
    p = synth.make_params(seed, D, N, random_A=random_A)
    p.conv_b = (0.1 * np.random.default_rng(seed).standard_normal(D)).astype(np.float32)  # nonzero bias
    tk = synth.make_tokens(seed, lead, D, N, io)
    g = synth.make_tokens(seed, lead, D, N, io, tag="grad").x
    h0 = c0 = dhf = dcf = None
    if state:
        h0, c0 = synth.make_state(seed, nseq, D, N, io, scale=0.5)
        dhf, dcf = synth.make_state(seed, nseq, D, N, io, scale=0.5, tag="grad")
    return p, tk, g, h0, c0, dhf, dcf, gate


def run_both(case, io, cu=None, max_seqlen=None):
    p, tk, g, h0, c0, dhf, dcf, gate = case
    z = tk.z if gate else None
    dv = lambda a: None if a is None else tdev(a, io, DEV)
    fv = lambda a: None if a is None else tf32(a, DEV)
    print("case: backward x", tk.x.shape, "N", tk.B.shape[-1], io, "gate", gate, "state", h0 is not None,
          "packed", cu is not None, flush=True)
    got = ss.backward(dv(g), dv(tk.x), dv(tk.dt), dv(tk.B), dv(tk.C), dv(z), fv(p.A), fv(p.Dskip), fv(p.dt_bias),
                      fv(p.conv_w), fv(p.conv_b), fv(h0), dv(c0), dh_final=fv(dhf), dconv_final=dv(dcf),
                      cu_seqlens=None if cu is None else torch.from_numpy(cu).to(DEV), max_seqlen=max_seqlen)
    torch.cuda.synchronize()
    ref = oracle.backward(tk.x, tk.dt, tk.B, tk.C, z, p.A, p.Dskip, p.dt_bias, p.conv_w, p.conv_b, g, h0=h0,
                          conv0=c0, dh_final=dhf, dconv_final=dcf, cu_seqlens=cu)
    return {k: None if v is None else host(v) for k, v in got.items()}, ref


def check(got, ref, io, names=TOKEN_GRADS + PARAM_GRADS + ("dh0", "dconv0")):
    for k in names:
        if ref.get(k) is None:
            assert got.get(k) is None, k
            continue
        e = rel_err(got[k], ref[k])
        print("  %-9s err %.3e (tol %.0e)" % (k, e, TOL[io]), flush=True)
        assert e <= TOL[io], k


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_backward_fixed_length_with_state(io):
    """Two sequences of 37 tokens (two full chunks and a ragged one), 96 channels (a full
    and a partial wave), incoming and outgoing state gradients."""
    check(*run_both(make(2000, (2, 37), 2, 96, 16, io), io), io)


def test_backward_random_A_long():
    check(*run_both(make(2001, (1, 300), 1, 128, 16, "f32", random_A=True), "f32"), "f32")


@pytest.mark.parametrize("L", [0, 1, 2, 3, 15, 16, 17])
def test_backward_short_sequences(L):
    check(*run_both(make(2010 + L, (2, L), 2, 64, 16, "f32"), "f32"), "f32")


def test_backward_small_state_no_gate():
    """d_state = 5 and no gate; d_inner = 100 leaves a partial wave."""
    check(*run_both(make(2020, (2, 45), 2, 100, 5, "f32", gate=False), "f32"), "f32")


def test_backward_without_state_inputs():
    check(*run_both(make(2030, (2, 50), 2, 64, 16, "bf16", state=False), "bf16"), "bf16")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_backward_packed(io):
    lens = [0, 1, 2, 3, 5, 17, 33, 0, 16, 40]
    cu = synth.cu_from_lengths(lens)
    T = int(cu[-1])
    check(*run_both(make(2040, (T,), len(lens), 64, 16, io), io, cu=cu, max_seqlen=max(lens)), io)


@pytest.mark.parametrize("io,N", [("bf16", 16), ("f32", 16), ("bf16", 7)])
def test_backward_packed_long(io, N):
    """Packed sequences long enough for many chunk groups per sequence (groups of 64 tokens
    cut at sequence ends, full chunks next to partial ones, the carry over tens of chunks), an
    empty sequence, 136 channels (two full waves and a partial one), and for N = 7 the
    per-element B / C rows."""
    lens = [1000, 37, 2049, 0, 513, 1601, 64, 65]
    cu = synth.cu_from_lengths(lens)
    T = int(cu[-1])
    check(*run_both(make(2060 + N, (T,), len(lens), 136, N, io), io, cu=cu, max_seqlen=max(lens)), io)


def test_backward_is_deterministic():
    case = make(2050, (2, 70), 2, 128, 16, "bf16")
    a, _ = run_both(case, "bf16")
    b, _ = run_both(case, "bf16")
    for k in TOKEN_GRADS + PARAM_GRADS + ("dh0", "dconv0"):
        np.testing.assert_array_equal(a[k], b[k])


def test_backward_argument_errors():
    x = torch.zeros((1, 4, 64), dtype=torch.bfloat16, device=DEV)
    Bm = torch.zeros((1, 4, 16), dtype=torch.bfloat16, device=DEV)
    prm = [torch.zeros((64, 16), device=DEV), None, None, torch.zeros((64, 4), device=DEV), None]
    with pytest.raises(ss.SambaError, match="WORKSPACE"):
        ss.backward(x, x, x, Bm, Bm, x, *prm, workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
