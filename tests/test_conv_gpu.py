"""GPU parity of the conv-only entry point (short causal conv + SiLU, the activation a full
layer feeds to x_proj) against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_samba_amd as ss
from selective_state_space_samba_amd import synth
from tests.helpers import TOL, host, rel_err, tdev, tf32

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def bias(seed, D):
    """A nonzero conv bias (the synthetic layer parameters start it at zero)."""
    return (0.1 * np.random.default_rng(seed).standard_normal(D)).astype(np.float32)


def check(u, cf, ur, cr, io, tag):
    e = rel_err(u, ur)
    print("  %s u err %.3e (tol %.0e)" % (tag, e, TOL[io]), flush=True)
    assert e <= TOL[io]
    if cf is not None:
        np.testing.assert_array_equal(cf, cr)  # the outgoing history is a copy: bit-exact


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("b,L,D", [(3, 333, 320), (2, 70, 100), (2, 129, 98), (1, 4096 + 5, 64)])
@pytest.mark.parametrize("with_hist", [False, True])
def test_conv_silu_fixed_length(io, b, L, D, with_hist):
    """Runs of 64 tokens with a ragged last run; d_inner = 100 and 98 leave the 16-byte
    channel vectors (98 for both dtypes, 100 for bf16) and take the one-channel path."""
    seed = 1000 + L + D
    print("case: conv", io, b, L, D, "hist", with_hist, flush=True)
    p = synth.make_params(seed, D, 16)
    tk = synth.make_tokens(seed, (b, L), D, 16, io)
    c0 = synth.make_state(seed, b, D, 16, io, scale=0.5)[1] if with_hist else None
    cb = bias(seed, D)
    u, cf = ss.conv_silu(tdev(tk.x, io, DEV), tf32(p.conv_w, DEV), tf32(cb, DEV),
                         None if c0 is None else tdev(c0, io, DEV))
    torch.cuda.synchronize()
    ur, cr = oracle.conv_silu(tk.x, p.conv_w, cb, conv0=c0)
    check(host(u), host(cf), ur, cr, io, "fixed")


@pytest.mark.parametrize("L", [0, 1, 2, 3, 64, 65])
def test_conv_silu_short_sequences(L):
    io, b, D = "bf16", 2, 128
    seed = 1100 + L
    print("case: conv short", L, flush=True)
    p = synth.make_params(seed, D, 16)
    tk = synth.make_tokens(seed, (b, L), D, 16, io)
    c0 = synth.make_state(seed, b, D, 16, io, scale=0.5)[1]
    u, cf = ss.conv_silu(tdev(tk.x, io, DEV), tf32(p.conv_w, DEV), tf32(p.conv_b, DEV), tdev(c0, io, DEV))
    torch.cuda.synchronize()
    ur, cr = oracle.conv_silu(tk.x, p.conv_w, p.conv_b, conv0=c0)
    check(host(u), host(cf), ur, cr, io, "short")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_conv_silu_packed(io):
    lens = [0, 1, 2, 3, 5, 100, 257, 0, 64, 130]
    cu = synth.cu_from_lengths(lens)
    T, D = int(cu[-1]), 192
    seed = 1200
    print("case: conv packed", lens, io, flush=True)
    p = synth.make_params(seed, D, 16)
    tk = synth.make_tokens(seed, (T,), D, 16, io)
    c0 = synth.make_state(seed, len(lens), D, 16, io, scale=0.5)[1]
    cb = bias(seed, D)
    u, cf = ss.conv_silu(tdev(tk.x, io, DEV), tf32(p.conv_w, DEV), tf32(cb, DEV), tdev(c0, io, DEV),
                         cu_seqlens=torch.from_numpy(cu).to(DEV), max_seqlen=max(lens))
    torch.cuda.synchronize()
    ur, cr = oracle.conv_silu(tk.x, p.conv_w, cb, conv0=c0, cu_seqlens=cu)
    check(host(u), host(cf), ur, cr, io, "packed")


def test_conv_silu_no_state_output_and_no_bias():
    io, b, L, D = "bf16", 2, 100, 64
    p = synth.make_params(1300, D, 16)
    tk = synth.make_tokens(1300, (b, L), D, 16, io)
    u, cf = ss.conv_silu(tdev(tk.x, io, DEV), tf32(p.conv_w, DEV), None, want_state=False)
    torch.cuda.synchronize()
    assert cf is None
    ur, _ = oracle.conv_silu(tk.x, p.conv_w, np.zeros(D))
    check(host(u), None, ur, None, io, "no bias")


def test_conv_silu_history_continues_across_chunks():
    """Two calls over halves of a sequence, the first call's outgoing history passed as
    the second's incoming one, equal one call over the whole sequence."""
    io, b, L, D = "bf16", 2, 300, 128
    p = synth.make_params(1400, D, 16)
    tk = synth.make_tokens(1400, (b, L), D, 16, io)
    x = tdev(tk.x, io, DEV)
    w, cb = tf32(p.conv_w, DEV), tf32(p.conv_b, DEV)
    u_all, cf_all = ss.conv_silu(x, w, cb)
    u1, cf1 = ss.conv_silu(x[:, :131].contiguous(), w, cb)
    u2, cf2 = ss.conv_silu(x[:, 131:].contiguous(), w, cb, cf1)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([u1, u2], dim=1), u_all)
    assert torch.equal(cf2, cf_all)
