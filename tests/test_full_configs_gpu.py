"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

The oracle is evaluated on a sample of channels (every channel's recurrence is
independent of the others, so a channel subset of the oracle is exactly the oracle's
value for those channels).  Samples include the first and last channels, channel-block
boundaries of the row kernel (multiples of 16) and random channels.
"""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_samba_amd as ss
from selective_state_space_samba_amd import synth
from tests.helpers import TOL, metrics, ordered_from_ring, tf32

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
D, N = 4096, 16


def sample_channels(seed, k_random=12):
    fixed = [0, 1, 15, 16, 17, 255, 256, 1023, 2048, 2049, 4079, 4080, 4095]
    rng = np.random.default_rng(seed)
    rnd = rng.choice(np.setdiff1d(np.arange(D), fixed), size=k_random, replace=False)
    return np.sort(np.concatenate([fixed, rnd])).astype(np.int64)


def bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(torch.bfloat16)


def params_dev(p):
    return [tf32(a, DEV) for a in (p.A, p.Dskip, p.dt_bias, p.conv_w, p.conv_b)]


def check(name, g, r, io="bf16"):
    s, e = metrics(g, r)
    print("  %s %s (tol %.0e)" % (name, s, TOL[io]), flush=True)
    assert e <= TOL[io], name


def run_prefill_case(cfg_index, b, L, conv_bias=False):
    seed = synth.seed_for(cfg_index)
    print("case: config %d batch %d L %d conv_bias %s" % (cfg_index, b, L, conv_bias), flush=True)
    p = synth.make_params(seed, D, N, conv_bias=conv_bias)
    tk = synth.make_tokens(seed, (b, L), D, N, "bf16")
    y, hf, cf = ss.prefill(bf16(tk.x), bf16(tk.dt), bf16(tk.B), bf16(tk.C), bf16(tk.z), *params_dev(p))
    chans = sample_channels(seed)
    ci = torch.from_numpy(chans).to(DEV)
    yg = y.index_select(2, ci).float().cpu().numpy()
    hg = hf.index_select(1, ci).cpu().numpy()
    cg = cf.index_select(2, ci).float().cpu().numpy()
    torch.cuda.synchronize()
    yr, hr, cr = oracle.prefill(tk.x, tk.dt, tk.B, tk.C, tk.z, p.A, p.Dskip, p.dt_bias, p.conv_w, p.conv_b,
                                chans=chans)
    check("y", yg, yr)
    check("h_final", hg, hr)
    np.testing.assert_array_equal(cg, cr)
    return y


def test_training_length_prefill_4x4096():
    run_prefill_case(1, 4, 4096)


def test_training_length_prefill_4x4096_conv_bias():
    """The same shape with a nonzero conv bias (the workload recipe has bias 0)."""
    run_prefill_case(1, 4, 4096, conv_bias=True)


def test_long_prompt_prefill_131072_conv_bias():
    """The long prompt with a nonzero conv bias, in the launch configuration the benchmark times."""
    run_prefill_case(2, 1, 131072, conv_bias=True)


def test_batch64_prefill_2048():
    """Many mid-length sequences: the one-lane-per-channel kernel's shape."""
    run_prefill_case(1, 64, 2048)


def test_long_prompt_prefill_131072():
    y = run_prefill_case(2, 1, 131072)
    assert torch.isfinite(y.float()).all()


def test_long_prompt_prefill_from_precomputed_u():
    """samba_scan_prefill_u at the long-prompt shape (batch 1, L = 131072, bf16): u from the
    oracle's conv of the prompt (sampled channels), rounded to bf16; the GPU runs all 4096
    channels on the same bf16 u (the unsampled channels' u are the workload's x values)."""
    seed = synth.seed_for(2)
    b, L = 1, 131072
    print("case: prefill_u batch %d L %d" % (b, L), flush=True)
    p = synth.make_params(seed, D, N, conv_bias=True)
    tk = synth.make_tokens(seed, (b, L), D, N, "bf16")
    chans = sample_channels(seed)
    u_s = synth.round_bf16(oracle.conv_silu(tk.x, p.conv_w, p.conv_b, chans=chans)[0].astype(np.float32))
    u = tk.x.copy()
    u[:, :, chans] = u_s
    y, hf = ss.prefill_u(bf16(u), bf16(tk.dt), bf16(tk.B), bf16(tk.C), bf16(tk.z), tf32(p.A, DEV),
                         tf32(p.Dskip, DEV), tf32(p.dt_bias, DEV))
    ci = torch.from_numpy(chans).to(DEV)
    yg = y.index_select(2, ci).float().cpu().numpy()
    hg = hf.index_select(1, ci).cpu().numpy()
    torch.cuda.synchronize()
    yr, hr = oracle.scan_u(u, tk.dt, tk.B, tk.C, tk.z, p.A, p.Dskip, p.dt_bias, chans=chans)
    check("y", yg, yr)
    check("h_final", hg, hr)


def test_training_length_backward_4x4096():
    """Gradients at the training shape (batch 4, L = 4096), every output against the
    oracle's gradients over all 4096 channels (dB and dC are sums over all of them)."""
    seed = synth.seed_for(1)
    print("case: backward batch 4 L 4096", flush=True)
    p = synth.make_params(seed, D, N)
    tk = synth.make_tokens(seed, (4, 4096), D, N, "bf16")
    g = synth.make_tokens(seed, (4, 4096), D, N, "bf16", tag="grad").x
    got = ss.backward(bf16(g), bf16(tk.x), bf16(tk.dt), bf16(tk.B), bf16(tk.C), bf16(tk.z), *params_dev(p))
    got = {k: None if v is None else v.float().cpu().numpy() for k, v in got.items()}
    torch.cuda.synchronize()
    ref = oracle.backward(tk.x, tk.dt, tk.B, tk.C, tk.z, p.A, p.Dskip, p.dt_bias, p.conv_w, p.conv_b, g)
    for k in ("dx", "ddt", "dz", "dB", "dC", "dA", "dD", "ddt_bias", "dconv_w", "dconv_b", "dh0", "dconv0"):
        check(k, got[k], ref[k])


def test_long_prompt_conv_silu_alone():
    """The conv-only entry point on the long prompt (the launch bench.py times)."""
    seed = synth.seed_for(2)
    print("case: conv alone, batch 1 L 131072", flush=True)
    p = synth.make_params(seed, D, N)
    tk = synth.make_tokens(seed, (1, 131072), D, N, "bf16")
    cb = (0.1 * np.random.default_rng(seed).standard_normal(D)).astype(np.float32)
    u, cf = ss.conv_silu(bf16(tk.x), tf32(p.conv_w, DEV), tf32(cb, DEV))
    chans = sample_channels(seed)
    ci = torch.from_numpy(chans).to(DEV)
    ug = u.index_select(2, ci).float().cpu().numpy()
    cg = cf.index_select(2, ci).float().cpu().numpy()
    torch.cuda.synchronize()
    ur, cr = oracle.conv_silu(tk.x, p.conv_w, cb, chans=chans)
    check("u", ug, ur)
    np.testing.assert_array_equal(cg, cr)


def test_long_prompt_is_bitwise_deterministic():
    seed = synth.seed_for(2)
    p = synth.make_params(seed, D, N)
    tk = synth.make_tokens(seed, (1, 131072), D, N, "bf16")
    ins = [bf16(a) for a in (tk.x, tk.dt, tk.B, tk.C, tk.z)]
    prm = params_dev(p)
    y1, h1, c1 = ss.prefill(*ins, *prm)
    y2, h2, c2 = ss.prefill(*ins, *prm)
    assert torch.equal(y1, y2) and torch.equal(h1, h2) and torch.equal(c1, c2)


def test_packed_varlen_8_sequences():
    seed = synth.seed_for(4)
    lens = synth.varlen_lengths(seed)
    cu = synth.cu_from_lengths(lens)
    T = int(cu[-1])
    print("case: varlen lengths", lens.tolist(), "total", T, flush=True)
    assert T <= 131072 and lens.min() >= 1024 and lens.max() <= 32768
    p = synth.make_params(seed, D, N)
    tk = synth.make_tokens(seed, (T,), D, N, "bf16")
    y, hf, cf = ss.varlen(torch.from_numpy(cu).to(DEV), bf16(tk.x), bf16(tk.dt), bf16(tk.B), bf16(tk.C),
                          bf16(tk.z), *params_dev(p), max_seqlen=int(lens.max()))
    chans = sample_channels(seed)
    ci = torch.from_numpy(chans).to(DEV)
    yg = y.index_select(1, ci).float().cpu().numpy()
    hg = hf.index_select(1, ci).cpu().numpy()
    cg = cf.index_select(2, ci).float().cpu().numpy()
    torch.cuda.synchronize()
    yr, hr, cr = oracle.varlen(cu, tk.x, tk.dt, tk.B, tk.C, tk.z, p.A, p.Dskip, p.dt_bias, p.conv_w, p.conv_b,
                               chans=chans)
    check("y", yg, yr)
    check("h_final", hg, hr)
    np.testing.assert_array_equal(cg, cr)


def test_streaming_decode_256_sequences_65536_steps():
    """256 resident sequences, 65536 single-token steps.  Step inputs cycle through a pool
    of 256 pre-drawn steps.  The starting state of the sampled (sequence, channel) pairs is
    the oracle's state after a random 1024-token prefill; other entries start from a random
    state of the same shape (channels and sequences are independent).  The oracle runs the
    sampled sequences as one long prefill over the same token stream (decode steps equal
    a prefill exactly in the oracle)."""
    seed = synth.seed_for(3)
    S, steps, P, Lw = 256, 65536, 256, 1024
    p = synth.make_params(seed, D, N)
    seqs = np.array([0, 1, 77, 128, 200, 255])
    chans = sample_channels(seed, k_random=6)
    # starting state
    h0, conv0 = synth.make_state(seed, S, D, N, "bf16", scale=0.1, tag="bg")
    warm = synth.make_tokens(seed, (len(seqs), Lw), D, N, "bf16", tag="warm")
    _, hw, cw = oracle.prefill(warm.x, warm.dt, warm.B, warm.C, warm.z, p.A, p.Dskip, p.dt_bias, p.conv_w,
                               p.conv_b, chans=chans)
    for i, s in enumerate(seqs):
        h0[s][chans] = hw[i].astype(np.float32)
        conv0[s][:, chans] = cw[i].astype(np.float32)
    pool = synth.make_tokens(seed, (P, S), D, N, "bf16", tag="pool")
    # GPU: 65536 decode steps, gathering the sampled outputs on the device
    h = tf32(h0, DEV)
    cs = bf16(conv0)  # the ring with head 0
    heads = [torch.zeros(S, dtype=torch.int32, device=DEV), torch.zeros(S, dtype=torch.int32, device=DEV)]
    px, pdt, pz, pB, pC = (bf16(a) for a in (pool.x, pool.dt, pool.z, pool.B, pool.C))
    prm = params_dev(p)
    si = torch.from_numpy(seqs).to(DEV)
    ci = torch.from_numpy(chans).to(DEV)
    y = torch.empty((S, D), dtype=torch.bfloat16, device=DEV)
    ys = torch.empty((steps, len(seqs), len(chans)), dtype=torch.bfloat16, device=DEV)
    print("case: decode S=%d steps=%d" % (S, steps), flush=True)
    for k in range(steps):
        q = k % P
        ss.decode(px[q], pdt[q], pB[q], pC[q], pz[q], *prm, h, cs, heads[k % 2], heads[(k + 1) % 2], out=y)
        ys[k] = y.index_select(0, si).index_select(1, ci)
    hg = h.index_select(0, si).index_select(1, ci).cpu().numpy()
    cg = ordered_from_ring(cs.index_select(0, si).index_select(2, ci).float().cpu().numpy(),
                           heads[steps % 2].index_select(0, si).cpu().numpy())
    yg = ys.float().cpu().numpy()
    torch.cuda.synchronize()
    # oracle: each sampled sequence as one prefill over its step stream
    idx = np.arange(steps) % P
    pc = [a[chans] for a in (p.A, p.Dskip, p.dt_bias, p.conv_w, p.conv_b)]
    for i, s in enumerate(seqs):
        stream = lambda a: a[:, s][:, chans][idx][None]     # [1, steps, nch]
        bc = lambda a: a[:, s][idx][None]                   # [1, steps, N]
        yr, hr, cr = oracle.prefill(stream(pool.x), stream(pool.dt), bc(pool.B), bc(pool.C), stream(pool.z),
                                    *pc, h0=h0[s:s + 1][:, chans], conv0=conv0[s:s + 1][:, :, chans])
        check("seq %d y (all steps)" % s, yg[:, i, :], yr[0])
        check("seq %d h" % s, hg[i], hr[0])
        np.testing.assert_array_equal(cg[i], cr[0])
