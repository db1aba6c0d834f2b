"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, element by element.

Sizes here are small enough for the oracle to finish in seconds while spanning several
workgroups / tiles and ragged tails.  Full-size configurations are in
test_full_configs_gpu.py.
"""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_samba_amd as ss
from selective_state_space_samba_amd import synth
from tests.helpers import TOL, host, metrics, ordered_from_ring, rel_err, ring_from_ordered, tdev, tf32

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(params=["split", "single", "lane"], autouse=True)
def scan_path(request, monkeypatch):
    """Run every prefill / varlen case on each prefill kernel: the two-role and the
    single-role row kernels and the one-lane-per-channel kernel (the decode step has a
    kernel of its own)."""
    monkeypatch.setenv("SAMBA_SCAN_PATH", request.param)
    print("path:", request.param, flush=True)
    return request.param


def make_case(seed, b, L, D, N, io, random_A=False, with_state=False, gate=True):
    # nonzero conv bias throughout: every prefill path must add it
    p = synth.make_params(seed, D, N, random_A=random_A, conv_bias=True)
    tk = synth.make_tokens(seed, (b, L), D, N, io)
    h0 = conv0 = None
    if with_state:
        h0, conv0 = synth.make_state(seed, b, D, N, io, scale=0.5)
    return p, tk, h0, conv0, gate


def run_both(p, tk, h0, conv0, gate, io):
    z = tk.z if gate else None
    print("case: x", tk.x.shape, "N", tk.B.shape[-1], "io", io, "state", h0 is not None, "gate", gate, flush=True)
    y, hf, cf = ss.prefill(tdev(tk.x, io, DEV), tdev(tk.dt, io, DEV), tdev(tk.B, io, DEV), tdev(tk.C, io, DEV),
                           None if z is None else tdev(z, io, DEV), tf32(p.A, DEV), tf32(p.Dskip, DEV),
                           tf32(p.dt_bias, DEV), tf32(p.conv_w, DEV), tf32(p.conv_b, DEV),
                           None if h0 is None else tf32(h0, DEV), None if conv0 is None else tdev(conv0, io, DEV))
    torch.cuda.synchronize()
    yr, hr, cr = oracle.prefill(tk.x, tk.dt, tk.B, tk.C, z, p.A, p.Dskip, p.dt_bias, p.conv_w, p.conv_b,
                                h0=h0, conv0=conv0)
    return (host(y), host(hf), host(cf)), (yr, hr, cr)


def check(g, r, io):
    (y, hf, cf), (yr, hr, cr) = g, r
    (sy, ey), (sh, eh) = metrics(y, yr), metrics(hf, hr)
    print("  y %s\n  h %s  (tol %.0e)" % (sy, sh, TOL[io]), flush=True)
    assert ey <= TOL[io]
    assert eh <= TOL[io]
    np.testing.assert_array_equal(cf, cr)  # the conv history is a copy: bit-exact


def test_tiny_config_fp32():
    """The tiny configuration exactly: batch 1, L=512, d_inner=256, d_state=16, fp32, zero state."""
    p, tk, h0, c0, gate = make_case(synth.seed_for(0), 1, 512, 256, 16, "f32")
    check(*run_both(p, tk, h0, c0, gate, "f32"), "f32")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_ragged_with_state_random_A(io):
    p, tk, h0, c0, gate = make_case(101, 3, 333, 320, 16, io, random_A=True, with_state=True)
    check(*run_both(p, tk, h0, c0, gate, io), io)


@pytest.mark.parametrize("L", [0, 1, 2, 3, 4, 7])
@pytest.mark.parametrize("N", [1, 5, 16])
def test_short_sequences_and_small_state(L, N):
    p, tk, h0, c0, gate = make_case(200 + L + 10 * N, 2, L, 96, N, "f32", with_state=True)
    check(*run_both(p, tk, h0, c0, gate, "f32"), "f32")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_unaligned_channel_count(io):
    """d_inner = 100 is not a multiple of 8: the row kernel's 16-byte token rows do not
    apply and the one-lane-per-channel kernel serves the call."""
    p, tk, h0, c0, gate = make_case(250, 2, 70, 100, 16, io, with_state=True)
    check(*run_both(p, tk, h0, c0, gate, io), io)


def test_no_gate():
    p, tk, h0, c0, _ = make_case(300, 2, 150, 128, 16, "bf16")
    check(*run_both(p, tk, h0, c0, False, "bf16"), "bf16")


def test_chunked_prefill_carries_state():
    """Prefill in three chunks, passing h_final / conv_final forward, equals one pass."""
    io = "bf16"
    p, tk, _, _, _ = make_case(400, 2, 700, 256, 16, io)
    args = [tf32(a, DEV) for a in (p.A, p.Dskip, p.dt_bias, p.conv_w, p.conv_b)]
    h = cs = None
    ys = []
    for lo, hi in ((0, 129), (129, 130), (130, 700)):
        sl = lambda a: tdev(np.ascontiguousarray(a[:, lo:hi]), io, DEV)
        y, h, cs = ss.prefill(sl(tk.x), sl(tk.dt), sl(tk.B), sl(tk.C), sl(tk.z), *args, h, cs)
        ys.append(host(y))
    torch.cuda.synchronize()
    yr, hr, cr = oracle.prefill(tk.x, tk.dt, tk.B, tk.C, tk.z, p.A, p.Dskip, p.dt_bias, p.conv_w, p.conv_b)
    check((np.concatenate(ys, axis=1), host(h), host(cs)), (yr, hr, cr), io)


def test_inplace_state_update():
    """h_final may alias h0 and conv_final may alias conv0."""
    io = "f32"
    p, tk, h0, c0, _ = make_case(450, 2, 64, 128, 16, io, with_state=True)
    h = tf32(h0, DEV)
    cs = tdev(c0, io, DEV)
    args = [tf32(a, DEV) for a in (p.A, p.Dskip, p.dt_bias, p.conv_w, p.conv_b)]
    y, _, _ = ss.prefill(tdev(tk.x, io, DEV), tdev(tk.dt, io, DEV), tdev(tk.B, io, DEV), tdev(tk.C, io, DEV),
                         tdev(tk.z, io, DEV), *args, h, cs, h_final=h, conv_final=cs)
    torch.cuda.synchronize()
    r = oracle.prefill(tk.x, tk.dt, tk.B, tk.C, tk.z, p.A, p.Dskip, p.dt_bias, p.conv_w, p.conv_b, h0=h0, conv0=c0)
    check((host(y), host(h), host(cs)), r, io)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_varlen_ragged(io):
    lens = [0, 1, 2, 3, 5, 100, 257, 0, 64]
    cu = synth.cu_from_lengths(lens)
    T, D, N = int(cu[-1]), 192, 16
    seed = 500
    p = synth.make_params(seed, D, N, random_A=True, conv_bias=True)
    tk = synth.make_tokens(seed, (T,), D, N, io)
    h0, c0 = synth.make_state(seed, len(lens), D, N, io, scale=0.5)
    print("case: varlen", lens, io, flush=True)
    y, hf, cf = ss.varlen(torch.from_numpy(cu).to(DEV), tdev(tk.x, io, DEV), tdev(tk.dt, io, DEV),
                          tdev(tk.B, io, DEV), tdev(tk.C, io, DEV), tdev(tk.z, io, DEV), tf32(p.A, DEV),
                          tf32(p.Dskip, DEV), tf32(p.dt_bias, DEV), tf32(p.conv_w, DEV), tf32(p.conv_b, DEV),
                          tf32(h0, DEV), tdev(c0, io, DEV))
    torch.cuda.synchronize()
    r = oracle.varlen(cu, tk.x, tk.dt, tk.B, tk.C, tk.z, p.A, p.Dskip, p.dt_bias, p.conv_w, p.conv_b, h0=h0, conv0=c0)
    check((host(y), host(hf), host(cf)), r, io)


def test_varlen_sequence_order():
    """Packed batches are visited longest sequence first when there are at most 64 sequences
    (ties by index) and in index order beyond that: 40 and 70 sequences of random lengths
    with repeated lengths and empty ones, every per-sequence output checked."""
    rng = np.random.default_rng(520)
    for nseq in (40, 70):
        lens = rng.integers(0, 48, nseq).tolist()
        lens[3] = lens[5] = 47
        lens[7] = 0
        cu = synth.cu_from_lengths(lens)
        T, D, N, io = int(cu[-1]), 64, 16, "bf16"
        p = synth.make_params(520 + nseq, D, N, conv_bias=True)
        tk = synth.make_tokens(520 + nseq, (T,), D, N, io)
        h0, c0 = synth.make_state(520 + nseq, nseq, D, N, io, scale=0.5)
        print("case: varlen", nseq, "sequences", flush=True)
        y, hf, cf = ss.varlen(torch.from_numpy(cu).to(DEV), tdev(tk.x, io, DEV), tdev(tk.dt, io, DEV),
                              tdev(tk.B, io, DEV), tdev(tk.C, io, DEV), tdev(tk.z, io, DEV), tf32(p.A, DEV),
                              tf32(p.Dskip, DEV), tf32(p.dt_bias, DEV), tf32(p.conv_w, DEV), tf32(p.conv_b, DEV),
                              tf32(h0, DEV), tdev(c0, io, DEV))
        torch.cuda.synchronize()
        r = oracle.varlen(cu, tk.x, tk.dt, tk.B, tk.C, tk.z, p.A, p.Dskip, p.dt_bias, p.conv_w, p.conv_b,
                          h0=h0, conv0=c0)
        check((host(y), host(hf), host(cf)), r, io)


def test_varlen_fresh_sequences():
    """No initial state: every sequence starts from zero state and zero history."""
    lens = [17, 3, 40]
    cu = synth.cu_from_lengths(lens)
    T, D, N, io = int(cu[-1]), 64, 16, "bf16"
    p = synth.make_params(510, D, N, conv_bias=True)
    tk = synth.make_tokens(510, (T,), D, N, io)
    y, hf, cf = ss.varlen(torch.from_numpy(cu).to(DEV), tdev(tk.x, io, DEV), tdev(tk.dt, io, DEV),
                          tdev(tk.B, io, DEV), tdev(tk.C, io, DEV), tdev(tk.z, io, DEV), tf32(p.A, DEV),
                          tf32(p.Dskip, DEV), tf32(p.dt_bias, DEV), tf32(p.conv_w, DEV), tf32(p.conv_b, DEV))
    torch.cuda.synchronize()
    r = oracle.varlen(cu, tk.x, tk.dt, tk.B, tk.C, tk.z, p.A, p.Dskip, p.dt_bias, p.conv_w, p.conv_b)
    check((host(y), host(hf), host(cf)), r, io)


@pytest.mark.parametrize("io,D,gate", [("f32", 192, True), ("bf16", 192, True), ("bf16", 200, True),
                                         ("f32", 72, False)])
def test_decode_steps(io, D, gate):
    """24 decode steps on 5 sequences; D = 200 and 72 leave a partly filled last wave of 64
    channels, and z = None exercises the ungated output.  The conv ring starts with a
    different head per sequence (including values outside 0..2, taken mod 3) and the heads
    ping-pong between two buffers, so every slot is overwritten eight times."""
    S, N, steps = 5, 16, 24
    seed = 600
    p = synth.make_params(seed, D, N, random_A=True, conv_bias=True)
    h0, c0 = synth.make_state(seed, S, D, N, io, scale=0.5)
    heads0 = np.array([0, 1, 2, 5, -1], dtype=np.int32)
    h = tf32(h0, DEV)
    ring = tdev(ring_from_ordered(c0, heads0 % 3), io, DEV)
    heads = [torch.from_numpy(heads0).to(DEV), torch.full((S,), -7, dtype=torch.int32, device=DEV)]
    hr = h0.astype(np.float64).copy()
    cr = c0.astype(np.float64).copy()
    args = [tf32(a, DEV) for a in (p.A, p.Dskip, p.dt_bias, p.conv_w, p.conv_b)]
    for k in range(steps):
        st = synth.make_tokens(seed, (S,), D, N, io, tag="s%d" % k)
        hin, hout = heads[k % 2], heads[(k + 1) % 2]
        y = ss.decode(tdev(st.x, io, DEV), tdev(st.dt, io, DEV), tdev(st.B, io, DEV), tdev(st.C, io, DEV),
                      tdev(st.z, io, DEV) if gate else None, *args, h, ring, hin, hout)
        yr = oracle.decode_step(st.x, st.dt, st.B, st.C, st.z if gate else None, p.A, p.Dskip, p.dt_bias,
                                p.conv_w, p.conv_b, hr, cr)
        torch.cuda.synchronize()
        e = rel_err(host(y), yr)
        assert e <= TOL[io], "step %d err %.3e" % (k, e)
        np.testing.assert_array_equal(hout.cpu().numpy(), (heads0 % 3 + k + 1) % 3)
    assert rel_err(host(h), hr) <= TOL[io]
    np.testing.assert_array_equal(ordered_from_ring(host(ring), heads[steps % 2].cpu().numpy()), cr)


def test_decode_writes_one_ring_slot_per_step():
    """A step overwrites only the head slot of the ring (with the new input x_t): the other
    two slots are left exactly as they were; with no head_out the heads are not touched."""
    io, S, D, N = "bf16", 3, 128, 16
    seed = 650
    p = synth.make_params(seed, D, N, conv_bias=True)
    h0, c0 = synth.make_state(seed, S, D, N, io, scale=0.5)
    heads = np.array([2, 0, 1], dtype=np.int32)
    ring0 = ring_from_ordered(c0, heads)
    ring = tdev(ring0, io, DEV)
    hd = torch.from_numpy(heads).to(DEV)
    st = synth.make_tokens(seed, (S,), D, N, io, tag="one")
    args = [tf32(a, DEV) for a in (p.A, p.Dskip, p.dt_bias, p.conv_w, p.conv_b)]
    ss.decode(tdev(st.x, io, DEV), tdev(st.dt, io, DEV), tdev(st.B, io, DEV), tdev(st.C, io, DEV),
              tdev(st.z, io, DEV), *args, tf32(h0, DEV), ring, hd)
    torch.cuda.synchronize()
    got = host(ring)
    for s in range(S):
        for slot in range(3):
            want = st.x[s] if slot == heads[s] else ring0[s, slot]
            np.testing.assert_array_equal(got[s, slot], want)
    np.testing.assert_array_equal(hd.cpu().numpy(), heads)


def test_decode_continues_prefill():
    """GPU prefill then GPU decode equals the oracle's prefill then decode: the prefill's
    conv_final is the ring with head 0."""
    io = "bf16"
    b, L, D, N = 3, 300, 128, 16
    seed = 700
    p = synth.make_params(seed, D, N, conv_bias=True)
    tk = synth.make_tokens(seed, (b, L), D, N, io)
    args = [tf32(a, DEV) for a in (p.A, p.Dskip, p.dt_bias, p.conv_w, p.conv_b)]
    _, h, cs = ss.prefill(tdev(tk.x, io, DEV), tdev(tk.dt, io, DEV), tdev(tk.B, io, DEV), tdev(tk.C, io, DEV),
                          tdev(tk.z, io, DEV), *args)
    _, hr, cr = oracle.prefill(tk.x, tk.dt, tk.B, tk.C, tk.z, p.A, p.Dskip, p.dt_bias, p.conv_w, p.conv_b)
    heads = [torch.zeros(b, dtype=torch.int32, device=DEV), torch.zeros(b, dtype=torch.int32, device=DEV)]
    for k in range(5):
        st = synth.make_tokens(seed, (b,), D, N, io, tag="d%d" % k)
        y = ss.decode(tdev(st.x, io, DEV), tdev(st.dt, io, DEV), tdev(st.B, io, DEV), tdev(st.C, io, DEV),
                      tdev(st.z, io, DEV), *args, h, cs, heads[k % 2], heads[(k + 1) % 2])
        yr = oracle.decode_step(st.x, st.dt, st.B, st.C, st.z, p.A, p.Dskip, p.dt_bias, p.conv_w, p.conv_b, hr, cr)
        torch.cuda.synchronize()
        assert rel_err(host(y), yr) <= TOL[io]
    np.testing.assert_array_equal(ordered_from_ring(host(cs), heads[5 % 2].cpu().numpy()), cr)


def test_extreme_delta():
    """Delta -> 0 (dt = -60) and Delta large (dt = +40) run through the same kernels."""
    io = "f32"
    for dtv in (-60.0, 40.0):
        p, tk, h0, c0, gate = make_case(800, 1, 90, 64, 16, io, with_state=True)
        tk.dt[:] = dtv
        check(*run_both(p, tk, h0, c0, gate, io), io)


def test_run_to_run_bitwise_deterministic():
    io = "bf16"
    p, tk, h0, c0, _ = make_case(900, 2, 1000, 512, 16, io, with_state=True)
    ins = [tdev(a, io, DEV) for a in (tk.x, tk.dt, tk.B, tk.C, tk.z)]
    args = [tf32(a, DEV) for a in (p.A, p.Dskip, p.dt_bias, p.conv_w, p.conv_b)]
    ref = None
    for _ in range(5):
        y, hf, cf = ss.prefill(*ins, *args, tf32(h0, DEV), tdev(c0, io, DEV))
        cur = (y.clone(), hf.clone(), cf.clone())
        if ref is None:
            ref = cur
        else:
            for a, b in zip(ref, cur):
                assert torch.equal(a, b)


def test_invalid_arguments_raise():
    io = "bf16"
    x = torch.zeros((1, 8, 16), dtype=torch.bfloat16, device=DEV)
    Bm = torch.zeros((1, 8, 17), dtype=torch.bfloat16, device=DEV)
    A = torch.zeros((16, 17), device=DEV)
    w = torch.zeros((16, 4), device=DEV)
    with pytest.raises(ss.SambaError) as ei:
        ss.prefill(x, x, Bm, Bm, x, A, None, None, w, None)
    assert ei.value.status == 2


def _round_io(a, io):
    """Values as the I/O dtype stores them (bf16: round to nearest even), as float32."""
    a = np.asarray(a, dtype=np.float32)
    return synth.round_bf16(a) if io == "bf16" else a


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("with_state", [False, True])
def test_prefill_from_precomputed_u(io, with_state):
    """samba_scan_prefill_u: the scan from u = SiLU(conv(x)) computed beforehand (here by the
    oracle's conv, rounded to the I/O dtype), against the oracle's scan from the same u;
    ragged length, d_inner not a multiple of 64, random A."""
    p, tk, h0, _, gate = make_case(1100, 3, 333, 320, 16, io, random_A=True, with_state=with_state)
    u = _round_io(oracle.conv_silu(tk.x, p.conv_w, p.conv_b)[0], io)
    print("case: prefill_u", u.shape, io, "state", with_state, flush=True)
    y, hf = ss.prefill_u(tdev(u, io, DEV), tdev(tk.dt, io, DEV), tdev(tk.B, io, DEV), tdev(tk.C, io, DEV),
                         tdev(tk.z, io, DEV), tf32(p.A, DEV), tf32(p.Dskip, DEV), tf32(p.dt_bias, DEV),
                         None if h0 is None else tf32(h0, DEV))
    torch.cuda.synchronize()
    yr, hr = oracle.scan_u(u, tk.dt, tk.B, tk.C, tk.z, p.A, p.Dskip, p.dt_bias, h0=h0)
    ey, eh = rel_err(host(y), yr), rel_err(host(hf), hr)
    print("  y err %.3e  h err %.3e  (tol %.0e)" % (ey, eh, TOL[io]), flush=True)
    assert ey <= TOL[io] and eh <= TOL[io]


@pytest.mark.parametrize("N", [1, 5])
def test_prefill_from_u_small_state_and_short(N):
    p, tk, h0, _, _ = make_case(1150 + N, 2, 7, 96, N, "f32", with_state=True)
    u = _round_io(oracle.conv_silu(tk.x, p.conv_w, p.conv_b)[0], "f32")
    y, hf = ss.prefill_u(tdev(u, "f32", DEV), tdev(tk.dt, "f32", DEV), tdev(tk.B, "f32", DEV),
                         tdev(tk.C, "f32", DEV), None, tf32(p.A, DEV), tf32(p.Dskip, DEV), tf32(p.dt_bias, DEV),
                         tf32(h0, DEV))
    torch.cuda.synchronize()
    yr, hr = oracle.scan_u(u, tk.dt, tk.B, tk.C, None, p.A, p.Dskip, p.dt_bias, h0=h0)
    assert rel_err(host(y), yr) <= TOL["f32"] and rel_err(host(hf), hr) <= TOL["f32"]


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_varlen_from_precomputed_u(io):
    lens = [0, 1, 2, 3, 5, 100, 257, 0, 64]
    cu = synth.cu_from_lengths(lens)
    T, D, N = int(cu[-1]), 192, 16
    seed = 1200
    p = synth.make_params(seed, D, N, random_A=True, conv_bias=True)
    tk = synth.make_tokens(seed, (T,), D, N, io)
    h0, _ = synth.make_state(seed, len(lens), D, N, io, scale=0.5)
    u = _round_io(oracle.conv_silu(tk.x, p.conv_w, p.conv_b, cu_seqlens=cu)[0], io)
    print("case: varlen_u", lens, io, flush=True)
    y, hf = ss.varlen_u(torch.from_numpy(cu).to(DEV), tdev(u, io, DEV), tdev(tk.dt, io, DEV), tdev(tk.B, io, DEV),
                        tdev(tk.C, io, DEV), tdev(tk.z, io, DEV), tf32(p.A, DEV), tf32(p.Dskip, DEV),
                        tf32(p.dt_bias, DEV), tf32(h0, DEV))
    torch.cuda.synchronize()
    yr, hr = oracle.scan_u(u, tk.dt, tk.B, tk.C, tk.z, p.A, p.Dskip, p.dt_bias, h0=h0, cu_seqlens=cu)
    assert rel_err(host(y), yr) <= TOL[io] and rel_err(host(hf), hr) <= TOL[io]


def test_prefill_u_ignores_conv_parameters():
    """conv_w and conv_b are not read by the u entry points: NULL is accepted (the binding
    passes none)."""
    io = "bf16"
    p, tk, _, _, _ = make_case(1300, 1, 50, 64, 16, io)
    u = _round_io(oracle.conv_silu(tk.x, p.conv_w, p.conv_b)[0], io)
    y, _ = ss.prefill_u(tdev(u, io, DEV), tdev(tk.dt, io, DEV), tdev(tk.B, io, DEV), tdev(tk.C, io, DEV),
                        tdev(tk.z, io, DEV), tf32(p.A, DEV), None, None)
    torch.cuda.synchronize()
    yr, _ = oracle.scan_u(u, tk.dt, tk.B, tk.C, tk.z, p.A, None, None)
    assert rel_err(host(y), yr) <= TOL[io]
