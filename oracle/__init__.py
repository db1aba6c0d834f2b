"""fp64 CPU oracle for the Mamba selective-scan layer core (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  The product package never imports it.  The
arithmetic lives in ``samba_oracle.c`` (plain C, double precision, sequential in time);
this module only marshals numpy arrays and builds the shared object with gcc.

Functions follow, in order, the steps stated on the page "Samba: Simple Hybrid State
Space Models for Efficient Unlimited Context Language Modeling" (paper-graph-ui
summary), section 3.4, subsections "Input Projection and Short Convolution",
"Input-Dependent Selective Gating", "The State Space Model Update (S6)" and "Gated
Output", with the conv tap order / padding, A = -exp(A_log) and the SiLU(z) gate taken
from "Samba Guide: Hybrid Mamba & Sliding Window Architecture", "Step 1: The Selective
State Space (Mamba) Layer".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "samba_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A prebuilt copy of the oracle to load instead (the sanitizer test runs the pins against an
# AddressSanitizer / UndefinedBehaviorSanitizer build); it is used as is, never rebuilt.
_PREBUILT = os.environ.get("SAMBA_ORACLE_LIB") or None
if _PREBUILT:
    _LIB = _PREBUILT
_lib = None


def build(force: bool = False) -> str:
    """Compile samba_oracle.c with gcc (OpenMP) into oracle/liboracle.so."""
    if _PREBUILT:
        return _LIB
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        _declare(lib)
        _lib = lib
    return _lib


def _declare(lib):
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_softplus.restype = ctypes.c_double
    lib.oracle_softplus.argtypes = [ctypes.c_double]
    lib.oracle_silu.restype = ctypes.c_double
    lib.oracle_silu.argtypes = [ctypes.c_double]
    lib.oracle_max_threads.restype = I
    lib.oracle_scan_sequence.argtypes = [I, I, I, I, I] + [P] * 13
    lib.oracle_prefill.argtypes = [I, I, I, I] + [P] * 13
    lib.oracle_varlen.argtypes = [I, P, I, I] + [P] * 13
    lib.oracle_decode_step.argtypes = [I, I, I] + [P] * 13
    lib.oracle_scan_u_varlen.argtypes = [I, P, I, I] + [P] * 10
    lib.oracle_scan_u_varlen.restype = None
    lib.oracle_conv_silu_varlen.argtypes = [I, P, I, P, P, P, P, P]
    lib.oracle_conv_silu_varlen.restype = None
    lib.oracle_backward.argtypes = [I, P, I, I] + [P] * 27
    lib.oracle_backward.restype = None
    lib.oracle_rope.argtypes = [P, I, ctypes.c_double, ctypes.c_double]
    lib.oracle_rope.restype = None
    lib.oracle_swa.argtypes = [I, P, I, I, I, I, ctypes.c_double, P, P, P, P, P, I]
    lib.oracle_swa.restype = None
    for f in (lib.oracle_scan_sequence, lib.oracle_prefill, lib.oracle_varlen, lib.oracle_decode_step):
        f.restype = None


def _use_library(path):
    """Point the wrappers at another build of the oracle (used by the mutation tests,
    which compile deliberately broken copies to show that the pins catch them)."""
    global _lib
    _lib = None
    saved = globals()["_LIB"]
    globals()["_LIB"] = path
    try:
        return _load_nobuild()
    finally:
        globals()["_LIB"] = saved


def _load_nobuild():
    global _lib
    lib = ctypes.CDLL(_LIB)
    _declare(lib)
    _lib = lib
    return lib


def _reset():
    global _lib
    _lib = None


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data


def softplus(a: float) -> float:
    return _load().oracle_softplus(float(a))


def silu(v: float) -> float:
    return _load().oracle_silu(float(v))


def max_threads() -> int:
    return _load().oracle_max_threads()


def set_threads(n: int) -> None:
    """Thread count of the channel-parallel loops (used to time the CPU baseline)."""
    lib = _load()
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_threads(int(n))


def _params(A, Dskip, dt_bias, conv_w, conv_b, chans):
    def sel(a, axis0=True):
        if a is None:
            return None
        a = np.asarray(a)
        return _f64(a if chans is None else a[chans])
    return sel(A), sel(Dskip), sel(dt_bias), sel(conv_w), sel(conv_b)


def prefill(x, dt, B, C, z, A, Dskip, dt_bias, conv_w, conv_b, h0=None, conv0=None, chans=None):
    """Fixed-length batch.  x, dt, z: [b, L, D]; B, C: [b, L, N]; A: [D, N]; Dskip,
    dt_bias, conv_b: [D]; conv_w: [D, 4]; h0: [b, D, N] or None (zero state);
    conv0: [b, 3, D] or None (zero history, oldest first).  ``chans`` restricts the
    computation to a subset of channels (channels are independent, so the values are
    exactly those of the full computation).  Returns (y [b, L, nch], h [b, nch, N],
    hist [b, 3, nch]) in float64."""
    lib = _load()
    x = np.asarray(x)
    b, L, D = x.shape
    N = np.asarray(B).shape[-1]
    assert N <= 64
    sl = (slice(None), slice(None), chans) if chans is not None else (Ellipsis,)
    xs, dts = _f64(x[sl]), _f64(np.asarray(dt)[sl])
    zs = None if z is None else _f64(np.asarray(z)[sl])
    nch = xs.shape[2]
    Bs, Cs = _f64(B), _f64(C)
    Ap, Dp, bp, wp, cbp = _params(A, Dskip, dt_bias, conv_w, conv_b, chans)
    h = np.zeros((b, nch, N)) if h0 is None else _f64(np.asarray(h0)[:, chans, :] if chans is not None else h0).copy()
    hist = np.zeros((b, 3, nch)) if conv0 is None else _f64(np.asarray(conv0)[:, :, chans] if chans is not None else conv0).copy()
    y = np.empty((b, L, nch))
    lib.oracle_prefill(b, L, nch, N, _ptr(xs), _ptr(dts), _ptr(Bs), _ptr(Cs), _ptr(zs), _ptr(Ap),
                       _ptr(Dp), _ptr(bp), _ptr(wp), _ptr(cbp), _ptr(h), _ptr(hist), _ptr(y))
    return y, h, hist


def varlen(cu_seqlens, x, dt, B, C, z, A, Dskip, dt_bias, conv_w, conv_b, h0=None, conv0=None, chans=None):
    """Packed batch.  x, dt, z: [T, D]; B, C: [T, N]; cu_seqlens: [nseq+1] int offsets.
    Sequence s starts from h0[s] / conv0[s] (zeros if None).  Returns (y [T, nch],
    h [nseq, nch, N], hist [nseq, 3, nch])."""
    lib = _load()
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    nseq = cu.shape[0] - 1
    x = np.asarray(x)
    T, D = x.shape
    N = np.asarray(B).shape[-1]
    assert N <= 64
    sl = (slice(None), chans) if chans is not None else (Ellipsis,)
    xs, dts = _f64(x[sl]), _f64(np.asarray(dt)[sl])
    zs = None if z is None else _f64(np.asarray(z)[sl])
    nch = xs.shape[1]
    Bs, Cs = _f64(B), _f64(C)
    Ap, Dp, bp, wp, cbp = _params(A, Dskip, dt_bias, conv_w, conv_b, chans)
    h = np.zeros((nseq, nch, N)) if h0 is None else _f64(np.asarray(h0)[:, chans, :] if chans is not None else h0).copy()
    hist = np.zeros((nseq, 3, nch)) if conv0 is None else _f64(np.asarray(conv0)[:, :, chans] if chans is not None else conv0).copy()
    y = np.empty((T, nch))
    lib.oracle_varlen(nseq, _ptr(cu), nch, N, _ptr(xs), _ptr(dts), _ptr(Bs), _ptr(Cs), _ptr(zs), _ptr(Ap),
                      _ptr(Dp), _ptr(bp), _ptr(wp), _ptr(cbp), _ptr(h), _ptr(hist), _ptr(y))
    return y, h, hist


def scan_u(u, dt, B, C, z, A, Dskip, dt_bias, h0=None, cu_seqlens=None, chans=None):
    """The scan from a precomputed u = SiLU(conv(x)) (no conv).  Fixed length: u, dt, z
    [b, L, D], B, C [b, L, N], h0 [b, D, N] or None.  Packed: u, dt, z [T, D], B, C [T, N] with
    cu_seqlens [nseq+1], h0 [nseq, D, N] or None.  Returns (y shaped like u restricted to
    ``chans``, h [nseq, nch, N]) in float64."""
    lib = _load()
    u = np.asarray(u)
    if cu_seqlens is None:
        b, L, D = u.shape
        cu = (np.arange(b + 1) * L).astype(np.int32)
        flat = lambda a: None if a is None else np.asarray(a).reshape(b * L, np.asarray(a).shape[-1])
    else:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        flat = lambda a: None if a is None else np.asarray(a)
    nseq = cu.shape[0] - 1
    sel = (lambda a: a) if chans is None else (lambda a: a[:, chans])
    us, dts = _f64(sel(flat(u))), _f64(sel(flat(dt)))
    zs = None if z is None else _f64(sel(flat(z)))
    Bs, Cs = _f64(flat(B)), _f64(flat(C))
    nch, N = us.shape[1], Bs.shape[1]
    Ap, Dp, bp, _, _ = _params(A, Dskip, dt_bias, None, None, chans)
    h = np.zeros((nseq, nch, N)) if h0 is None else \
        _f64(np.asarray(h0)[:, chans, :] if chans is not None else h0).copy()
    y = np.empty_like(us)
    lib.oracle_scan_u_varlen(nseq, _ptr(cu), nch, N, _ptr(us), _ptr(dts), _ptr(Bs), _ptr(Cs), _ptr(zs), _ptr(Ap),
                             _ptr(Dp), _ptr(bp), _ptr(h), _ptr(y))
    if cu_seqlens is None:
        y = y.reshape(u.shape[0], u.shape[1], nch)
    return y, h


def decode_step(x, dt, B, C, z, A, Dskip, dt_bias, conv_w, conv_b, h, hist, chans=None):
    """One token per sequence.  x, dt, z: [S, D]; B, C: [S, N]; h: [S, nch, N] and
    hist: [S, 3, nch] (float64, already restricted to ``chans``) are updated in place.
    Returns y [S, nch]."""
    lib = _load()
    x = np.asarray(x)
    S, D = x.shape
    N = np.asarray(B).shape[-1]
    sl = (slice(None), chans) if chans is not None else (Ellipsis,)
    xs, dts = _f64(x[sl]), _f64(np.asarray(dt)[sl])
    zs = None if z is None else _f64(np.asarray(z)[sl])
    nch = xs.shape[1]
    assert h.dtype == np.float64 and h.flags.c_contiguous and h.shape == (S, nch, N)
    assert hist.dtype == np.float64 and hist.flags.c_contiguous and hist.shape == (S, 3, nch)
    Bs, Cs = _f64(B), _f64(C)
    Ap, Dp, bp, wp, cbp = _params(A, Dskip, dt_bias, conv_w, conv_b, chans)
    y = np.empty((S, nch))
    lib.oracle_decode_step(S, nch, N, _ptr(xs), _ptr(dts), _ptr(Bs), _ptr(Cs), _ptr(zs), _ptr(Ap),
                           _ptr(Dp), _ptr(bp), _ptr(wp), _ptr(cbp), _ptr(h), _ptr(hist), _ptr(y))
    return y


def conv_silu(x, conv_w, conv_b, conv0=None, cu_seqlens=None, chans=None):
    """The short convolution + SiLU alone (the activation u a full layer feeds to x_proj).
    Fixed length: x [b, L, D], conv0 [b, 3, D] or None.  Packed: x [T, D] with cu_seqlens
    [nseq+1], conv0 [nseq, 3, D] or None.  Returns (u shaped like x restricted to
    ``chans``, hist [nseq, 3, nch]) in float64; hist holds each sequence's last three
    inputs, oldest first."""
    lib = _load()
    x = np.asarray(x)
    if cu_seqlens is None:
        b, L, D = x.shape
        cu = (np.arange(b + 1) * L).astype(np.int32)
        xt = x.reshape(b * L, D)
    else:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        xt = x
    nseq = cu.shape[0] - 1
    xs = _f64(xt if chans is None else xt[:, chans])
    nch = xs.shape[1]
    _, _, _, wp, cbp = _params(None, None, None, conv_w, conv_b, chans)
    hist = np.zeros((nseq, 3, nch)) if conv0 is None else \
        _f64(np.asarray(conv0)[:, :, chans] if chans is not None else conv0).copy()
    u = np.empty_like(xs)
    lib.oracle_conv_silu_varlen(nseq, _ptr(cu), nch, _ptr(xs), _ptr(wp), _ptr(cbp), _ptr(hist), _ptr(u))
    if cu_seqlens is None:
        u = u.reshape(x.shape[0], x.shape[1], nch)
    return u, hist


def backward(x, dt, B, C, z, A, Dskip, dt_bias, conv_w, conv_b, dout, h0=None, conv0=None,
             dh_final=None, dconv_final=None, cu_seqlens=None, chans=None):
    """Gradients of the layer (reverse-mode, from the same formulas as ``prefill``).  The
    incoming gradients are dout (shaped like x), dh_final [nseq, D, N] and dconv_final
    [nseq, 3, D] (None = zero).  Fixed length: x, dt, z, dout [b, L, D], B, C [b, L, N];
    packed: [T, D] / [T, N] with cu_seqlens.  ``chans`` restricts the channels: token and
    parameter gradients of those channels are exact, while dB and dC (sums over all
    channels) are then only those channels' share.  Returns a dict of float64 arrays: dx,
    ddt, dz (shaped like x, restricted to chans; dz None without a gate), dB, dC (shaped
    like B), dA [nch, N], dD, ddt_bias, dconv_b [nch], dconv_w [nch, 4], dh0 [nseq, nch, N],
    dconv0 [nseq, 3, nch]."""
    lib = _load()
    x = np.asarray(x)
    fixed = cu_seqlens is None
    if fixed:
        b, L, D = x.shape
        cu = (np.arange(b + 1) * L).astype(np.int32)
        flat = lambda a: None if a is None else np.asarray(a).reshape((b * L,) + np.asarray(a).shape[2:])
    else:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        flat = lambda a: None if a is None else np.asarray(a)
    nseq = cu.shape[0] - 1
    T = int(cu[-1])
    N = np.asarray(B).shape[-1]
    assert N <= 64
    sel = (lambda a: None if a is None else _f64(a if chans is None else a[:, chans]))
    xs, dts, zs, gs = sel(flat(x)), sel(flat(dt)), sel(flat(z)), sel(flat(dout))
    nch = xs.shape[1]
    Bs, Cs = _f64(flat(B)), _f64(flat(C))
    Ap, Dp, bp, wp, cbp = _params(A, Dskip, dt_bias, conv_w, conv_b, chans)
    per_seq = lambda a, shape, ax: np.zeros(shape) if a is None else \
        _f64(np.take(np.asarray(a), chans, axis=ax) if chans is not None else a)
    h0s = per_seq(h0, (nseq, nch, N), 1)
    c0s = per_seq(conv0, (nseq, 3, nch), 2)
    dhf = None if dh_final is None else per_seq(dh_final, None, 1)
    dcf = None if dconv_final is None else per_seq(dconv_final, None, 2)
    out = dict(dx=np.zeros((T, nch)), ddt=np.zeros((T, nch)), dz=None if zs is None else np.zeros((T, nch)),
               dB=np.zeros((T, N)), dC=np.zeros((T, N)), dA=np.zeros((nch, N)), dD=np.zeros(nch),
               ddt_bias=np.zeros(nch), dconv_w=np.zeros((nch, 4)), dconv_b=np.zeros(nch),
               dh0=np.zeros((nseq, nch, N)), dconv0=np.zeros((nseq, 3, nch)))
    lib.oracle_backward(nseq, _ptr(cu), nch, N, _ptr(xs), _ptr(dts), _ptr(Bs), _ptr(Cs), _ptr(zs), _ptr(Ap),
                        _ptr(Dp), _ptr(bp), _ptr(wp), _ptr(cbp), _ptr(h0s), _ptr(c0s), _ptr(gs), _ptr(dhf), _ptr(dcf),
                        *[_ptr(out[k]) for k in ("dx", "ddt", "dz", "dB", "dC", "dA", "dD", "ddt_bias", "dconv_w",
                                                 "dconv_b", "dh0", "dconv0")])
    if fixed:
        for k in ("dx", "ddt", "dz"):
            if out[k] is not None:
                out[k] = out[k].reshape(b, L, nch)
        for k in ("dB", "dC"):
            out[k] = out[k].reshape(b, L, N)
    return out


def rope(vec, pos, base=10000.0):
    """RoPE of one head vector at position pos (pairs (2i, 2i+1), angle pos * base^(-2i/dh))."""
    v = _f64(np.array(vec, dtype=np.float64))
    _load().oracle_rope(_ptr(v), v.shape[0], float(pos), float(base))
    return v


def swa(q, k, v, window=2048, base=10000.0, cu_seqlens=None, rows=None):
    """Sliding window attention with RoPE and grouped KV heads.  Fixed length: q [b, L, Hq, dh],
    k, v [b, L, Hkv, dh]; packed: [T, H, dh] with cu_seqlens.  ``rows`` (flat token indices)
    restricts the computed query tokens; other output rows are NaN.  Returns out shaped like q
    (float64)."""
    lib = _load()
    q = np.asarray(q)
    fixed = cu_seqlens is None
    if fixed:
        b, L = q.shape[:2]
        cu = (np.arange(b + 1) * L).astype(np.int32)
        flat = lambda a: np.asarray(a).reshape((b * L,) + np.asarray(a).shape[2:])
    else:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        flat = lambda a: np.asarray(a)
    qs, ks, vs = _f64(flat(q)), _f64(flat(k)), _f64(flat(v))
    T, Hq, dh = qs.shape
    Hkv = ks.shape[1]
    assert Hq % Hkv == 0 and dh % 2 == 0
    out = np.full((T, Hq, dh), np.nan)
    rr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    lib.oracle_swa(cu.shape[0] - 1, _ptr(cu), Hq, Hkv, dh, int(window), float(base), _ptr(qs), _ptr(ks), _ptr(vs),
                   _ptr(out), _ptr(rr), 0 if rr is None else rr.shape[0])
    return out.reshape(q.shape) if fixed else out


def timed(fn, *args, **kw):
    t0 = time.perf_counter()
    out = fn(*args, **kw)
    return out, time.perf_counter() - t0
