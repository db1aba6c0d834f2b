"""Seeded synthetic inputs for the selective-scan core.

This module only draws random numbers; it holds none of the method's arithmetic and is
shared by the HIP path's tests/benchmark and by the CPU oracle's callers, so both sides
start from the same bytes.

Recipe (distributions are those of the parameter initialisation stated on the page
"Samba: Simple Hybrid State Space Models for Efficient Unlimited Context Language
Modeling", section 3.4: A_ij = log j (S4D-Real) used as A = -exp(A_log) as in "Samba
Guide: Hybrid Mamba & Sliding Window Architecture", Step 1; D initialised near 1; the
Delta bias placing Delta in [0.001, 0.1]):

* x, z, B, C ~ N(0, 1); conv weights ~ N(0, 0.5) (0.5 is the standard deviation);
  conv bias 0; dt ~ N(0, 0.5); D ~ N(1, 0.1);
* dt_bias[d] = softplus^-1(Delta0[d]) = log(expm1(Delta0[d])) with Delta0 log-uniform in
  [1e-3, 1e-1];
* A[d, n] = -exp(A_log[d, n]), A_log[d, n] = log(n + 1) (or, for the "random A"
  variant, A_log ~ N(log(n + 1), 0.5));
* values are drawn in float64, rounded to float32, and for bfloat16 I/O rounded to the
  nearest bfloat16 (ties to even).  Arrays are returned as float32 holding exactly the
  values the device receives.

Every tensor has its own child stream of ``SeedSequence(seed)`` keyed by its name, so a
tensor's values do not depend on which other tensors were drawn.
"""
from __future__ import annotations

import concurrent.futures
import os
import zlib
from dataclasses import dataclass

import numpy as np

_CHUNK = 1 << 22  # elements per independent child stream
_THREADS = max(1, min(16, os.cpu_count() or 1))

CONV_K = 4

CONFIGS = {
    # name: (batch, L, d_inner, d_state, io)
    "tiny": dict(batch=1, L=512, D=256, N=16, io="f32"),
    "train4k": dict(batch=4, L=4096, D=4096, N=16, io="bf16"),
    "prompt128k": dict(batch=1, L=131072, D=4096, N=16, io="bf16"),
    "decode256": dict(nseq=256, D=4096, N=16, io="bf16", steps=65536, warm_L=1024),
    "varlen8": dict(nseq=8, lo=1024, hi=32768, total_max=131072, D=4096, N=16, io="bf16"),
}


def _rng(seed: int, name: str) -> np.random.Generator:
    key = zlib.crc32(name.encode())
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, key])))


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    # leave NaN/Inf untouched (none are drawn here, but keep the function total)
    special = (u & np.uint32(0x7F800000)) == np.uint32(0x7F800000)
    r = np.where(special, u, r)
    return r.view(np.float32)


def _normal(seed, name, shape, mean=0.0, std=1.0, io="f32"):
    """Normal draws; element block c (of _CHUNK elements) comes from its own child stream
    SeedSequence([seed, crc32(name), c]), so the values do not depend on how many threads
    fill the array."""
    key = zlib.crc32(name.encode())
    out = np.empty(int(np.prod(shape)), dtype=np.float32)
    nchunk = (out.size + _CHUNK - 1) // _CHUNK

    def fill(c):
        s = c * _CHUNK
        e = min(out.size, s + _CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, key, c])))
        v = g.standard_normal(e - s)  # float64
        if std != 1.0:
            v *= std
        if mean != 0.0:
            v += mean
        out[s:e] = v
        if io == "bf16":
            out[s:e] = round_bf16(out[s:e])

    if nchunk <= 1:
        for c in range(nchunk):
            fill(c)
    else:
        with concurrent.futures.ThreadPoolExecutor(min(_THREADS, nchunk)) as ex:
            list(ex.map(fill, range(nchunk)))
    return out.reshape(shape)


@dataclass
class Params:
    A: np.ndarray        # [D, N] float32
    Dskip: np.ndarray    # [D]
    dt_bias: np.ndarray  # [D]
    conv_w: np.ndarray   # [D, 4]; tap k multiplies x[t-3+k]
    conv_b: np.ndarray   # [D]


def make_params(seed: int, D: int, N: int, random_A: bool = False, conv_bias: bool = False) -> Params:
    """Layer parameters drawn as in the workloads' recipe (conv bias 0).  conv_bias=True
    draws the conv bias ~ N(0, 0.5) instead, so that tests exercise the bias term."""
    conv_w = _normal(seed, "conv_w", (D, CONV_K), std=0.5)
    conv_b = _normal(seed, "conv_b", (D,), std=0.5) if conv_bias else np.zeros(D, dtype=np.float32)
    g = _rng(seed, "dt_bias")
    delta0 = np.exp(g.uniform(np.log(1e-3), np.log(1e-1), size=D))
    dt_bias = np.log(np.expm1(delta0)).astype(np.float32)
    Dskip = _normal(seed, "D", (D,), mean=1.0, std=0.1)
    A_log = np.tile(np.log(np.arange(1, N + 1, dtype=np.float64)), (D, 1))
    if random_A:
        A_log = A_log + 0.5 * _rng(seed, "A_log").standard_normal((D, N))
    A = (-np.exp(A_log)).astype(np.float32)
    return Params(A=A, Dskip=Dskip, dt_bias=dt_bias, conv_w=conv_w, conv_b=conv_b)


@dataclass
class Tokens:
    x: np.ndarray
    dt: np.ndarray
    z: np.ndarray
    B: np.ndarray
    C: np.ndarray


def make_tokens(seed: int, lead: tuple, D: int, N: int, io: str, tag: str = "") -> Tokens:
    """Per-token tensors with leading shape ``lead`` (e.g. (b, L) or (T,) or (S,))."""
    return Tokens(
        x=_normal(seed, tag + "x", lead + (D,), io=io),
        dt=_normal(seed, tag + "dt", lead + (D,), std=0.5, io=io),
        z=_normal(seed, tag + "z", lead + (D,), io=io),
        B=_normal(seed, tag + "B", lead + (N,), io=io),
        C=_normal(seed, tag + "C", lead + (N,), io=io),
    )


def make_state(seed: int, nseq: int, D: int, N: int, io: str, scale: float = 1.0, tag: str = ""):
    """A random resident state: h [nseq, D, N] float32 and conv history [nseq, 3, D] in
    the I/O dtype (as float32 values)."""
    h = _normal(seed, tag + "h0", (nseq, D, N), std=scale)
    hist = _normal(seed, tag + "conv0", (nseq, 3, D), io=io)
    return h, hist


def varlen_lengths(seed: int, nseq: int = 8, lo: int = 1024, hi: int = 32768, total_max: int = 131072):
    """Integer lengths uniform in [lo, hi] (inclusive); all nseq are redrawn from the same
    stream until their sum is <= total_max."""
    g = _rng(seed, "varlen_lengths")
    while True:
        lens = g.integers(lo, hi + 1, size=nseq)
        if int(lens.sum()) <= total_max:
            return lens.astype(np.int64)


def cu_from_lengths(lens) -> np.ndarray:
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    return cu


def seed_for(config_index: int) -> int:
    return 20260000 + config_index


# ---------------------------------------------------------------- whole-model stacks
# Shapes of the page's 1.7B configuration ("Samba 1.7B": 48 layers, d_m = 2048, d_p = 8196,
# 32 query heads, 4 KV heads; d_e = 2 d_m, d_r = d_m / 16, d_s = 16, w = 2048, RoPE base
# 10000).  d_ff is the stored MLP width: d_p rounded up to a multiple of 8, the extra W1/W2
# rows and W3 columns zero.
MODEL_1P7B = dict(d_model=2048, d_inner=4096, d_state=16, dt_rank=128, d_p=8196, d_ff=8200, n_heads=32,
                  n_kv_heads=4, head_dim=64, window=2048, rope_base=10000.0, norm_eps=1e-5, n_layers=48)
PATTERN = ("mamba", "mlp", "mamba", "mlp", "swa", "mlp")  # the repeating unit of the layer stack


def layer_kinds(n_layers: int):
    return [PATTERN[i % len(PATTERN)] for i in range(n_layers)]


def make_model(seed: int, cfg: dict, n_layers: int):
    """Random-initialised weights of a Samba stack (no trained weights exist here): every
    projection W^T [d_out, d_in] ~ N(0, 1/d_in), rounded to bfloat16 (the values the device
    receives); RMSNorm weights ~ N(1, 0.1); Mamba parameters as make_params.  Projections that
    read the same input are stacked: w_in_gate = [W_in; W_g], w_xproj = [W_r; W_b; W_c],
    w_qkv = [W_q; W_k; W_v], w12 = [W1; W2] (each W given as W^T, one row per output).  Returns
    (layers: list of dicts of float32 arrays, final_norm_w)."""
    dm, de, N, dr = cfg["d_model"], cfg["d_inner"], cfg["d_state"], cfg["dt_rank"]
    dp, dff = cfg.get("d_p", cfg["d_ff"]), cfg["d_ff"]
    hq, hk = cfg["n_heads"] * cfg["head_dim"], cfg["n_kv_heads"] * cfg["head_dim"]

    def w(name, dout, din):
        return _normal(seed, name, (dout, din), std=din ** -0.5, io="bf16")

    layers = []
    for i, kind in enumerate(layer_kinds(n_layers)):
        p = "L%d." % i
        ly = dict(kind=kind, norm_w=_normal(seed, p + "norm", (dm,), mean=1.0, std=0.1))
        if kind == "mamba":
            prm = make_params(seed + 7919 * (i + 1), de, N, conv_bias=True)
            ly.update(w_in_gate=np.concatenate([w(p + "w_in", de, dm), w(p + "w_gate", de, dm)]),
                      w_xproj=np.concatenate([w(p + "w_r", dr, de), w(p + "w_b", N, de), w(p + "w_c", N, de)]),
                      w_dt_up=w(p + "w_q", de, dr), w_out=w(p + "w_out", dm, de), A=prm.A, D=prm.Dskip,
                      dt_bias=prm.dt_bias, conv_w=prm.conv_w, conv_b=prm.conv_b)
        elif kind == "swa":
            ly.update(w_qkv=np.concatenate([w(p + "wq", hq, dm), w(p + "wk", hk, dm), w(p + "wv", hk, dm)]),
                      w_o=w(p + "wo", dm, hq))
        else:
            w12 = np.zeros((2 * dff, dm), dtype=np.float32)
            w12[:dp] = w(p + "w1", dp, dm)
            w12[dff:dff + dp] = w(p + "w2", dp, dm)
            w3 = np.zeros((dm, dff), dtype=np.float32)
            w3[:, :dp] = w(p + "w3", dm, dp)
            ly.update(w12=w12, w3=w3)
        layers.append(ly)
    return layers, _normal(seed, "final_norm", (dm,), mean=1.0, std=0.1)


def make_hidden(seed: int, step: int, nseq: int, d_model: int):
    """The new tokens' embeddings for one step, N(0, 1)."""
    return _normal(seed, "emb%d" % step, (nseq, d_model))
