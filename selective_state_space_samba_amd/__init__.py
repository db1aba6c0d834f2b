"""MI355X (gfx950) selective-scan core of a Mamba layer -- Python binding.

A thin ctypes layer over ``libsamba_scan.so`` (C ABI declared in
``include/samba_scan.h``).  It only marshals torch tensors into device pointers, sizes
and the current HIP stream; every step of the computation runs in the library's HIP
kernels.  There is no CPU or PyTorch fallback: if the library is missing the calls raise.

Entry points mirror the C ABI: ``prefill``, ``prefill_u``, ``varlen``, ``varlen_u``, ``decode``, ``conv_silu``,
``backward``, ``swa`` (sliding window attention), ``swa_decode`` and ``swa_kv_fill``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

__all__ = ["prefill", "prefill_u", "varlen", "varlen_u", "decode", "conv_silu", "backward", "swa", "swa_decode", "swa_kv_fill", "gemm", "rmsnorm",
           "decode_step", "decode_step_workspace_bytes",
           "workspace_bytes", "lib_path", "SambaError", "version"]

_PKG = os.path.dirname(os.path.abspath(__file__))
# SAMBA_LIB names another build of the same sources to load instead (the sanitizer test loads
# a host-AddressSanitizer / UndefinedBehaviorSanitizer build this way).
LIB_PATH = os.environ.get("SAMBA_LIB") or os.path.join(_PKG, "libsamba_scan.so")
_lib = None

SAMBA_F32, SAMBA_BF16 = 0, 1
GEMM_EPILOGUES = {"store": 0, "add": 1, "swiglu": 2}
_STATUS = {0: "OK", 1: "SAMBA_ERR_INVALID_ARG", 2: "SAMBA_ERR_UNSUPPORTED", 3: "SAMBA_ERR_WORKSPACE", 4: "SAMBA_ERR_HIP"}


class SambaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (_STATUS.get(status, str(status)), msg))
        self.status = status


class Params(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("D", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
                ("conv_w", ctypes.c_void_p), ("conv_b", ctypes.c_void_p)]


class ModelConfig(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int), ("d_inner", ctypes.c_int), ("d_state", ctypes.c_int),
                ("dt_rank", ctypes.c_int), ("d_ff", ctypes.c_int), ("n_heads", ctypes.c_int),
                ("n_kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int), ("window", ctypes.c_int),
                ("rope_base", ctypes.c_float), ("norm_eps", ctypes.c_float)]


LAYER_KINDS = {"mamba": 0, "swa": 1, "mlp": 2}
_LAYER_PTRS = ("norm_w", "w_in_gate", "w_xproj", "w_dt_up", "w_out")
_LAYER_PTRS2 = ("h", "conv_state", "w_qkv", "w_o", "k_cache", "v_cache", "w12", "w3")


class Layer(ctypes.Structure):
    _fields_ = ([("kind", ctypes.c_int)] + [(n, ctypes.c_void_p) for n in _LAYER_PTRS] + [("ssm", Params)] +
                [(n, ctypes.c_void_p) for n in _LAYER_PTRS2])


def lib_path() -> str:
    return LIB_PATH


def load():
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libsamba_scan.so is not built (run __graft_entry__.build()); "
                               "there is no fallback path")
        lib = ctypes.CDLL(LIB_PATH)
        P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        lib.samba_last_error.restype = ctypes.c_char_p
        lib.samba_version.restype = ctypes.c_char_p
        lib.samba_scan_workspace_bytes.restype = Z
        lib.samba_scan_workspace_bytes.argtypes = [I, I, I, I]
        lib.samba_scan_prefill.restype = I
        lib.samba_scan_prefill.argtypes = [I, I, I, I, I, P, P, P, P, P, ctypes.POINTER(Params), P, P, P, P, P, P, Z, P]
        lib.samba_scan_prefill_u.restype = I
        lib.samba_scan_prefill_u.argtypes = [I, I, I, I, I, P, P, P, P, P, ctypes.POINTER(Params), P, P, P, P, Z, P]
        lib.samba_scan_varlen_u.restype = I
        lib.samba_scan_varlen_u.argtypes = [I, P, I, I, I, I, I, P, P, P, P, P, ctypes.POINTER(Params), P, P, P, P, Z,
                                            P]
        lib.samba_scan_varlen.restype = I
        lib.samba_scan_varlen.argtypes = [I, P, I, I, I, I, I, P, P, P, P, P, ctypes.POINTER(Params), P, P, P, P, P,
                                          P, Z, P]
        lib.samba_scan_decode.restype = I
        lib.samba_scan_decode.argtypes = [I, I, I, I, P, P, P, P, P, ctypes.POINTER(Params), P, P, P, P, P, P]
        lib.samba_scan_backward_workspace_bytes.restype = Z
        lib.samba_scan_backward_workspace_bytes.argtypes = [I, I, I, I, I]
        lib.samba_scan_backward.restype = I
        lib.samba_scan_backward.argtypes = [I, P, I, I, I, I, I, P, P, P, P, P, ctypes.POINTER(Params), P, P, P, P, P,
                                            P, P, P, P, P, P, P, P, P, P, P, P, P, Z, P]
        lib.samba_swa_workspace_bytes.restype = Z
        lib.samba_swa_workspace_bytes.argtypes = [I, I, I]
        lib.samba_swa_prefill.restype = I
        lib.samba_swa_prefill.argtypes = [I, P, I, I, I, I, I, I, ctypes.c_float, I, P, P, P, P, P, Z, P]
        lib.samba_swa_decode_workspace_bytes.restype = Z
        lib.samba_swa_decode_workspace_bytes.argtypes = [I, I, I]
        lib.samba_swa_decode.restype = I
        lib.samba_swa_decode.argtypes = [I, I, I, I, I, ctypes.c_float, I, P, P, P, P, P, P, P, P, Z, P]
        lib.samba_swa_decode_noalloc.restype = I
        lib.samba_swa_decode_noalloc.argtypes = [I, I, I, I, I, ctypes.c_float, I, P, P, P, P, P, P, P, P]
        lib.samba_swa_decode_noalloc_max_bytes.restype = Z
        lib.samba_swa_decode_noalloc_max_bytes.argtypes = []
        lib.samba_swa_kv_fill.restype = I
        lib.samba_swa_kv_fill.argtypes = [I, P, I, I, I, I, I, ctypes.c_float, I, P, P, P, P, P]
        lib.samba_conv_silu.restype = I
        lib.samba_conv_silu.argtypes = [I, P, I, I, I, I, P, P, P, P, P, P, P]
        lib.samba_rmsnorm.restype = I
        lib.samba_rmsnorm.argtypes = [I, I, P, P, ctypes.c_float, P, P]
        lib.samba_decode_step_workspace_bytes.restype = Z
        lib.samba_decode_step_workspace_bytes.argtypes = [ctypes.POINTER(ModelConfig), I]
        lib.samba_decode_step.restype = I
        lib.samba_decode_step.argtypes = [ctypes.POINTER(ModelConfig), I, ctypes.POINTER(Layer), P, I, P, P, P, P, P,
                                          Z, P]
        lib.samba_gemm_workspace_bytes.restype = Z
        lib.samba_gemm_workspace_bytes.argtypes = [I, I, I, I]
        lib.samba_gemm.restype = I
        lib.samba_gemm.argtypes = [I, I, I, I, P, I, P, P, I, P, I, P, Z, P]
        _lib = lib
    return _lib


def version() -> str:
    return load().samba_version().decode()


def _io(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SAMBA_F32
    if t.dtype == torch.bfloat16:
        return SAMBA_BF16
    raise TypeError("I/O tensors must be float32 or bfloat16, got %s" % t.dtype)


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, device=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if device is not None and t.device != device:
        raise ValueError("%s must be on %s, got %s" % (name, device, t.device))
    return t.data_ptr() if t.numel() > 0 else None


def _shape(t, shape, name):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _params(A, Dskip, dt_bias, conv_w, conv_b, dev, D, N, needs_conv=True):
    f = torch.float32
    if A is None or (needs_conv and conv_w is None):
        raise ValueError("A and conv_w are required")
    _shape(A, (D, N), "A")
    _shape(Dskip, (D,), "Dskip")
    _shape(dt_bias, (D,), "dt_bias")
    _shape(conv_w, (D, 4), "conv_w")
    _shape(conv_b, (D,), "conv_b")
    return Params(_ptr(A, "A", f, dev), _ptr(Dskip, "Dskip", f, dev), _ptr(dt_bias, "dt_bias", f, dev),
                  _ptr(conv_w, "conv_w", f, dev), _ptr(conv_b, "conv_b", f, dev))


def _gpu_device(x: torch.Tensor) -> torch.device:
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
        raise ValueError("inputs must be tensors on a GPU (got %s); the library has no CPU path"
                         % (getattr(x, "device", type(x))))
    return x.device


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def _check(st: int):
    if st != 0:
        raise SambaError(st, load().samba_last_error().decode())


def workspace_bytes(nseq: int, max_seqlen: int, d_inner: int, d_state: int) -> int:
    return int(load().samba_scan_workspace_bytes(nseq, max_seqlen, d_inner, d_state))


def _workspace(nseq, max_seqlen, D, N, dev, workspace):
    need = workspace_bytes(nseq, max_seqlen, D, N)
    if need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    return workspace, workspace.numel() * workspace.element_size()


def prefill(x, dt, B, C, z, A, Dskip, dt_bias, conv_w, conv_b, h0=None, conv0=None, *,
            out=None, h_final=None, conv_final=None, want_state=True, workspace=None):
    """Fixed-length prefill.  x, dt, z: [b, L, D]; B, C: [b, L, N] (float32 or bfloat16, all
    the same dtype, on one GPU); A [D, N], Dskip/dt_bias/conv_b [D], conv_w [D, 4] float32;
    h0 [b, D, N] float32 or None; conv0 [b, 3, D] (I/O dtype) or None.  Returns
    (out, h_final, conv_final); the last two are None when want_state is False."""
    dev = _gpu_device(x)
    b, L, D = x.shape
    N = B.shape[-1]
    io = _io(x)
    if out is None:
        out = torch.empty_like(x)
    if want_state and h_final is None:
        h_final = torch.empty((b, D, N), dtype=torch.float32, device=dev)
    if want_state and conv_final is None:
        conv_final = torch.empty((b, 3, D), dtype=x.dtype, device=dev)
    for t, n in ((dt, "dt"), (z, "z"), (out, "out")):
        _shape(t, (b, L, D), n)
    _shape(C, (b, L, N), "C")
    _shape(h0, (b, D, N), "h0")
    _shape(h_final, (b, D, N), "h_final")
    _shape(conv0, (b, 3, D), "conv0")
    _shape(conv_final, (b, 3, D), "conv_final")
    p = _params(A, Dskip, dt_bias, conv_w, conv_b, dev, D, N)
    ws, wsb = _workspace(b, L, D, N, dev, workspace)
    st = load().samba_scan_prefill(
        b, L, D, N, io, _ptr(x, "x", x.dtype, dev), _ptr(dt, "dt", x.dtype, dev), _ptr(B, "B", x.dtype, dev),
        _ptr(C, "C", x.dtype, dev), _ptr(z, "z", x.dtype, dev), ctypes.byref(p),
        _ptr(h0, "h0", torch.float32, dev), _ptr(conv0, "conv0", x.dtype, dev), _ptr(out, "out", x.dtype, dev),
        _ptr(h_final, "h_final", torch.float32, dev), _ptr(conv_final, "conv_final", x.dtype, dev),
        _ptr(ws, "workspace"), wsb, _stream(dev))
    _check(st)
    return out, h_final, conv_final


def prefill_u(u, dt, B, C, z, A, Dskip, dt_bias, h0=None, *, out=None, h_final=None, want_state=True,
              workspace=None):
    """Fixed-length prefill from a precomputed u = SiLU(conv(x)) (samba_scan_prefill_u: the
    activation a full layer computes once for x_proj, see conv_silu).  u, dt, z: [b, L, D];
    B, C: [b, L, N]; A [D, N], Dskip/dt_bias [D] float32; h0 [b, D, N] or None.  Returns
    (out, h_final); h_final is None when want_state is False."""
    dev = _gpu_device(u)
    b, L, D = u.shape
    N = B.shape[-1]
    io = _io(u)
    if out is None:
        out = torch.empty_like(u)
    if want_state and h_final is None:
        h_final = torch.empty((b, D, N), dtype=torch.float32, device=dev)
    for t, n in ((dt, "dt"), (z, "z"), (out, "out")):
        _shape(t, (b, L, D), n)
    _shape(B, (b, L, N), "B")
    _shape(C, (b, L, N), "C")
    _shape(h0, (b, D, N), "h0")
    _shape(h_final, (b, D, N), "h_final")
    p = _params(A, Dskip, dt_bias, None, None, dev, D, N, needs_conv=False)
    ws, wsb = _workspace(b, L, D, N, dev, workspace)
    st = load().samba_scan_prefill_u(
        b, L, D, N, io, _ptr(u, "u", u.dtype, dev), _ptr(dt, "dt", u.dtype, dev), _ptr(B, "B", u.dtype, dev),
        _ptr(C, "C", u.dtype, dev), _ptr(z, "z", u.dtype, dev), ctypes.byref(p),
        _ptr(h0, "h0", torch.float32, dev), _ptr(out, "out", u.dtype, dev),
        _ptr(h_final, "h_final", torch.float32, dev), _ptr(ws, "workspace"), wsb, _stream(dev))
    _check(st)
    return out, h_final


def varlen_u(cu_seqlens, u, dt, B, C, z, A, Dskip, dt_bias, h0=None, *, max_seqlen=None, out=None, h_final=None,
             workspace=None):
    """Packed variable-length prefill from a precomputed u (samba_scan_varlen_u); layouts as
    for varlen.  Returns (out, h_final [nseq, D, N])."""
    dev = _gpu_device(u)
    T, D = u.shape
    N = B.shape[-1]
    nseq = cu_seqlens.numel() - 1
    io = _io(u)
    if max_seqlen is None:
        max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if nseq > 0 else 0
    if out is None:
        out = torch.empty_like(u)
    if h_final is None:
        h_final = torch.empty((nseq, D, N), dtype=torch.float32, device=dev)
    for t, n in ((dt, "dt"), (z, "z"), (out, "out")):
        _shape(t, (T, D), n)
    _shape(B, (T, N), "B")
    _shape(C, (T, N), "C")
    _shape(cu_seqlens, (nseq + 1,), "cu_seqlens")
    _shape(h0, (nseq, D, N), "h0")
    _shape(h_final, (nseq, D, N), "h_final")
    p = _params(A, Dskip, dt_bias, None, None, dev, D, N, needs_conv=False)
    ws, wsb = _workspace(nseq, max_seqlen, D, N, dev, workspace)
    st = load().samba_scan_varlen_u(
        nseq, _ptr(cu_seqlens, "cu_seqlens", torch.int32, dev), T, int(max_seqlen), D, N, io,
        _ptr(u, "u", u.dtype, dev), _ptr(dt, "dt", u.dtype, dev), _ptr(B, "B", u.dtype, dev),
        _ptr(C, "C", u.dtype, dev), _ptr(z, "z", u.dtype, dev), ctypes.byref(p),
        _ptr(h0, "h0", torch.float32, dev), _ptr(out, "out", u.dtype, dev),
        _ptr(h_final, "h_final", torch.float32, dev), _ptr(ws, "workspace"), wsb, _stream(dev))
    _check(st)
    return out, h_final


def varlen(cu_seqlens, x, dt, B, C, z, A, Dskip, dt_bias, conv_w, conv_b, h0=None, conv0=None, *,
           max_seqlen=None, out=None, h_final=None, conv_final=None, workspace=None):
    """Packed variable-length prefill.  cu_seqlens: int32 [nseq+1] on the GPU; x, dt, z:
    [T, D]; B, C: [T, N].  ``max_seqlen`` (host int) is computed from cu_seqlens when not
    given (that costs a device-to-host copy).  Returns (out, h_final [nseq, D, N],
    conv_final [nseq, 3, D])."""
    dev = _gpu_device(x)
    T, D = x.shape
    N = B.shape[-1]
    nseq = cu_seqlens.numel() - 1
    io = _io(x)
    if max_seqlen is None:
        max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if nseq > 0 else 0
    if out is None:
        out = torch.empty_like(x)
    if h_final is None:
        h_final = torch.empty((nseq, D, N), dtype=torch.float32, device=dev)
    if conv_final is None:
        conv_final = torch.empty((nseq, 3, D), dtype=x.dtype, device=dev)
    for t, n in ((dt, "dt"), (z, "z"), (out, "out")):
        _shape(t, (T, D), n)
    _shape(B, (T, N), "B")
    _shape(C, (T, N), "C")
    _shape(cu_seqlens, (nseq + 1,), "cu_seqlens")
    _shape(h0, (nseq, D, N), "h0")
    _shape(h_final, (nseq, D, N), "h_final")
    _shape(conv0, (nseq, 3, D), "conv0")
    _shape(conv_final, (nseq, 3, D), "conv_final")
    p = _params(A, Dskip, dt_bias, conv_w, conv_b, dev, D, N)
    ws, wsb = _workspace(nseq, max_seqlen, D, N, dev, workspace)
    st = load().samba_scan_varlen(
        nseq, _ptr(cu_seqlens, "cu_seqlens", torch.int32, dev), T, int(max_seqlen), D, N, io,
        _ptr(x, "x", x.dtype, dev), _ptr(dt, "dt", x.dtype, dev), _ptr(B, "B", x.dtype, dev),
        _ptr(C, "C", x.dtype, dev), _ptr(z, "z", x.dtype, dev), ctypes.byref(p),
        _ptr(h0, "h0", torch.float32, dev), _ptr(conv0, "conv0", x.dtype, dev), _ptr(out, "out", x.dtype, dev),
        _ptr(h_final, "h_final", torch.float32, dev), _ptr(conv_final, "conv_final", x.dtype, dev),
        _ptr(ws, "workspace"), wsb, _stream(dev))
    _check(st)
    return out, h_final, conv_final


def decode(x, dt, B, C, z, A, Dskip, dt_bias, conv_w, conv_b, h, conv_ring, ring_head_in, ring_head_out=None, *,
           out=None):
    """One decode step for S sequences: x, dt, z [S, D]; B, C [S, N]; h [S, D, N] float32
    and the conv ring [S, 3, D] (I/O dtype) are updated in place; ring_head_in int32 [S] (the
    slot of each sequence's oldest input) is read, and ring_head_out int32 [S] (optional, a
    different tensor) receives the next heads.  Returns out [S, D]."""
    dev = _gpu_device(x)
    S, D = x.shape
    N = B.shape[-1]
    io = _io(x)
    if out is None:
        out = torch.empty_like(x)
    for t, n in ((dt, "dt"), (z, "z"), (out, "out")):
        _shape(t, (S, D), n)
    _shape(B, (S, N), "B")
    _shape(C, (S, N), "C")
    _shape(h, (S, D, N), "h")
    _shape(conv_ring, (S, 3, D), "conv_ring")
    _shape(ring_head_in, (S,), "ring_head_in")
    _shape(ring_head_out, (S,), "ring_head_out")
    p = _params(A, Dskip, dt_bias, conv_w, conv_b, dev, D, N)
    st = load().samba_scan_decode(
        S, D, N, io, _ptr(x, "x", x.dtype, dev), _ptr(dt, "dt", x.dtype, dev), _ptr(B, "B", x.dtype, dev),
        _ptr(C, "C", x.dtype, dev), _ptr(z, "z", x.dtype, dev), ctypes.byref(p),
        _ptr(h, "h", torch.float32, dev), _ptr(conv_ring, "conv_ring", x.dtype, dev),
        _ptr(ring_head_in, "ring_head_in", torch.int32, dev), _ptr(ring_head_out, "ring_head_out", torch.int32, dev),
        _ptr(out, "out", x.dtype, dev), _stream(dev))
    _check(st)
    return out


def conv_silu(x, conv_w, conv_b=None, conv0=None, *, cu_seqlens=None, max_seqlen=None, out=None,
              conv_final=None, want_state=True):
    """The short causal conv + SiLU alone: u = SiLU(conv_b + sum_k conv_w[:, k] x_{t-3+k}),
    the activation a full layer feeds to x_proj.  Fixed length: x [b, L, D], conv0
    [b, 3, D] or None.  Packed: x [T, D] with cu_seqlens (int32 [nseq+1] on the GPU) and
    ``max_seqlen`` (computed from cu_seqlens when not given, at the cost of a copy to the
    host).  conv_w [D, 4], conv_b [D] float32.  Returns (u, conv_final [nseq, 3, D] or
    None when want_state is False)."""
    dev = _gpu_device(x)
    io = _io(x)
    f = torch.float32
    if cu_seqlens is None:
        b, L, D = x.shape
        nseq, total = b, b * L
    else:
        T, D = x.shape
        nseq = cu_seqlens.numel() - 1
        total = T
        _shape(cu_seqlens, (nseq + 1,), "cu_seqlens")
        if max_seqlen is None:
            max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if nseq > 0 else 0
        L = int(max_seqlen)
    if out is None:
        out = torch.empty_like(x)
    if want_state and conv_final is None:
        conv_final = torch.empty((nseq, 3, D), dtype=x.dtype, device=dev)
    _shape(out, tuple(x.shape), "out")
    _shape(conv_w, (D, 4), "conv_w")
    _shape(conv_b, (D,), "conv_b")
    _shape(conv0, (nseq, 3, D), "conv0")
    _shape(conv_final, (nseq, 3, D), "conv_final")
    st = load().samba_conv_silu(
        nseq, _ptr(cu_seqlens, "cu_seqlens", torch.int32, dev), L, total, D, io, _ptr(x, "x", x.dtype, dev),
        _ptr(conv_w, "conv_w", f, dev), _ptr(conv_b, "conv_b", f, dev), _ptr(conv0, "conv0", x.dtype, dev),
        _ptr(out, "out", x.dtype, dev), _ptr(conv_final, "conv_final", x.dtype, dev), _stream(dev))
    _check(st)
    return out, conv_final


def backward(dout, x, dt, B, C, z, A, Dskip, dt_bias, conv_w, conv_b, h0=None, conv0=None, *,
             dh_final=None, dconv_final=None, cu_seqlens=None, max_seqlen=None, want_state_grads=True,
             workspace=None):
    """Gradients of the layer.  dout is the gradient of the output (shaped like x); dh_final
    [nseq, D, N] and dconv_final [nseq, 3, D] those of the final state and history (None =
    zero).  Fixed length: x, dt, z, dout [b, L, D], B, C [b, L, N]; packed: [T, D] / [T, N]
    with cu_seqlens (int32 [nseq+1] on the GPU) and max_seqlen.  Returns a dict: dx, ddt,
    dz (None without a gate), dB, dC (I/O dtype, shaped like their inputs), dA, dD,
    ddt_bias, dconv_w, dconv_b (float32, summed over sequences), dh0, dconv0 (None when
    want_state_grads is False)."""
    dev = _gpu_device(x)
    io = _io(x)
    f = torch.float32
    N = B.shape[-1]
    if cu_seqlens is None:
        b, L, D = x.shape
        nseq, total = b, b * L
    else:
        T, D = x.shape
        nseq = cu_seqlens.numel() - 1
        total = T
        _shape(cu_seqlens, (nseq + 1,), "cu_seqlens")
        if max_seqlen is None:
            max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if nseq > 0 else 0
        L = int(max_seqlen)
    for t, n in ((dt, "dt"), (z, "z"), (dout, "dout")):
        _shape(t, tuple(x.shape), n)
    _shape(C, tuple(B.shape), "C")
    _shape(h0, (nseq, D, N), "h0")
    _shape(conv0, (nseq, 3, D), "conv0")
    _shape(dh_final, (nseq, D, N), "dh_final")
    _shape(dconv_final, (nseq, 3, D), "dconv_final")
    p = _params(A, Dskip, dt_bias, conv_w, conv_b, dev, D, N)
    g = dict(dx=torch.empty_like(x), ddt=torch.empty_like(x), dz=None if z is None else torch.empty_like(x),
             dB=torch.empty_like(B), dC=torch.empty_like(C), dA=torch.empty((D, N), dtype=f, device=dev),
             dD=torch.empty(D, dtype=f, device=dev), ddt_bias=torch.empty(D, dtype=f, device=dev),
             dconv_w=torch.empty((D, 4), dtype=f, device=dev), dconv_b=torch.empty(D, dtype=f, device=dev),
             dh0=torch.empty((nseq, D, N), dtype=f, device=dev) if want_state_grads else None,
             dconv0=torch.empty((nseq, 3, D), dtype=x.dtype, device=dev) if want_state_grads else None)
    need = int(load().samba_scan_backward_workspace_bytes(nseq, L, total, D, N))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    wsb = workspace.numel() * workspace.element_size()
    st = load().samba_scan_backward(
        nseq, _ptr(cu_seqlens, "cu_seqlens", torch.int32, dev), L, total, D, N, io,
        _ptr(x, "x", x.dtype, dev), _ptr(dt, "dt", x.dtype, dev), _ptr(B, "B", x.dtype, dev),
        _ptr(C, "C", x.dtype, dev), _ptr(z, "z", x.dtype, dev), ctypes.byref(p),
        _ptr(h0, "h0", f, dev), _ptr(conv0, "conv0", x.dtype, dev), _ptr(dout, "dout", x.dtype, dev),
        _ptr(dh_final, "dh_final", f, dev), _ptr(dconv_final, "dconv_final", x.dtype, dev),
        *[_ptr(g[k], k) for k in ("dx", "ddt", "dB", "dC", "dz", "dA", "dD", "ddt_bias", "dconv_w", "dconv_b",
                                  "dh0", "dconv0")],
        _ptr(workspace, "workspace"), wsb, _stream(dev))
    _check(st)
    return g


def swa(q, k, v, *, window=2048, rope_base=10000.0, cu_seqlens=None, max_seqlen=None, out=None, workspace=None):
    """Sliding window attention with RoPE and grouped KV heads (bfloat16).  Fixed length:
    q [b, L, Hq, dh], k, v [b, L, Hkv, dh]; packed: [T, H, dh] with cu_seqlens (int32
    [nseq+1] on the GPU) and max_seqlen.  Returns out shaped like q."""
    dev = _gpu_device(q)
    io = _io(q)
    if cu_seqlens is None:
        b, L, Hq, dh = q.shape
        nseq, total = b, b * L
    else:
        T, Hq, dh = q.shape
        nseq = cu_seqlens.numel() - 1
        total = T
        _shape(cu_seqlens, (nseq + 1,), "cu_seqlens")
        if max_seqlen is None:
            max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if nseq > 0 else 0
        L = int(max_seqlen)
    Hkv = k.shape[-2]
    _shape(k, tuple(q.shape[:-2]) + (Hkv, dh), "k")
    _shape(v, tuple(k.shape), "v")
    if out is None:
        out = torch.empty_like(q)
    _shape(out, tuple(q.shape), "out")
    need = int(load().samba_swa_workspace_bytes(total, Hkv, dh))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = load().samba_swa_prefill(
        nseq, _ptr(cu_seqlens, "cu_seqlens", torch.int32, dev), L, total, Hq, Hkv, dh, int(window), float(rope_base),
        io, _ptr(q, "q", q.dtype, dev), _ptr(k, "k", q.dtype, dev), _ptr(v, "v", q.dtype, dev),
        _ptr(out, "out", q.dtype, dev), _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(dev))
    _check(st)
    return out


def swa_decode(q, k, v, pos, k_cache, v_cache, *, window=2048, rope_base=10000.0, out=None, workspace=None):
    """One decode step of sliding window attention: q [S, Hq, dh], k, v [S, Hkv, dh] (bf16),
    pos int32 [S] on the GPU (the new token's position), k_cache / v_cache
    [S, Hkv, window + 1, dh] ring buffers updated in place.  Returns out [S, Hq, dh]."""
    dev = _gpu_device(q)
    S, Hq, dh = q.shape
    Hkv = k.shape[1]
    _shape(k, (S, Hkv, dh), "k")
    _shape(v, (S, Hkv, dh), "v")
    _shape(pos, (S,), "pos")
    _shape(k_cache, (S, Hkv, int(window) + 1, dh), "k_cache")
    _shape(v_cache, (S, Hkv, int(window) + 1, dh), "v_cache")
    if out is None:
        out = torch.empty_like(q)
    need = int(load().samba_swa_decode_workspace_bytes(S, Hq, dh))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = load().samba_swa_decode(
        S, Hq, Hkv, dh, int(window), float(rope_base), _io(q), _ptr(q, "q", q.dtype, dev), _ptr(k, "k", q.dtype, dev),
        _ptr(v, "v", q.dtype, dev), _ptr(pos, "pos", torch.int32, dev), _ptr(k_cache, "k_cache", q.dtype, dev),
        _ptr(v_cache, "v_cache", q.dtype, dev), _ptr(out, "out", q.dtype, dev), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(dev))
    _check(st)
    return out


def swa_decode_noalloc(q, k, v, pos, k_cache, v_cache, *, window=2048, rope_base=10000.0, out=None):
    """swa_decode through samba_swa_decode_noalloc: no workspace, the split partials in the
    library's own device array (calls on one GPU must not overlap)."""
    dev = _gpu_device(q)
    S, Hq, dh = q.shape
    Hkv = k.shape[1]
    _shape(k, (S, Hkv, dh), "k")
    _shape(v, (S, Hkv, dh), "v")
    _shape(pos, (S,), "pos")
    _shape(k_cache, (S, Hkv, int(window) + 1, dh), "k_cache")
    _shape(v_cache, (S, Hkv, int(window) + 1, dh), "v_cache")
    if out is None:
        out = torch.empty_like(q)
    st = load().samba_swa_decode_noalloc(
        S, Hq, Hkv, dh, int(window), float(rope_base), _io(q), _ptr(q, "q", q.dtype, dev), _ptr(k, "k", q.dtype, dev),
        _ptr(v, "v", q.dtype, dev), _ptr(pos, "pos", torch.int32, dev), _ptr(k_cache, "k_cache", q.dtype, dev),
        _ptr(v_cache, "v_cache", q.dtype, dev), _ptr(out, "out", q.dtype, dev), _stream(dev))
    _check(st)
    return out


def swa_kv_fill(k, v, k_cache, v_cache, *, window=2048, rope_base=10000.0, cu_seqlens=None, max_seqlen=None):
    """Writes a prefill's keys (rotated) and values into the ring-buffer caches: k, v
    [b, L, Hkv, dh] or packed [T, Hkv, dh] with cu_seqlens; caches [nseq, Hkv, window + 1, dh]."""
    dev = _gpu_device(k)
    if cu_seqlens is None:
        b, L, Hkv, dh = k.shape
        nseq, total = b, b * L
    else:
        T, Hkv, dh = k.shape
        nseq, total = cu_seqlens.numel() - 1, T
        if max_seqlen is None:
            max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if nseq > 0 else 0
        L = int(max_seqlen)
    _shape(v, tuple(k.shape), "v")
    _shape(k_cache, (nseq, Hkv, int(window) + 1, dh), "k_cache")
    _shape(v_cache, (nseq, Hkv, int(window) + 1, dh), "v_cache")
    st = load().samba_swa_kv_fill(
        nseq, _ptr(cu_seqlens, "cu_seqlens", torch.int32, dev), L, total, Hkv, dh, int(window), float(rope_base),
        _io(k), _ptr(k, "k", k.dtype, dev), _ptr(v, "v", k.dtype, dev), _ptr(k_cache, "k_cache", k.dtype, dev),
        _ptr(v_cache, "v_cache", k.dtype, dev), _stream(dev))
    _check(st)


def _rows(t, name, dtype, dev):
    """Pointer and row pitch of a 2-D tensor whose rows are contiguous (stride(1) == 1)."""
    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise ValueError("%s must be a 2-D tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.device != dev:
        raise ValueError("%s must be on %s, got %s" % (name, dev, t.device))
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("%s must have contiguous rows" % name)
    ld = t.stride(0) if t.shape[0] > 1 else t.shape[1]
    return (t.data_ptr() if t.numel() > 0 else None), int(ld)


def gemm(a, w, *, epilogue="store", out=None, residual=None, workspace=None):
    """out = epilogue(a @ w.T) on the matrix cores (fp32 accumulation).
    a bf16 [M, K] (rows may be a strided view), w bf16 [N, K] ([2N, K] = [W1; W2] for
    "swiglu").  epilogue "store": out bf16 [M, N]; "add": out fp32 = residual + a @ w.T
    (residual fp32 [M, N], may be out itself); "swiglu": out bf16 = (a W1^T) * SiLU(a W2^T)."""
    dev = _gpu_device(a)
    if epilogue not in GEMM_EPILOGUES:
        raise ValueError("epilogue must be one of %s" % sorted(GEMM_EPILOGUES))
    epi = GEMM_EPILOGUES[epilogue]
    M, K = a.shape
    N = w.shape[0] // 2 if epilogue == "swiglu" else w.shape[0]
    if epilogue == "swiglu" and w.shape[0] % 2:
        raise ValueError("swiglu weight must have an even number of rows ([W1; W2])")
    _shape(w, (w.shape[0], K), "w")
    pa, lda = _rows(a, "a", torch.bfloat16, dev)
    pw = _ptr(w, "w", torch.bfloat16, dev)
    odt = torch.float32 if epilogue == "add" else torch.bfloat16
    if out is None:
        out = torch.empty((M, N), dtype=odt, device=dev)
    _shape(out, (M, N), "out")
    po, ldo = _rows(out, "out", odt, dev)
    pr, ldr = None, 0
    if epilogue == "add":
        if residual is None:
            raise ValueError("epilogue 'add' needs residual")
        _shape(residual, (M, N), "residual")
        pr, ldr = _rows(residual, "residual", torch.float32, dev)
    need = int(load().samba_gemm_workspace_bytes(M, N, K, epi))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    pws = _ptr(workspace, "workspace") if workspace is not None else None
    nws = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().samba_gemm(M, N, K, epi, pa, max(lda, K), pw, po, max(ldo, N), pr, max(ldr, N), pws, nws,
                           _stream(dev))
    _check(st)
    return out


def rmsnorm(x, weight, *, eps=1e-5, out=None):
    """out bf16 [rows, d] = x / sqrt(mean(x^2) + eps) * weight for fp32 x [rows, d]."""
    dev = _gpu_device(x)
    rows, d = x.shape
    _shape(weight, (d,), "weight")
    if out is None:
        out = torch.empty((rows, d), dtype=torch.bfloat16, device=dev)
    _shape(out, (rows, d), "out")
    _check(load().samba_rmsnorm(rows, d, _ptr(x, "x", torch.float32, dev), _ptr(weight, "weight", torch.float32, dev),
                                float(eps), _ptr(out, "out", torch.bfloat16, dev), _stream(dev)))
    return out


def _model_config(cfg):
    return ModelConfig(*(int(cfg[k]) for k in ("d_model", "d_inner", "d_state", "dt_rank", "d_ff", "n_heads",
                                                "n_kv_heads", "head_dim", "window")),
                       float(cfg.get("rope_base", 10000.0)), float(cfg.get("norm_eps", 1e-5)))


def decode_step_workspace_bytes(cfg, nseq):
    return int(load().samba_decode_step_workspace_bytes(ctypes.byref(_model_config(cfg)), int(nseq)))


class DecodeStep:
    """Marshals a Samba stack once (config, per-layer weights and decode state: dicts of GPU
    tensors keyed like the fields of samba_layer, plus "kind") and runs samba_decode_step.
    The tensors must stay alive as long as this object is used."""

    def __init__(self, cfg, layers, final_norm_w, nseq):
        self.cfg = _model_config(cfg)
        self.nseq = int(nseq)
        self.dev = _gpu_device(final_norm_w)
        arr = (Layer * max(1, len(layers)))()
        for i, ly in enumerate(layers):
            L = arr[i]
            L.kind = LAYER_KINDS[ly["kind"]]
            for n in _LAYER_PTRS + _LAYER_PTRS2:
                t = ly.get(n)
                setattr(L, n, _ptr(t, n, None, self.dev) if t is not None else None)
            if ly["kind"] == "mamba":
                L.ssm = _params(ly["A"], ly.get("D"), ly.get("dt_bias"), ly["conv_w"], ly.get("conv_b"), self.dev,
                                int(cfg["d_inner"]), int(cfg["d_state"]))
        self.layers = arr
        self.n_layers = len(layers)
        self.final_norm_w = final_norm_w
        self.ws_bytes = decode_step_workspace_bytes(cfg, nseq)
        self.workspace = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=self.dev)

    def __call__(self, hidden, pos, conv_head, out=None):
        """hidden fp32 [nseq, d_model] (updated in place), pos int32 [nseq] (advanced by one),
        conv_head int32 [nseq] (the Mamba layers' conv-ring head, advanced mod 3; None for a
        stack without Mamba layers); returns out bf16 [nseq, d_model] = the final RMSNorm of
        hidden, or None if out is False."""
        S, dm = self.nseq, self.cfg.d_model
        _shape(hidden, (S, dm), "hidden")
        _shape(pos, (S,), "pos")
        _shape(conv_head, (S,), "conv_head")
        if out is None:
            out = torch.empty((S, dm), dtype=torch.bfloat16, device=self.dev)
        po = None if out is False else _ptr(out, "out", torch.bfloat16, self.dev)
        _check(load().samba_decode_step(
            ctypes.byref(self.cfg), self.n_layers, self.layers, _ptr(self.final_norm_w, "final_norm_w", torch.float32,
                                                                     self.dev),
            S, _ptr(hidden, "hidden", torch.float32, self.dev), po, _ptr(pos, "pos", torch.int32, self.dev),
            _ptr(conv_head, "conv_head", torch.int32, self.dev),
            _ptr(self.workspace, "workspace"), self.ws_bytes, _stream(self.dev)))
        return None if out is False else out


def decode_step(cfg, layers, final_norm_w, hidden, pos, conv_head, out=None):
    """One-shot form of DecodeStep (marshals the stack on every call)."""
    return DecodeStep(cfg, layers, final_norm_w, hidden.shape[0])(hidden, pos, conv_head, out)


_F32_KEYS = ("norm_w", "A", "D", "dt_bias", "conv_w", "conv_b")


def upload_stack(cfg, layers, nseq, device):
    """Device copies of a stack given as numpy arrays (weights bf16, RMSNorm and Mamba
    parameters fp32) plus a zero decode state for nseq sequences: per Mamba layer h
    [nseq, d_inner, d_state] fp32 and conv_state [nseq, 3, d_inner] bf16, per SWA layer
    k_cache / v_cache [nseq, n_kv_heads, window + 1, head_dim] bf16."""
    out = []
    for ly in layers:
        d = {"kind": ly["kind"]}
        for k, a in ly.items():
            if k == "kind":
                continue
            t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
            d[k] = t if k in _F32_KEYS else t.to(torch.bfloat16)
        if ly["kind"] == "mamba":
            d["h"] = torch.zeros((nseq, cfg["d_inner"], cfg["d_state"]), dtype=torch.float32, device=device)
            d["conv_state"] = torch.zeros((nseq, 3, cfg["d_inner"]), dtype=torch.bfloat16, device=device)
        elif ly["kind"] == "swa":
            shape = (nseq, cfg["n_kv_heads"], cfg["window"] + 1, cfg["head_dim"])
            d["k_cache"] = torch.zeros(shape, dtype=torch.bfloat16, device=device)
            d["v_cache"] = torch.zeros(shape, dtype=torch.bfloat16, device=device)
        out.append(d)
    return out
