"""GPU parity of the bf16 matrix-core GEMM (samba_gemm) against the fp64 oracle's
projections, through the C ABI: plain store, the fp32 residual add (in place) and the
fused SwiGLU, on single tiles, ragged tiles, split K ranges and the 1.7B projection
shapes."""
import numpy as np
import pytest
import torch

import selective_state_space_samba_amd as ss
from oracle import model
from tests.helpers import host, rel_err

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
# bf16 output: rounding alone is <= 2^-9 relative; fp32 accumulation adds ~K * 2^-24.
TOL_BF16_OUT = 4e-3
TOL_F32_OUT = 1e-5


def bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(torch.bfloat16)


def operands(seed, M, N, K, wrows=None):
    rng = np.random.default_rng(seed)
    a = bf16(rng.standard_normal((M, K)))
    w = bf16(rng.standard_normal((wrows or N, K)) / np.sqrt(max(K, 1)))
    return a, w


def check(got, ref, tol):
    e = rel_err(host(got), ref)
    print("  err %.3e (tol %.0e)" % (e, tol), flush=True)
    assert e <= tol


SHAPES = [(1, 1, 8), (5, 3, 16), (37, 50, 72), (128, 128, 64), (300, 260, 200), (256, 160, 4096),
          (256, 16, 4096), (256, 4096, 128), (256, 2048, 8200), (700, 900, 1000), (1100, 2304, 512),
          (2048, 2048, 256),
          # 512 tiles of 128 x 128: no split, two workgroups per CU
          (4096, 2048, 200)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_store(M, N, K):
    print("case: gemm store", M, N, K, "workspace", ss.load().samba_gemm_workspace_bytes(M, N, K, 0), flush=True)
    a, w = operands(100 + M + N + K, M, N, K)
    out = ss.gemm(a, w)
    torch.cuda.synchronize()
    check(out, model.linear(host(a), host(w)), TOL_BF16_OUT)


@pytest.mark.parametrize("M,N,K", [(3, 40, 24), (256, 2048, 8200), (300, 260, 200), (1024, 1024, 1024)])
def test_gemm_residual_add_in_place(M, N, K):
    print("case: gemm add", M, N, K, flush=True)
    a, w = operands(200 + M + N + K, M, N, K)
    r = torch.from_numpy(np.random.default_rng(7).standard_normal((M, N)).astype(np.float32)).to(DEV)
    r0 = host(r)
    out = ss.gemm(a, w, epilogue="add", residual=r, out=r)
    torch.cuda.synchronize()
    assert out.data_ptr() == r.data_ptr()
    check(out, r0 + model.linear(host(a), host(w)), TOL_F32_OUT)


@pytest.mark.parametrize("M,N,K", [(5, 24, 40), (256, 8196, 2048), (300, 100, 72), (1100, 700, 256)])
def test_gemm_swiglu(M, N, K):
    print("case: gemm swiglu", M, N, K, "workspace", ss.load().samba_gemm_workspace_bytes(M, N, K, 2), flush=True)
    a, w = operands(300 + M + N + K, M, N, K, wrows=2 * N)
    out = ss.gemm(a, w, epilogue="swiglu")
    torch.cuda.synchronize()
    wh = host(w)
    check(out, model.swiglu(host(a), wh[:N], wh[N:]), TOL_BF16_OUT)


# Problems with at least 256 tiles of 256 x 256 take the 8-wave tiles with loads straight into
# LDS; ragged in M, N and K.
@pytest.mark.parametrize("M,N,K,epi", [(4100, 4110, 72, "store"), (4097, 4100, 200, "add"),
                                       (4100, 8196, 40, "swiglu")])
def test_gemm_large_tiles(M, N, K, epi):
    print("case: gemm large tiles", epi, M, N, K, flush=True)
    a, w = operands(400 + M + N + K, M, N, K, wrows=2 * N if epi == "swiglu" else None)
    ah, wh = host(a), host(w)
    if epi == "swiglu":
        out = ss.gemm(a, w, epilogue="swiglu")
        ref = model.swiglu(ah, wh[:N], wh[N:])
        tol = TOL_BF16_OUT
    elif epi == "add":
        r = torch.from_numpy(np.random.default_rng(8).standard_normal((M, N)).astype(np.float32)).to(DEV)
        ref = host(r) + model.linear(ah, wh)
        out = ss.gemm(a, w, epilogue="add", residual=r, out=r)
        tol = TOL_F32_OUT
    else:
        out = ss.gemm(a, w)
        ref = model.linear(ah, wh)
        tol = TOL_BF16_OUT
    torch.cuda.synchronize()
    check(out, ref, tol)


# The same tiles forced onto small ragged problems (single partial tiles, K tails).
@pytest.mark.parametrize("M,N,K", [(1, 1, 8), (37, 50, 72), (300, 260, 200), (257, 129, 1000)])
def test_gemm_large_tiles_on_ragged_shapes(M, N, K, monkeypatch):
    monkeypatch.setenv("SAMBA_GEMM_TILE", "256")
    print("case: gemm 256 tiles forced", M, N, K, flush=True)
    a, w = operands(500 + M + N + K, M, N, K)
    out = ss.gemm(a, w)
    torch.cuda.synchronize()
    check(out, model.linear(host(a), host(w)), TOL_BF16_OUT)
    a, w = operands(600 + M + N + K, M, N, K, wrows=2 * N)
    out = ss.gemm(a, w, epilogue="swiglu")
    torch.cuda.synchronize()
    wh = host(w)
    check(out, model.swiglu(host(a), wh[:N], wh[N:]), TOL_BF16_OUT)


def test_gemm_strided_rows_and_output_pitch():
    """A as a column slice of a wider matrix (lda > K), output into a column slice."""
    print("case: gemm strided", flush=True)
    a_full, w = operands(400, 70, 48, 200)
    a = a_full[:, 64:176]  # K = 112, lda = 200
    w = w[:, :112].contiguous()
    big = torch.zeros((70, 100), dtype=torch.bfloat16, device=DEV)
    ss.gemm(a, w, out=big[:, 30:78])
    torch.cuda.synchronize()
    hb = host(big)
    check(big[:, 30:78], model.linear(host(a), host(w)), TOL_BF16_OUT)
    assert np.all(hb[:, :30] == 0) and np.all(hb[:, 78:] == 0)


# Every kernel a skinny product can take (the plan picks one by an estimate; SAMBA_GEMM_STREAM
# forces the stream kernel's tile shape and split count, "r2" the 128 x 128 ring kernel, "0"
# the register-staged kernel), on ragged shapes and every epilogue.
@pytest.mark.parametrize("force", ["4x4", "4x2", "2x4", "2x2", "4x4s2", "2x2s3", "4x2s8", "r2", "r3s2", "0"])
@pytest.mark.parametrize("M,N,K,epi", [(37, 50, 72, "store"), (256, 300, 1000, "add"), (200, 100, 520, "swiglu"),
                                       (256, 160, 4096, "store"), (3, 16, 8, "add")])
def test_gemm_skinny_kernels(force, M, N, K, epi, monkeypatch):
    monkeypatch.setenv("SAMBA_GEMM_STREAM", force)
    print("case: gemm skinny", force, epi, M, N, K, flush=True)
    Nw = 2 * N if epi == "swiglu" else N
    a, w = operands(700 + M + N + K, M, N, K, wrows=Nw)
    if epi == "add":
        r = torch.from_numpy(np.random.default_rng(9).standard_normal((M, N)).astype(np.float32)).to(DEV)
        r0 = host(r)
        out = ss.gemm(a, w, epilogue="add", residual=r)
        torch.cuda.synchronize()
        check(out, r0 + model.linear(host(a), host(w)), TOL_F32_OUT)
    elif epi == "swiglu":
        out = ss.gemm(a, w, epilogue="swiglu")
        torch.cuda.synchronize()
        wh = host(w)
        check(out, model.swiglu(host(a), wh[:N], wh[N:]), TOL_BF16_OUT)
    else:
        out = ss.gemm(a, w)
        torch.cuda.synchronize()
        check(out, model.linear(host(a), host(w)), TOL_BF16_OUT)


def test_gemm_is_deterministic():
    a, w = operands(500, 256, 2048, 8200)
    o1 = host(ss.gemm(a, w))
    o2 = host(ss.gemm(a, w))
    np.testing.assert_array_equal(o1, o2)


def test_gemm_argument_errors():
    a, w = operands(600, 8, 8, 16)
    with pytest.raises(ss.SambaError, match="UNSUPPORTED"):
        ss.gemm(a[:, :12].contiguous(), w[:, :12].contiguous())
    buf = torch.zeros(80, device=DEV)
    with pytest.raises(ss.SambaError, match="INVALID_ARG"):  # residual partially overlaps out
        ss.gemm(a, w, epilogue="add", residual=buf[:64].view(8, 8), out=buf[4:68].view(8, 8))
    # a few rows and columns over a long K range: the K range is split across workgroups
    a2, w2 = operands(601, 16, 64, 8192)
    assert ss.load().samba_gemm_workspace_bytes(16, 64, 8192, 0) > 0
    with pytest.raises(ss.SambaError, match="WORKSPACE"):
        ss.gemm(a2, w2, workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
