"""Host-side argument checks of every C ABI entry point (no GPU needed).

Each call below breaks one documented rule of include/samba_scan.h and must come back with
the documented status and a message naming the function, before anything is enqueued.  The
pointers are fake device addresses, so these calls only run where no GPU is visible: a check
that stopped refusing would otherwise launch a kernel on them.
"""
import ctypes

import pytest
import torch

import selective_state_space_samba_amd as ss

pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                reason="fake device pointers: host-only checks run where no GPU is visible")

INVALID, UNSUPPORTED, WORKSPACE = 1, 2, 3
F, G, H = 4096, 1 << 20, 2 << 20  # fake, 16-byte aligned device addresses far apart


def _params(conv=True):
    return ss.Params(F, None, None, F + 4096 if conv else None, None)


p, pu = _params(), _params(conv=False)
P = ctypes.byref
cfg = ss.ModelConfig(256, 512, 16, 16, 1024, 4, 2, 64, 16, 10000.0, 1e-5)
bad_layer = (ss.Layer * 1)()
bad_layer[0].kind = 9
CASES = [
    # scan entry points: dtype, pointers, sizes
    ("prefill_u io 7", INVALID, "unknown io dtype 7",
     lambda lib: lib.samba_scan_prefill_u(1, 4, 8, 16, 7, F, F, F, F, None, P(pu), None, G, None, None, 0, None)),
    ("prefill_u io -3", INVALID, "unknown io dtype -3",
     lambda lib: lib.samba_scan_prefill_u(1, 4, 8, 16, -3, F, F, F, F, None, P(pu), None, G, None, None, 0, None)),
    ("prefill_u u NULL", INVALID, "u is NULL",
     lambda lib: lib.samba_scan_prefill_u(1, 4, 8, 16, 1, None, F, F, F, None, P(pu), None, G, None, None, 0, None)),
    ("prefill_u A NULL", INVALID, "params->A is NULL",
     lambda lib: lib.samba_scan_prefill_u(1, 4, 8, 16, 1, F, F, F, F, None, P(ss.Params()), None, G, None, None, 0,
                                      None)),
    ("varlen_u cu NULL", INVALID, "cu_seqlens is NULL",
     lambda lib: lib.samba_scan_varlen_u(2, None, 10, 5, 8, 16, 1, F, F, F, F, None, P(pu), None, G, None, None, 0,
                                     None)),
    ("varlen_u max_seqlen", INVALID, "max_seqlen=11 exceeds total_tokens=10",
     lambda lib: lib.samba_scan_varlen_u(2, F, 10, 11, 8, 16, 1, F, F, F, F, None, P(pu), None, G, None, None, 0,
                                     None)),
    ("varlen total -1", INVALID, "must be >= 0",
     lambda lib: lib.samba_scan_varlen(2, F, -1, 5, 8, 16, 1, F, F, F, F, None, P(p), None, None, G, None, None,
                                   None, 0, None)),
    ("prefill d_state 17", UNSUPPORTED, "d_state=17",
     lambda lib: lib.samba_scan_prefill(1, 4, 8, 17, 1, F, F, F, F, None, P(p), None, None, G, None, None, None, 0,
                                    None)),
    ("decode io 9", INVALID, "unknown io dtype 9",
     lambda lib: lib.samba_scan_decode(4, 8, 16, 9, F, F, F, F, None, P(p), F, F, F + 8192, None, F, None)),
    # outputs overlapping inputs (4 tokens x 8 channels x 2 bytes = 64-byte token arrays)
    ("prefill out overlaps x", INVALID, "out overlaps x",
     lambda lib: lib.samba_scan_prefill(1, 4, 8, 16, 1, G, G + 4096, G + 8192, G + 12288, None, P(p), None, None,
                                    G + 32, None, None, None, 0, None)),
    ("prefill h_final overlaps h0", INVALID, "h_final overlaps h0",
     lambda lib: lib.samba_scan_prefill(1, 4, 8, 16, 1, G, G + 4096, G + 8192, G + 12288, None, P(p), H, None,
                                    G + 16384, H + 64, None, None, 0, None)),
    ("prefill conv_final overlaps out", INVALID, "overlaps",
     lambda lib: lib.samba_scan_prefill(1, 4, 8, 16, 1, G, G + 4096, G + 8192, G + 12288, None, P(p), None, None,
                                    G + 16384, None, G + 16384 + 16, None, 0, None)),
    ("prefill out overlaps params->A", INVALID, "out overlaps params->A",
     lambda lib: lib.samba_scan_prefill(1, 4, 8, 16, 1, G, G + 4096, G + 8192, G + 12288, None, P(p), None, None,
                                    F + 16, None, None, None, 0, None)),
    ("varlen_u out overlaps cu_seqlens", INVALID, "out overlaps cu_seqlens",
     lambda lib: lib.samba_scan_varlen_u(2, H, 4, 4, 8, 16, 1, G, G + 4096, G + 8192, G + 12288, None, P(pu), None,
                                     H, None, None, 0, None)),
    ("decode h overlaps conv_ring", INVALID, "h overlaps conv_ring",
     lambda lib: lib.samba_scan_decode(4, 8, 16, 1, G, G + 4096, G + 8192, G + 12288, None, P(p), H, H + 1024,
                                   H + 65536, None, G + 16384, None)),
    ("decode out overlaps x", INVALID, "out overlaps x",
     lambda lib: lib.samba_scan_decode(4, 8, 16, 1, G, G + 4096, G + 8192, G + 12288, None, P(p), H, H + 8192,
                                   H + 65536, None, G + 16, None)),
    # backward
    ("backward workspace", WORKSPACE, "workspace of",
     lambda lib: lib.samba_scan_backward(1, None, 64, 0, 64, 16, 1, *([F] * 4), None, P(p), None, None, F, None,
                                     None, *([G] * 5), *([G] * 5), None, None, H, 0, None)),
    ("backward dout NULL", INVALID, "dout is NULL",
     lambda lib: lib.samba_scan_backward(1, None, 64, 0, 64, 16, 1, *([F] * 4), None, P(p), None, None, None, None,
                                     None, *([G] * 5), *([G] * 5), None, None, H, 1 << 30, None)),
    ("backward dx overlaps dout", INVALID, "dx overlaps dout",
     lambda lib: lib.samba_scan_backward(1, None, 4, 0, 8, 16, 1, G, G + 4096, G + 8192, G + 12288, None, P(p),
                                     None, None, H, None, None, H + 32, H + 4096, H + 8192, H + 12288, None,
                                     H + 16384, H + 20480, H + 24576, H + 28672, H + 32768, None, None,
                                     1 << 24, 1 << 30, None)),
    # attention
    ("swa head_dim 96", UNSUPPORTED, "head_dim=96",
     lambda lib: lib.samba_swa_prefill(1, None, 64, 0, 4, 2, 96, 16, 10000.0, 1, F, F, F, G, H, 1 << 30, None)),
    ("swa heads", INVALID, "positive multiple",
     lambda lib: lib.samba_swa_prefill(1, None, 64, 0, 3, 2, 64, 16, 10000.0, 1, F, F, F, G, H, 1 << 30, None)),
    ("swa fp32", UNSUPPORTED, "bfloat16",
     lambda lib: lib.samba_swa_prefill(1, None, 64, 0, 4, 2, 64, 16, 10000.0, 0, F, F, F, G, H, 1 << 30, None)),
    ("swa window -1", INVALID, "window=-1",
     lambda lib: lib.samba_swa_prefill(1, None, 64, 0, 4, 2, 64, -1, 10000.0, 1, F, F, F, G, H, 1 << 30, None)),
    ("swa workspace", WORKSPACE, "workspace of",
     lambda lib: lib.samba_swa_prefill(1, None, 64, 0, 4, 2, 64, 16, 10000.0, 1, F, F, F, G, H, 0, None)),
    ("swa out overlaps q", INVALID, "out overlaps q",
     lambda lib: lib.samba_swa_prefill(1, None, 64, 0, 4, 2, 64, 16, 10000.0, 1, G, G + 65536, G + 98304, G + 64,
                                   H, 1 << 30, None)),
    ("swa_decode pos NULL", INVALID, "pos is NULL",
     lambda lib: lib.samba_swa_decode(2, 4, 2, 64, 16, 10000.0, 1, F, F, F, None, G, G + H, H + H, None, 0, None)),
    ("swa_decode workspace", WORKSPACE, "workspace of",
     lambda lib: lib.samba_swa_decode(2, 4, 2, 64, 16, 10000.0, 1, F, F, F, F, G, G + H, H + H, None, 0, None)),
    ("swa_decode v_cache overlaps k_cache", INVALID, "k_cache overlaps v_cache",
     lambda lib: lib.samba_swa_decode(2, 4, 2, 64, 16, 10000.0, 1, F, F + 1024, F + 2048, F + 3072, G, G + 64,
                                  H, H + 65536, 1 << 20, None)),
    ("swa_decode_noalloc io 5", UNSUPPORTED, "bfloat16",
     lambda lib: lib.samba_swa_decode_noalloc(2, 4, 2, 64, 16, 10000.0, 5, F, F, F, F, G, G + H, H + H, None)),
    ("swa_decode_noalloc beyond the scratch array", UNSUPPORTED, "scratch array",
     lambda lib: lib.samba_swa_decode_noalloc(60000, 64, 8, 128, 2048, 10000.0, 1, F, F, F, F, G, G + H, H + H,
                                          None)),
    ("swa_decode_noalloc out overlaps q", INVALID, "out overlaps q",
     lambda lib: lib.samba_swa_decode_noalloc(2, 4, 2, 64, 16, 10000.0, 1, G, G + 4096, G + 8192, G + 12288, H,
                                          H + 65536, G + 16, None)),
    ("kv_fill k NULL", INVALID, "k is NULL",
     lambda lib: lib.samba_swa_kv_fill(1, None, 64, 0, 2, 64, 16, 10000.0, 1, None, F, G, H, None)),
    ("kv_fill k_cache overlaps v", INVALID, "k_cache overlaps v",
     lambda lib: lib.samba_swa_kv_fill(1, None, 64, 0, 2, 64, 16, 10000.0, 1, F, G, G + 64, H, None)),
    # projections, norm, whole step
    ("gemm epilogue 7", INVALID, "unknown epilogue 7",
     lambda lib: lib.samba_gemm(64, 64, 64, 7, F, 64, G, H, 64, None, 0, None, 0, None)),
    ("gemm epilogue -1", INVALID, "unknown epilogue -1",
     lambda lib: lib.samba_gemm(64, 64, 64, -1, F, 64, G, H, 64, None, 0, None, 0, None)),
    ("gemm lda", INVALID, "lda=32",
     lambda lib: lib.samba_gemm(64, 64, 64, 0, F, 32, G, H, 64, None, 0, None, 0, None)),
    ("gemm residual NULL", INVALID, "residual is NULL",
     lambda lib: lib.samba_gemm(64, 64, 64, 1, F, 64, G, H, 64, None, 0, None, 0, None)),
    ("rmsnorm d -1", INVALID, "d=-1",
     lambda lib: lib.samba_rmsnorm(4, -1, F, G, 1e-5, H, None)),
    ("rmsnorm weight NULL", INVALID, "weight is NULL",
     lambda lib: lib.samba_rmsnorm(4, 64, F, None, 1e-5, H, None)),
    ("decode_step layer kind 9", INVALID, "unknown kind 9",
     lambda lib: lib.samba_decode_step(P(cfg), 1, bad_layer, F, 2, G, H, F + 64, F + 128, None, 0, None)),
    ("decode_step layers NULL", INVALID, "layers is NULL",
     lambda lib: lib.samba_decode_step(P(cfg), 1, None, F, 2, G, H, F + 64, F + 128, None, 0, None)),
    ("decode_step n_layers -1", INVALID, "n_layers=-1",
     lambda lib: lib.samba_decode_step(P(cfg), -1, bad_layer, F, 2, G, H, F + 64, F + 128, None, 0, None)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_refused_before_launch(case):
    name, status, text, call = case
    lib = ss.load()
    got = call(lib)
    msg = lib.samba_last_error().decode()
    assert got == status, (name, got, msg)
    assert text in msg, (name, msg)
    assert msg.startswith("samba_"), (name, msg)


def test_size_queries_refuse_bad_arguments_with_zero():
    lib = ss.load()
    assert lib.samba_scan_backward_workspace_bytes(-1, 64, 0, 64, 16) == 0
    assert lib.samba_gemm_workspace_bytes(64, 64, 64, 9) == 0
    assert lib.samba_swa_workspace_bytes(-5, 2, 64) == 0
    assert lib.samba_swa_decode_workspace_bytes(2, 0, 64) == 0
    assert lib.samba_decode_step_workspace_bytes(None, 2) == 0
    assert lib.samba_swa_decode_noalloc_max_bytes() > 0
