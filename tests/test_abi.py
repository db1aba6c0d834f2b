"""Host-side checks of the C ABI library (no GPU needed): it loads, exports every function
declared in include/*.h, and rejects bad arguments before touching the GPU."""
import ctypes
import glob
import os
import re

import pytest

import selective_state_space_samba_amd as ss

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b(samba_\w+)\s*\(", text):
            names.add(m.group(1))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("samba_scan_prefill", "samba_scan_varlen", "samba_scan_decode", "samba_conv_silu", "samba_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(ss.lib_path())
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_version_string():
    assert "gfx950" in ss.version()


def _call_prefill(lib, b=1, L=4, D=8, N=16, io=1, params=True, ptrs=True):
    p = ss.Params(16, None, None, 32 if params else None, None) if params else None
    fake = 4096 if ptrs else None
    return lib.samba_scan_prefill(b, L, D, N, io, fake, fake, fake, fake, None,
                                  ctypes.byref(p) if p is not None else None,
                                  None, None, fake, None, None, None, 0, None)


def test_argument_errors_are_reported_without_launching():
    lib = ss.load()
    assert _call_prefill(lib, params=False) == 1
    assert b"params is NULL" in lib.samba_last_error()
    assert _call_prefill(lib, N=17) == 2
    assert b"d_state=17" in lib.samba_last_error()
    assert _call_prefill(lib, N=0) == 1
    assert _call_prefill(lib, D=0) == 1
    assert _call_prefill(lib, b=-1) == 1
    assert _call_prefill(lib, io=7) == 1
    assert _call_prefill(lib, ptrs=False) == 1
    assert b"x is NULL" in lib.samba_last_error()
    # misaligned pointer
    p = ss.Params(16, None, None, 32, None)
    st = lib.samba_scan_prefill(1, 4, 8, 16, 1, 4098, 4096, 4096, 4096, None, ctypes.byref(p), None, None, 4096,
                                None, None, None, 0, None)
    assert st == 1 and b"aligned" in lib.samba_last_error()
    # batch == 0 is a no-op that succeeds without touching any pointer
    assert _call_prefill(lib, b=0, ptrs=False) == 0


def test_varlen_and_decode_argument_errors():
    lib = ss.load()
    p = ss.Params(16, None, None, 32, None)
    st = lib.samba_scan_varlen(2, None, 10, 5, 8, 16, 1, 4096, 4096, 4096, 4096, None, ctypes.byref(p), None, None,
                               4096, None, None, None, 0, None)
    assert st == 1 and b"cu_seqlens is NULL" in lib.samba_last_error()
    st = lib.samba_scan_varlen(2, 4096, 10, 11, 8, 16, 1, 4096, 4096, 4096, 4096, None, ctypes.byref(p), None,
                               None, 4096, None, None, None, 0, None)
    assert st == 1 and b"max_seqlen" in lib.samba_last_error()
    # decode: (nseq, D, N, io, x, dt, B, C, z, params, h, conv_ring, ring_head_in, ring_head_out, out, stream)
    st = lib.samba_scan_decode(4, 8, 16, 1, 4096, 4096, 4096, 4096, None, ctypes.byref(p), None, 4096, 8192, None,
                               4096, None)
    assert st == 1 and b"h is NULL" in lib.samba_last_error()
    st = lib.samba_scan_decode(4, 8, 16, 1, 4096, 4096, 4096, 4096, None, ctypes.byref(p), 4096, 4096, None, None,
                               4096, None)
    assert st == 1 and b"ring_head_in is NULL" in lib.samba_last_error()
    # the heads are double-buffered: head_out may not overlap head_in
    st = lib.samba_scan_decode(4, 8, 16, 1, 4096, 4096, 4096, 4096, None, ctypes.byref(p), 4096, 4096, 8192, 8200,
                               4096, None)
    assert st == 1 and b"overlaps ring_head_in" in lib.samba_last_error()
    st = lib.samba_scan_decode(4, 8, 16, 1, 4096, 4096, 4096, 4096, None, ctypes.byref(p), 4096, 4096, 8194, None,
                               4096, None)
    assert st == 1 and b"4-byte aligned" in lib.samba_last_error()
    # one grid row per sequence: more than 65535 sequences is refused before any launch
    st = lib.samba_scan_decode(65536, 8, 16, 1, 4096, 4096, 4096, 4096, None, ctypes.byref(p), 4096, 4096, 8192,
                               None, 4096, None)
    assert st == 2 and b"65535" in lib.samba_last_error()
    assert lib.samba_scan_decode(0, 8, 16, 1, None, None, None, None, None, ctypes.byref(p), None, None, None,
                                 None, None, None) == 0


def test_binding_refuses_cpu_tensors_before_calling():
    import torch
    x = torch.zeros((1, 4, 8), dtype=torch.bfloat16)
    Bm = torch.zeros((1, 4, 16), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="on a GPU"):
        ss.prefill(x, x, Bm, Bm, x, torch.zeros((8, 16)), None, None, torch.zeros((8, 4)), None)
    with pytest.raises(ValueError, match="on a GPU"):
        ss.decode(x[0], x[0], Bm[0], Bm[0], x[0], torch.zeros((8, 16)), None, None, torch.zeros((8, 4)), None,
                  torch.zeros((4, 8, 16)), torch.zeros((4, 3, 8), dtype=torch.bfloat16), torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError, match="on a GPU"):
        ss.varlen(torch.zeros(2, dtype=torch.int32), x[0], x[0], Bm[0], Bm[0], x[0], torch.zeros((8, 16)), None,
                  None, torch.zeros((8, 4)), None, max_seqlen=4)


def test_conv_silu_argument_errors():
    lib = ss.load()
    # nseq, cu, seqlen, total, D, io, x, conv_w, conv_b, conv0, u, conv_final, stream
    assert lib.samba_conv_silu(1, None, 4, 0, 8, 1, 4096, None, None, None, 8192, None, None) == 1
    assert b"conv_w is NULL" in lib.samba_last_error()
    assert lib.samba_conv_silu(1, None, 4, 0, 8, 1, None, 4096, None, None, 8192, None, None) == 1
    assert b"x is NULL" in lib.samba_last_error()
    # u overlapping x (4 tokens x 8 channels x 2 bytes = 64 bytes)
    assert lib.samba_conv_silu(1, None, 4, 0, 8, 1, 4096, 4096, None, None, 4096 + 48, None, None) == 1
    assert b"overlaps x" in lib.samba_last_error()
    # conv_final overlapping conv0 (3 x 8 x 2 = 48 bytes)
    assert lib.samba_conv_silu(1, None, 4, 0, 8, 1, 4096, 4096, None, 1 << 20, 8192, (1 << 20) + 32, None) == 1
    assert b"conv_final overlaps conv0" in lib.samba_last_error()
    assert lib.samba_conv_silu(2, 4096, 11, 10, 8, 1, 4096, 4096, None, None, 8192, None, None) == 1
    assert b"max_seqlen" in lib.samba_last_error()
    assert lib.samba_conv_silu(-1, None, 4, 0, 8, 1, None, None, None, None, None, None, None) == 1
    assert lib.samba_conv_silu(0, None, 4, 0, 8, 1, None, None, None, None, None, None, None) == 0
    with pytest.raises(ValueError, match="on a GPU"):
        import torch
        ss.conv_silu(torch.zeros((1, 4, 8)), torch.zeros((8, 4)))


def test_struct_layouts_match_the_binding(tmp_path):
    """samba_params, samba_model_config and samba_layer as the C compiler lays them out (gcc
    on the header) equal the ctypes structures the binding passes: size and every offset."""
    import ctypes
    import subprocess
    import selective_state_space_samba_amd as ss
    structs = {"samba_params": ss.Params, "samba_model_config": ss.ModelConfig, "samba_layer": ss.Layer}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "samba_scan.h"', 'int main(void) {']
    for cname, py in structs.items():
        lines.append('printf("%s size %%zu\\n", sizeof(%s));' % (cname, cname))
        for f, _ in py._fields_:
            lines.append('printf("%s %s %%zu\\n", offsetof(%s, %s));' % (cname, f, cname, f))
    lines += ['return 0;', '}']
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(l.rsplit(" ", 1) for l in subprocess.run([str(exe)], check=True, capture_output=True,
                                                         text=True).stdout.splitlines())
    for cname, py in structs.items():
        assert int(got["%s size" % cname]) == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert int(got["%s %s" % (cname, f)]) == getattr(py, f).offset, (cname, f)
