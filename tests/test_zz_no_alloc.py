"""The allocation-free entry point samba_swa_decode_noalloc (GPU): the same outputs as
samba_swa_decode with a caller workspace, bit for bit, on two calls in a row, the second
with fewer sequences (the library's device array keeps the first call's partials; every
partial the second call reads must be its own)."""
import numpy as np
import pytest
import torch

import selective_state_space_samba_amd as ss

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _case(g, S, Hq, Hkv, dh, w):
    mk = lambda *shape: torch.randn(shape, generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    q, k, v = mk(S, Hq, dh), mk(S, Hkv, dh), mk(S, Hkv, dh)
    kc, vc = mk(S, Hkv, w + 1, dh), mk(S, Hkv, w + 1, dh)
    # positions: inside the first window, past it (full ring wrapping), one inactive sequence
    pos = torch.tensor([(i * 97) % (3 * w) for i in range(S)], dtype=torch.int32, device=DEV)
    pos[S // 2] = -1
    return q, k, v, kc, vc, pos


@pytest.mark.parametrize("Hq,Hkv,dh", [(32, 4, 64), (8, 1, 128)])
def test_noalloc_equals_workspace_entry_point_on_two_calls(Hq, Hkv, dh):
    print("case: swa_decode_noalloc Hq %d Hkv %d dh %d" % (Hq, Hkv, dh), flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(77 + dh)
    w = 300
    for S in (40, 9):  # the second call is smaller than the first
        q, k, v, kc, vc, pos = _case(g, S, Hq, Hkv, dh, w)
        kc2, vc2 = kc.clone(), vc.clone()
        ref = ss.swa_decode(q, k, v, pos, kc, vc, window=w)
        got = ss.swa_decode_noalloc(q, k, v, pos, kc2, vc2, window=w)
        torch.cuda.synchronize()
        assert torch.equal(ref, got), "outputs differ at S=%d" % S
        assert torch.equal(kc, kc2) and torch.equal(vc, vc2)
        assert torch.isfinite(got.float()).all()
        assert (got[S // 2] == 0).all()  # the inactive sequence gets no attention output


def test_noalloc_rejects_problems_beyond_its_array():
    lib = ss.load()
    cap = int(lib.samba_swa_decode_noalloc_max_bytes())
    need = int(lib.samba_swa_decode_workspace_bytes(4096, 32, 128))
    assert need > cap
    q = torch.zeros((4096, 32, 128), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((4096, 4, 128), dtype=torch.bfloat16, device=DEV)
    cache = torch.zeros((4096, 4, 2, 128), dtype=torch.bfloat16, device=DEV)
    pos = torch.zeros(4096, dtype=torch.int32, device=DEV)
    with pytest.raises(ss.SambaError) as ei:
        ss.swa_decode_noalloc(q, kv, kv, pos, cache, cache.clone(), window=1)
    assert ei.value.status == 2 and "scratch array" in str(ei.value)
