"""GPU parity of samba_rmsnorm (the RMSNorm before every layer of the decode step) against
the fp64 oracle, through the C ABI: the 16-byte path (d a multiple of 8, aligned rows, one to
four 2048-element chunks per thread) and the element path (any other d or alignment)."""
import numpy as np
import pytest
import torch

import selective_state_space_samba_amd as ss
from oracle import model
from tests.helpers import host, rel_err

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = 4e-3  # bf16 output: rounding alone is <= 2^-9 relative


@pytest.mark.parametrize("rows,d", [(1, 8), (3, 2048), (256, 2048), (5, 2056), (2, 8192), (7, 5), (4, 2047)])
def test_rmsnorm(rows, d):
    print("case: rmsnorm", rows, d, flush=True)
    rng = np.random.default_rng(rows * 10007 + d)
    x = torch.from_numpy((rng.standard_normal((rows, d)) * 3).astype(np.float32)).to(DEV)
    w = torch.from_numpy(rng.uniform(0.5, 1.5, d).astype(np.float32)).to(DEV)
    out = ss.rmsnorm(x, w, eps=1e-5)
    torch.cuda.synchronize()
    e = rel_err(host(out), model.rmsnorm(host(x), host(w), 1e-5))
    print("  err %.3e" % e, flush=True)
    assert e <= TOL


def test_rmsnorm_unaligned_output_takes_the_element_path():
    print("case: rmsnorm unaligned out", flush=True)
    rows, d = 3, 2048
    rng = np.random.default_rng(11)
    x = torch.from_numpy(rng.standard_normal((rows, d)).astype(np.float32)).to(DEV)
    w = torch.from_numpy(rng.uniform(0.5, 1.5, d).astype(np.float32)).to(DEV)
    buf = torch.zeros(rows * d + 1, dtype=torch.bfloat16, device=DEV)
    out = buf[1:].view(rows, d)  # 2-byte aligned only
    ss.rmsnorm(x, w, eps=1e-5, out=out)
    torch.cuda.synchronize()
    assert float(host(buf[:1])[0]) == 0.0
    assert rel_err(host(out), model.rmsnorm(host(x), host(w), 1e-5)) <= TOL
