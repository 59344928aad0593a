"""GPU parity of the gated RMSNorm (through the C ABI) against the fp64 oracle.

Inputs are seeded: y, z, dout ~ N(0, 1) rounded to bf16, weight ~ U(0.5, 1.5)
fp32; the oracle runs on the same bf16 values in float64.  Tolerances
(normwise, max |gpu - ref| / max |ref| per tensor): out, dy, dz are stored in
bf16, whose rounding alone is up to 2^-9 of a value: out <= 4e-3, dy and dz
<= 1e-2 (dv is a difference of two terms); rstd and dweight are fp32:
<= 1e-5 and <= 1e-4."""
import numpy as np
import pytest
import torch

from helpers import has_gpu, normwise
from oracle import norm

ssd = pytest.importorskip("mamba_ssd_chunked_03_amd.ssd")
pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def make(rows, dim, seed, gate=True):
    g = torch.Generator().manual_seed(seed)
    y = torch.randn(rows, dim, generator=g).to(torch.bfloat16)
    z = torch.randn(rows, dim, generator=g).to(torch.bfloat16) if gate else None
    w = torch.rand(dim, generator=g) + 0.5
    dout = torch.randn(rows, dim, generator=g).to(torch.bfloat16)
    return y, z, w, dout


def f64(t):
    return None if t is None else t.double().numpy()


def run(y, z, w, dout, group, eps):
    c = lambda t: None if t is None else t.cuda()
    rows, dim = y.shape
    rstd = torch.empty(rows, dim // group, device="cuda")
    out = ssd.gated_rmsnorm_fwd(c(y), c(z), c(w), group, eps, rstd=rstd)
    dy, dz, dw = ssd.gated_rmsnorm_bwd(c(dout), c(y), c(z), c(w), group, eps)
    torch.cuda.synchronize()
    return out.cpu(), rstd.cpu(), dy.cpu(), None if dz is None else dz.cpu(), dw.cpu()


CASES = [  # rows, dim, group, gate
    (37, 4096, 512, True), (5, 512, 256, True), (100, 2048, 2048, False), (64, 8192, 8192, True),
    (1100, 1024, 1024, True), (3, 4096, 4096, True), (1, 8192, 2048, False), (300, 1536, 512, True),
]


@pytest.mark.parametrize("rows,dim,group,gate", CASES)
def test_norm_matches_oracle(rows, dim, group, gate):
    eps = 1e-5
    y, z, w, dout = make(rows, dim, 11 + rows, gate)
    out, rstd, dy, dz, dw = run(y, z, w, dout, group, eps)
    o_out, o_r = norm.fwd(f64(y), f64(z), f64(w), group, eps)
    o_dy, o_dz, o_dw = norm.bwd(f64(dout), f64(y), f64(z), f64(w), group, eps)
    assert normwise(f64(out), o_out) <= 4e-3
    assert normwise(f64(rstd), o_r) <= 1e-5
    assert normwise(f64(dy), o_dy) <= 1e-2
    if gate:
        assert normwise(f64(dz), o_dz) <= 1e-2
    else:
        assert dz is None
    assert normwise(f64(dw), o_dw) <= 1e-4


def test_norm_deterministic():
    y, z, w, dout = make(1500, 4096, 5)
    a = run(y, z, w, dout, 512, 1e-5)
    b = run(y, z, w, dout, 512, 1e-5)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_norm_full_size_sampled():
    """The layer workload (rows = batch 2 x seqlen 8192, dim = 64 heads x
    headdim 64, group = dim / 8 groups): sampled rows of out, dy, dz, and the
    whole dweight (the oracle summed over every row in blocks)."""
    rows, dim, group, eps = 16384, 4096, 512, 1e-5
    y, z, w, dout = make(rows, dim, 2)
    out, rstd, dy, dz, dw = run(y, z, w, dout, group, eps)
    idx = np.random.default_rng(0).choice(rows, 48, replace=False)
    o_out, o_r = norm.fwd(f64(y[idx]), f64(z[idx]), f64(w), group, eps)
    o_dy, o_dz, _ = norm.bwd(f64(dout[idx]), f64(y[idx]), f64(z[idx]), f64(w), group, eps)
    assert normwise(f64(out[idx]), o_out) <= 4e-3
    assert normwise(f64(rstd[idx]), o_r) <= 1e-5
    assert normwise(f64(dy[idx]), o_dy) <= 1e-2
    assert normwise(f64(dz[idx]), o_dz) <= 1e-2
    o_dw = np.zeros(dim)
    for r0 in range(0, rows, 2048):
        o_dw += norm.bwd(f64(dout[r0:r0 + 2048]), f64(y[r0:r0 + 2048]), f64(z[r0:r0 + 2048]), f64(w),
                         group, eps)[2]
    assert normwise(f64(dw), o_dw) <= 1e-4


def test_norm_no_rows():
    """No rows: the forward queues nothing; the backward still writes dweight = 0."""
    y = torch.empty(0, 1024, dtype=torch.bfloat16, device="cuda")
    w = torch.rand(1024, device="cuda") + 0.5
    out = ssd.gated_rmsnorm_fwd(y, y, w, 512)
    dw = torch.full((1024,), 7.0, device="cuda")
    dy, dz, dw = ssd.gated_rmsnorm_bwd(y, y, y, w, 512, grads=(torch.empty_like(y), torch.empty_like(y), dw))
    torch.cuda.synchronize()
    assert out.shape == (0, 1024) and torch.count_nonzero(dw).item() == 0


@pytest.mark.parametrize("pieces", [1, 255, 256, 1000003])
def test_util_copy(pieces):
    """The plain copy kernel (counter calibration): every byte copied, nothing past the end."""
    src = torch.randint(-2**31, 2**31 - 1, (pieces * 4 + 4,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    ssd.util_copy(dst[:pieces * 4], src[:pieces * 4])
    torch.cuda.synchronize()
    assert torch.equal(dst[:pieces * 4], src[:pieces * 4])
    assert torch.equal(dst[pieces * 4:], torch.zeros(4, dtype=torch.int32, device="cuda"))
