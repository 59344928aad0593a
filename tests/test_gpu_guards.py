"""Write-bounds and read-before-write checks of ssd_fwd / ssd_bwd on the GPU.

* Guard bands: every output (y, final states, every gradient) is a view into a
  larger buffer whose bands before and after it hold a sentinel; after the call
  the bands must be unchanged (no write outside an output) and the outputs equal
  to a call on plain tensors.
* Poisoned workspace: the workspace is filled with NaN bytes (0xFF) before the
  call; the outputs must equal, bit for bit, those of a call on a zeroed
  workspace (no value is read from the workspace before the call wrote it).
Covered: bf16 and fp32 io, batched ragged and packed (with empty and 1-token
sequences), the training pair (save / from saved) and the chained forward."""
import ctypes

import pytest
import torch

from helpers import has_gpu, to_dev
from mamba_ssd_chunked_03_amd import inputs

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]

ssd = pytest.importorskip("mamba_ssd_chunked_03_amd.ssd")

PAD = 64  # elements of guard band on each side (a multiple of 16 bytes for both dtypes)


def guarded(shape, dtype, sentinel):
    n = 1
    for s in shape:
        n *= s
    buf = torch.full((n + 2 * PAD,), sentinel, dtype=dtype, device="cuda")
    return buf, buf[PAD:PAD + n].view(*shape)


def bands_intact(buf, sentinel):
    return bool((buf[:PAD] == sentinel).all()) and bool((buf[-PAD:] == sentinel).all())


def problem_inputs(kind):
    if kind == "bf16":
        return inputs.make_inputs(2, 700, 16, 64, 128, 2, io="bf16", init="randn", bwd=True, d_final=True,
                                  seed=111), 256
    if kind == "f32":
        return inputs.make_inputs(2, 150, 2, 16, 32, 1, io="f32", init="randn", bwd=True, d_final=True,
                                  seed=112), 64
    lengths = [1, 0, 300, 513, 77]
    return inputs.make_inputs(1, sum(lengths), 4, 64, 128, 2, io="bf16", init="randn", bwd=True,
                              d_final=True, lengths=lengths, seed=113), 128


def ws_bytes(d, Q, save):
    prob = ssd.problem(d["x"], d["B"], d["cu_seqlens"])
    packed = int(d["cu_seqlens"] is not None)
    L = ssd.lib()
    return (L.ssd_bwd_workspace_bytes if save else L.ssd_fwd_workspace_bytes)(ctypes.byref(prob), Q, packed)


def fwd_args(d, inp, Q):
    return (d["x"], d["dt"], d["A"], d["B"], d["C"]), dict(D=d["D"], dt_bias=d["dt_bias"], init=d["init"],
                                                            cu_seqlens=d["cu_seqlens"], chunk_size=Q,
                                                            dt_softplus=inp["dt_softplus"])


@pytest.mark.parametrize("kind", ["bf16", "f32", "packed"])
def test_output_guard_bands(kind):
    inp, Q = problem_inputs(kind)
    d = to_dev(inp)
    args, kw = fwd_args(d, inp, Q)
    y0, f0 = ssd.fwd(*args, **kw)
    g0 = ssd.bwd(*args, d["dout"], d_final=d["d_final"], **kw)
    torch.cuda.synchronize()
    S = {torch.bfloat16: -7.0, torch.float32: -7.0}
    ybuf, y = guarded(y0.shape, y0.dtype, S[y0.dtype])
    fbuf, fin = guarded(f0.shape, torch.float32, -7.0)
    ssd.fwd(*args, out=y, final=fin, **kw)
    torch.cuda.synchronize()
    assert bands_intact(ybuf, -7.0) and bands_intact(fbuf, -7.0)
    assert torch.equal(y, y0) and torch.equal(fin, f0)
    bufs, grads = {}, {}
    for k, v in g0.items():
        if v is None:
            grads[k] = None
            continue
        bufs[k], grads[k] = guarded(v.shape, v.dtype, -7.0)
    ssd.bwd(*args, d["dout"], d_final=d["d_final"], grads=grads, **kw)
    torch.cuda.synchronize()
    for k, b in bufs.items():
        assert bands_intact(b, -7.0), k
        assert torch.equal(grads[k], g0[k]), k


@pytest.mark.parametrize("kind", ["bf16", "f32", "packed"])
def test_poisoned_workspace(kind):
    inp, Q = problem_inputs(kind)
    d = to_dev(inp)
    args, kw = fwd_args(d, inp, Q)
    results = []
    for fill in (0x00, 0xFF):
        out = {}
        ws = torch.full((max(1, ws_bytes(d, Q, False)),), fill, dtype=torch.uint8, device="cuda")
        out["y"], out["final"] = ssd.fwd(*args, workspace=ws, **kw)
        wsb = torch.full((max(1, ws_bytes(d, Q, True)),), fill, dtype=torch.uint8, device="cuda")
        out["ys"], out["fs"] = ssd.fwd(*args, workspace=wsb, save_for_backward=True, **kw)
        g = ssd.bwd(*args, d["dout"], d_final=d["d_final"], workspace=wsb, from_saved=True, **kw)
        wsr = torch.full((max(1, ws_bytes(d, Q, True)),), fill, dtype=torch.uint8, device="cuda")
        g2 = ssd.bwd(*args, d["dout"], d_final=d["d_final"], workspace=wsr, **kw)
        if kind != "f32":
            wsc = torch.full((max(1, ws_bytes(d, Q, False)),), fill, dtype=torch.uint8, device="cuda")
            out["yc"], out["fc"] = ssd.fwd(*args, workspace=wsc, chained=True, **kw)
        torch.cuda.synchronize()
        out.update({"saved_" + k: v for k, v in g.items() if v is not None})
        out.update({"recomputed_" + k: v for k, v in g2.items() if v is not None})
        results.append(out)
    for k in results[0]:
        assert torch.equal(results[0][k], results[1][k]), k
        assert bool(torch.isfinite(results[1][k].float()).all()), k
