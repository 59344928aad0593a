"""GPU parity of the fused chained forward (SSD_FLAG_CHAINED_FWD): one kernel forms
each chunk's state, takes the carry from the previous chunk's workgroup and writes
the output.  Against the token-by-token oracle, with the forward gates (bf16 y
ulp-aware <= 2e-2, final states normwise <= 1e-3, scan-only y normwise <= 1e-2),
on ragged, packed and 512-chunk inputs; after every call the workspace's wait-error
word must be zero (no wait for a carry ran out)."""
import ctypes

import numpy as np
import pytest
import torch

from helpers import bf16_excess, has_gpu, normwise, np64, oracle_args, to_dev
from mamba_ssd_chunked_03_amd import inputs
from oracle import recurrence

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]

ssd = pytest.importorskip("mamba_ssd_chunked_03_amd.ssd")


def chained(inp, Q, save=False):
    d = to_dev(inp)
    prob = ssd.problem(d["x"], d["B"], d["cu_seqlens"])
    packed = int(d["cu_seqlens"] is not None)
    L = ssd.lib()
    nbytes = (L.ssd_bwd_workspace_bytes if save else L.ssd_fwd_workspace_bytes)(ctypes.byref(prob), Q, packed)
    ws = torch.full((max(1, nbytes),), 0x7F, dtype=torch.uint8, device="cuda")  # garbage flags/counters
    y, final = ssd.fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], dt_bias=d["dt_bias"],
                       init=d["init"], cu_seqlens=d["cu_seqlens"], chunk_size=Q,
                       dt_softplus=inp["dt_softplus"], workspace=ws, save_for_backward=save, chained=True)
    torch.cuda.synchronize()
    off = L.ssd_fwd_chained_error_offset(ctypes.byref(prob), Q, packed)
    if nbytes:
        assert int(ws[off:off + 4].view(torch.int32).item()) == 0, "a wait for a carry ran out"
    return y, final, ws


def check(inp, y, final, heads=None, scan_only=False):
    y_ref, f_ref = recurrence.fwd(**oracle_args(inp), heads=heads)
    if heads is not None:
        y, final = y[:, :, heads], final[:, heads]
    if scan_only:
        assert normwise(np64(y), y_ref) <= 1e-2
    else:
        assert bf16_excess(np64(y), y_ref) <= 2e-2
    assert normwise(np64(final), f_ref) <= 1e-3


CASES = [
    ("ragged_fused_cb", dict(batch=2, seqlen=700, nheads=16, headdim=64, dstate=128, ngroups=2,
                             init="randn", seed=91), (128, 256)),
    ("odd_heads", dict(batch=1, seqlen=420, nheads=3, headdim=64, dstate=128, ngroups=1,
                       init="randn", seed=92), (256,)),
    ("p32n64", dict(batch=1, seqlen=333, nheads=4, headdim=32, dstate=64, ngroups=2,
                    init="zeros", seed=93), (64,)),
    ("p128n128", dict(batch=1, seqlen=300, nheads=2, headdim=128, dstate=128, ngroups=1,
                      init="randn", seed=94), (128,)),
    ("short", dict(batch=3, seqlen=37, nheads=2, headdim=64, dstate=64, ngroups=1,
                   init="none", seed=95), (256,)),
]


@pytest.mark.parametrize("name,kw,qs", CASES, ids=[c[0] for c in CASES])
def test_chained_end_to_end(name, kw, qs):
    inp = inputs.make_inputs(io="bf16", **kw)
    for Q in qs:
        y, final, _ = chained(inp, Q)
        check(inp, y, final)


def test_chained_packed_and_scan_only():
    lengths = [1, 0, 300, 513, 77, 256]
    inp = inputs.make_inputs(1, sum(lengths), 8, 64, 128, 2, io="bf16", init="randn", lengths=lengths,
                             seed=96)
    for Q in (128, 256):
        y, final, _ = chained(inp, Q)
        check(inp, y, final)
        assert torch.equal(final[1].cpu(), inp["init"][1])  # the empty sequence
    inp["D"] = None
    y, final, _ = chained(inp, 256)
    check(inp, y, final, scan_only=True)


def test_chained_deterministic_and_agrees_with_staged():
    inp = inputs.make_inputs(2, 1500, 16, 64, 128, 2, io="bf16", init="randn", seed=97)
    y1, f1, _ = chained(inp, 256)
    y2, f2, _ = chained(inp, 256)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)
    d = to_dev(inp)
    y0, f0 = ssd.fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], dt_bias=d["dt_bias"],
                     init=d["init"], chunk_size=256)
    torch.cuda.synchronize()
    assert normwise(np64(f1), np64(f0)) <= 1e-4
    assert float((y1.float() - y0.float()).abs().max()) <= 2e-2


@pytest.mark.parametrize("cfg,heads", [(1, [0, 9, 63]), (3, [2, 31]), (4, [12, 57])])
def test_chained_full_size(cfg, heads):
    """The layer, the 512-chunk long-context and the packed workloads (sampled heads),
    with and without the skip term."""
    inp = inputs.config_inputs(cfg)
    y, final, _ = chained(inp, 256)
    check(inp, y, final, heads=heads)
    inp["D"] = None
    y, final, _ = chained(inp, 256)
    check(inp, y, final, heads=heads, scan_only=True)


def test_chained_saved_context_feeds_the_backward():
    """A chained forward that keeps its intermediates, then ssd_bwd from them: the
    gradients against the oracle (the gradient gate, normwise <= 3e-2)."""
    from oracle import recurrence as rec
    inp = inputs.make_inputs(2, 700, 16, 64, 128, 2, io="bf16", init="randn", bwd=True, d_final=True,
                             seed=98)
    y, final, ws = chained(inp, 256, save=True)
    d = to_dev(inp)
    g = ssd.bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["dout"], D=d["D"], dt_bias=d["dt_bias"],
                init=d["init"], d_final=d["d_final"], chunk_size=256, workspace=ws, from_saved=True)
    torch.cuda.synchronize()
    o = oracle_args(inp)
    a = inputs.to_f64(inp)
    ref = rec.bwd(o["x"], o["dt"], o["A"], o["B"], o["C"], a["dout"], D=o["D"], dt_bias=o["dt_bias"],
                  init=o["init"], d_final=a["d_final"], dt_softplus=o["dt_softplus"])
    for k in ("dx", "ddt", "dA", "dB", "dC", "dD", "d_dt_bias", "d_init"):
        assert normwise(np64(g[k]), ref[k]) <= 3e-2, k


def test_chained_unsupported_shapes_refused():
    for kw in (dict(headdim=16, dstate=16, io="f32"), dict(headdim=64, dstate=32, io="bf16")):
        inp = inputs.make_inputs(1, 100, 2, ngroups=1, **kw)
        d = to_dev(inp)
        with pytest.raises(ssd.SSDError) as e:
            ssd.fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], chunk_size=64, chained=True)
        assert e.value.status == 3


def test_chained_without_tokens():
    """No tokens at all (batched seqlen 0): the final states are the initial states."""
    inp = inputs.make_inputs(2, 0, 4, 64, 128, 2, io="bf16", init="randn", seed=99)
    y, final, _ = chained(inp, 256)
    assert y.numel() == 0 and torch.equal(final.cpu(), inp["init"])
