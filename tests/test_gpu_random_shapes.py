"""GPU parity over seeded random shapes: forward and backward against the oracle.

Each case draws (io dtype, headdim, dstate, groups, heads per group, chunk size,
batch rows or packed sequence lengths, initial and final states, skip term)
from a fixed seed, so the set is the same on every run; together they reach
shape combinations the hand-picked cases do not (one head per group, headdim
and dstate far apart, chunks longer than the sequence, empty and one-token
sequences); half of them are held to the bf16 matrix-core kernels.  Gates as
elsewhere: fp32 io normwise <= 1e-4; bf16 io y within 2e-2 beyond half a bf16
ulp (and normwise <= 1e-2 without the skip term), final states <= 1e-3,
gradients <= 3e-2; the per-head sums dA, d_dt_bias and dD may instead be held
to that bar against the summed magnitudes of their terms (check_bwd).

The same shapes also check what include/ssd.h promises of each opt-in form:
one stream, every chunk-state form and the saved context give the default's
results bit for bit; the one-kernel dB/dC gives its dB, dC, dx and d_init bit
for bit; a forced state-passing kernel and the chained forward agree to
rounding, so they are held to the oracle gates.
"""
import ctypes

import numpy as np
import pytest
import torch

from helpers import bf16_excess, gpu_bwd, gpu_fwd, has_gpu, normwise, np64, oracle_args, to_dev
from mamba_ssd_chunked_03_amd import inputs
from oracle import recurrence

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]

ssd = pytest.importorskip("mamba_ssd_chunked_03_amd.ssd")

KEYS = ["dx", "ddt", "dA", "dB", "dC", "dD", "d_dt_bias", "d_init"]


def draw(seed, main=False):
    """One case from its seed.  main: bf16 with headdim and dstate >= 32 (the bf16
    matrix-core kernels), eight heads per group and chunk 256 drawn more often (the
    shape where the chunk-state kernel also forms C.B^T)."""
    rng = np.random.default_rng(1000 + seed)
    if main:
        io = "bf16"
        P, N = (int(v) for v in rng.choice([32, 64, 128], size=2))
        G = int(rng.choice([1, 2]))
        hpg = int(rng.choice([1, 2, 4, 8, 8]))
        Q = int(rng.choice([64, 128, 256, 256]))
    else:
        io = ["bf16", "f32"][rng.integers(2)]
        P, N = (int(v) for v in rng.choice([16, 32, 64, 128], size=2))
        G = int(rng.choice([1, 2]))
        hpg = int(rng.choice([1, 2, 4, 8]))
        Q = int(rng.choice([64, 128, 256]))
    kw = dict(nheads=G * hpg, headdim=P, dstate=N, ngroups=G, io=io, seed=2000 + seed,
              init=["zeros", "randn", "none"][rng.integers(3)], with_D=bool(rng.integers(2)),
              d_final=bool(rng.integers(2)), bwd=True)
    if rng.integers(3) == 0:  # packed sequences, some empty or one token long
        lengths = [int(v) for v in rng.choice([0, 1, 37, 200, 300, 513], size=int(rng.integers(2, 5)))]
        if sum(lengths) == 0:
            lengths[0] = 5
        kw.update(batch=1, seqlen=sum(lengths), lengths=lengths)
    else:
        kw.update(batch=int(rng.integers(1, 4)), seqlen=int(rng.integers(1, 600)))
    if kw["init"] == "none" and kw.get("lengths") is None and rng.integers(2):
        kw["dt_mode"] = "direct"  # raw step sizes, no softplus and no bias
    return kw, Q


# 24 cases over every supported dtype and size, 24 on the bf16 matrix-core kernels
CASES = [(s, False) for s in range(24)] + [(s, True) for s in range(24, 48)]
IDS = ["%s%d" % ("main" if m else "mix", s) for s, m in CASES]


def label_of(seed, kw, Q):
    return "seed %d: %s Q=%d" % (seed, {k: v for k, v in kw.items() if k != "seed"}, Q)


def oracle_both(inp):
    o = oracle_args(inp)
    y_ref, f_ref = recurrence.fwd(**o)
    a = inputs.to_f64(inp)
    ref = recurrence.bwd(o["x"], o["dt"], o["A"], o["B"], o["C"], a["dout"], D=o["D"],
                         dt_bias=o["dt_bias"], init=o["init"], d_final=a["d_final"],
                         dt_softplus=o["dt_softplus"], cu_seqlens=o["cu_seqlens"])
    return y_ref, f_ref, ref


def check_fwd(kw, y, final, y_ref, f_ref, label):
    if kw["io"] == "f32":
        assert normwise(np64(y), y_ref) <= 1e-4, label
        assert normwise(np64(final), f_ref) <= 1e-4, label
    else:
        assert bf16_excess(np64(y), y_ref) <= 2e-2, label
        if not kw["with_D"]:  # the scan's output alone: normwise too
            assert normwise(np64(y), y_ref) <= 1e-2, label
        assert normwise(np64(final), f_ref) <= 1e-3, label


def sum_scales(inp, ref):
    """Per head, the summed magnitudes of the terms that dA, d_dt_bias and dD add up:
    the oracle's dA_abs, sum |ddt| over tokens, sum |dy . x| over tokens."""
    a = inputs.to_f64(inp)
    sc = {"dA": ref["dA_abs"], "d_dt_bias": np.abs(ref["ddt"]).sum(axis=(0, 1))}
    if ref["dD"] is not None:
        sc["dD"] = np.abs(np.einsum("bthp,bthp->bth", a["dout"], a["x"])).sum(axis=(0, 1))
    return sc


def check_bwd(io, g, ref, label, scales=None):
    """normwise <= tol for every gradient.  dA, d_dt_bias and dD are per-head sums
    over tokens whose terms can cancel (with one head, dA came out at 1/84 to 1/562
    of its terms' summed size in drawn cases): for them the error may instead be
    measured against those summed magnitudes, the usual error measure of a sum."""
    tol = 1e-4 if io == "f32" else 3e-2
    errs = {}
    for k in KEYS:
        if ref[k] is None:
            assert g[k] is None or k == "dD", (label, k)
            continue
        errs[k] = normwise(np64(g[k]), ref[k])
        if scales is not None and k in scales and float(np.max(scales[k])) > 0:
            diff = float(np.max(np.abs(np64(g[k]) - ref[k])))
            errs[k] = min(errs[k], diff / float(np.max(scales[k])))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, (label, errs)


def same(a, b, keys=KEYS):
    return [k for k in keys if (a[k] is None) != (b[k] is None) or
            (a[k] is not None and not torch.equal(a[k], b[k]))]


@pytest.mark.parametrize("seed,main", CASES, ids=IDS)
def test_random_shape(seed, main):
    kw, Q = draw(seed, main)
    label = label_of(seed, kw, Q)
    inp = inputs.make_inputs(**kw)
    y_ref, f_ref, ref = oracle_both(inp)
    y, final = gpu_fwd(ssd, inp, Q)
    g = gpu_bwd(ssd, inp, Q)
    torch.cuda.synchronize()
    check_fwd(kw, y, final, y_ref, f_ref, label)
    check_bwd(kw["io"], g, ref, label, sum_scales(inp, ref))


def saved_workspace(inp, Q, flags=0):
    d = to_dev(inp)
    prob = ssd.problem(d["x"], d["B"], d["cu_seqlens"], flags=flags)
    need = ssd.lib().ssd_bwd_workspace_bytes(ctypes.byref(prob), Q, int(d["cu_seqlens"] is not None))
    return torch.empty(max(1, need), dtype=torch.uint8, device="cuda")


def unsupported(call):
    """call() or None where the library refuses the shape (SSD_ERR_UNSUPPORTED)."""
    try:
        return call()
    except ssd.SSDError as e:
        assert e.status == 3, e
        return None


@pytest.mark.parametrize("seed,main", CASES, ids=IDS)
def test_random_shape_opt_in_forms(seed, main):
    kw, Q = draw(seed, main)
    label = label_of(seed, kw, Q)
    io = kw["io"]
    inp = inputs.make_inputs(**kw)
    y0, f0 = gpu_fwd(ssd, inp, Q)
    g0 = gpu_bwd(ssd, inp, Q)
    # one stream: the same kernels in the same order
    y1, f1 = gpu_fwd(ssd, inp, Q, one_stream=True)
    g1 = gpu_bwd(ssd, inp, Q, one_stream=True)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(f0, f1), label
    assert not same(g0, g1), (label, "one stream", same(g0, g1))
    # the saved context gives the recomputing pair's gradients
    ws = saved_workspace(inp, Q)
    y2, f2 = gpu_fwd(ssd, inp, Q, workspace=ws, save_for_backward=True)
    g2 = gpu_bwd(ssd, inp, Q, workspace=ws, from_saved=True)
    torch.cuda.synchronize()
    assert torch.equal(y0, y2) and torch.equal(f0, f2), label
    assert not same(g0, g2), (label, "saved context", same(g0, g2))
    # every chunk-state form the shape can run: bit for bit
    for v in (1, 2, 3):
        r = unsupported(lambda: gpu_fwd(ssd, inp, Q, cs_variant=v))
        if r is None:
            continue
        gv = gpu_bwd(ssd, inp, Q, cs_variant=v)
        torch.cuda.synchronize()
        assert torch.equal(y0, r[0]) and torch.equal(f0, r[1]), (label, "chunk-state form", v)
        assert not same(g0, gv), (label, "chunk-state form", v, same(g0, gv))
    # the one-kernel dB/dC (the three-kernel form where it does not apply)
    gf = gpu_bwd(ssd, inp, Q, fused=True)
    torch.cuda.synchronize()
    assert not same(g0, gf, ["dx", "dB", "dC", "d_init"]), (label, "fused dB/dC")
    y_ref, f_ref, ref = oracle_both(inp)
    sc = sum_scales(inp, ref)
    check_bwd(io, gf, ref, label + " fused dB/dC", sc)
    # a forced state-passing kernel (associative scan shapes 1-4, sequential carry 5-7)
    v = 1 + seed % 7
    ys, fs = gpu_fwd(ssd, inp, Q, scan_variant=v)
    gs = gpu_bwd(ssd, inp, Q, scan_variant=v)
    torch.cuda.synchronize()
    check_fwd(kw, ys, fs, y_ref, f_ref, "%s scan variant %d" % (label, v))
    check_bwd(io, gs, ref, "%s scan variant %d" % (label, v), sc)
    # the chained forward where the shape allows it; its saved context feeds the backward
    wc = saved_workspace(inp, Q)
    r = unsupported(lambda: gpu_fwd(ssd, inp, Q, chained=True, workspace=wc, save_for_backward=True))
    if r is not None:
        torch.cuda.synchronize()
        d = to_dev(inp)
        prob = ssd.problem(d["x"], d["B"], d["cu_seqlens"])
        off = ssd.lib().ssd_fwd_chained_error_offset(ctypes.byref(prob), Q, int(d["cu_seqlens"] is not None))
        assert int(wc[off:off + 4].view(torch.int32).item()) == 0, (label, "a wait for a carry ran out")
        gc = gpu_bwd(ssd, inp, Q, workspace=wc, from_saved=True)
        torch.cuda.synchronize()
        check_fwd(kw, r[0], r[1], y_ref, f_ref, label + " chained")
        check_bwd(io, gc, ref, label + " chained, saved context", sc)
