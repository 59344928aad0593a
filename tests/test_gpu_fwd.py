"""GPU parity of the forward path against the oracle (through the C ABI).

Stage tests feed each HIP stage the oracle's own intermediates (rounded to the
stage's input precision) and compare its output with the oracle's stage output,
so a failure names the kernel.  End-to-end tests compare ssd_fwd with the
token-by-token oracle.  Gates:
  fp32 io:  normwise relative error <= 1e-4 on y and final states;
  bf16 io:  y: max(|y - y_ref| - half a bf16 ulp of y_ref) <= 2e-2 (the output
            rounding alone costs half an ulp), final states normwise <= 1e-3,
            and a run without the D skip term (which dominates y) normwise <= 1e-2
            on the scan-only output.
"""
import ctypes

import numpy as np
import pytest
import torch

from helpers import (LOG2E, bf16_excess, bf16_kernels, cb_frag, cb_rows, gpu_fwd, has_gpu, normwise, np64,
                     oracle_args, to_dev)
from mamba_ssd_chunked_03_amd import inputs
from oracle import chunked, recurrence

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]

ssd = pytest.importorskip("mamba_ssd_chunked_03_amd.ssd")

# (name, make_inputs kwargs, chunk sizes)
CASES = [
    ("bf16_ragged", dict(batch=2, seqlen=700, nheads=4, headdim=64, dstate=128, ngroups=2,
                         io="bf16", init="randn", seed=11), (64, 128, 256)),
    ("bf16_p32n64", dict(batch=1, seqlen=333, nheads=2, headdim=32, dstate=64, ngroups=1,
                         io="bf16", init="randn", seed=12), (64,)),
    ("bf16_p128n32", dict(batch=1, seqlen=300, nheads=4, headdim=128, dstate=32, ngroups=4,
                          io="bf16", init="zeros", seed=13), (128,)),
    ("bf16_short", dict(batch=3, seqlen=37, nheads=2, headdim=64, dstate=64, ngroups=1,
                        io="bf16", init="randn", seed=14), (256,)),
    # an odd number of heads per group: kernels that pair a group's heads in one
    # workgroup take their one-head form here
    ("bf16_odd_heads", dict(batch=1, seqlen=420, nheads=3, headdim=64, dstate=128, ngroups=1,
                            io="bf16", init="randn", seed=17), (256,)),
    ("f32_cfg0_shape", dict(batch=1, seqlen=256, nheads=4, headdim=16, dstate=16, ngroups=1,
                            io="f32", dt_mode="direct", init="none", seed=0), (64,)),
    ("f32_ragged", dict(batch=2, seqlen=150, nheads=2, headdim=16, dstate=32, ngroups=1,
                        io="f32", init="randn", seed=15), (64, 128)),
    ("f32_p128", dict(batch=1, seqlen=70, nheads=2, headdim=128, dstate=128, ngroups=2,
                      io="f32", init="randn", seed=16), (64,)),
    # the fp32 matrix-core kernels over several row blocks and output tiles, with a
    # ragged last chunk, at every headdim and dstate above 16, two and four heads per group
    ("f32_p64n128", dict(batch=2, seqlen=600, nheads=4, headdim=64, dstate=128, ngroups=2,
                         io="f32", init="randn", seed=18), (128, 256)),
    ("f32_p128n64", dict(batch=1, seqlen=333, nheads=2, headdim=128, dstate=64, ngroups=1,
                         io="f32", init="randn", seed=19), (256,)),
    ("f32_p32n128", dict(batch=1, seqlen=290, nheads=8, headdim=32, dstate=128, ngroups=2,
                         io="f32", init="zeros", seed=20), (64, 256)),
    # bf16 io with headdim or dstate 16: the fp32 matrix-core kernels on bf16 tensors
    ("bf16_p16n64", dict(batch=2, seqlen=333, nheads=4, headdim=16, dstate=64, ngroups=2,
                         io="bf16", init="randn", seed=24), (64, 256)),
    ("bf16_p64n16", dict(batch=1, seqlen=400, nheads=8, headdim=64, dstate=16, ngroups=2,
                         io="bf16", init="randn", seed=25), (128,)),
    ("bf16_p16n16", dict(batch=1, seqlen=256, nheads=4, headdim=16, dstate=16, ngroups=1,
                         io="bf16", dt_mode="direct", init="none", seed=26), (64,)),
]
PACKED = [
    ("packed_bf16", dict(nheads=4, headdim=64, dstate=128, ngroups=2, io="bf16", init="randn",
                         seed=21), [1, 0, 300, 513, 77], (128, 256)),
    ("packed_f32", dict(nheads=2, headdim=16, dstate=16, ngroups=1, io="f32", init="randn",
                        seed=22), [65, 0, 0, 64, 3], (64,)),
    ("packed_f32_p64", dict(nheads=4, headdim=64, dstate=64, ngroups=2, io="f32", init="randn",
                            seed=23), [1, 0, 300, 257, 77], (128, 256)),
    ("packed_bf16_p16", dict(nheads=4, headdim=16, dstate=128, ngroups=2, io="bf16", init="randn",
                             seed=27), [1, 0, 300, 257, 77], (64, 256)),
]


def check_fwd(inp, y, final, io, label=""):
    o = oracle_args(inp)
    y_ref, f_ref = recurrence.fwd(**o)
    y = np64(y)
    f = np64(final)
    if io == "f32":
        assert normwise(y, y_ref) <= 1e-4, (label, normwise(y, y_ref))
        assert normwise(f, f_ref) <= 1e-4, (label, normwise(f, f_ref))
    else:
        assert bf16_excess(y, y_ref) <= 2e-2, (label, bf16_excess(y, y_ref))
        assert normwise(f, f_ref) <= 1e-3, (label, normwise(f, f_ref))
    return y_ref, f_ref


@pytest.mark.parametrize("name,kw,qs", CASES, ids=[c[0] for c in CASES])
def test_fwd_end_to_end(name, kw, qs):
    inp = inputs.make_inputs(**kw)
    for Q in qs:
        y, final = gpu_fwd(ssd, inp, Q)
        torch.cuda.synchronize()
        check_fwd(inp, y, final, kw["io"], "%s Q=%d" % (name, Q))


@pytest.mark.parametrize("name,kw,lengths,qs", PACKED, ids=[c[0] for c in PACKED])
def test_fwd_packed(name, kw, lengths, qs):
    inp = inputs.make_inputs(batch=1, seqlen=sum(lengths), lengths=lengths, **kw)
    for Q in qs:
        y, final = gpu_fwd(ssd, inp, Q)
        torch.cuda.synchronize()
        check_fwd(inp, y, final, kw["io"], "%s Q=%d" % (name, Q))
        # an empty sequence's final state is its init state, bit for bit
        assert torch.equal(final[1].cpu(), inp["init"][1])


def test_fwd_without_D_scan_only():
    # D x dominates y; without it the scan's own output must still match.
    inp = inputs.make_inputs(2, 700, 4, 64, 128, 2, io="bf16", init="randn", seed=31, with_D=False)
    y, final = gpu_fwd(ssd, inp, 256)
    y_ref, f_ref = recurrence.fwd(**oracle_args(inp))
    assert normwise(np64(y), y_ref) <= 1e-2
    assert normwise(np64(final), f_ref) <= 1e-3


def test_fwd_init_none_equals_zeros():
    a = inputs.make_inputs(1, 300, 2, 64, 64, 1, io="bf16", init="none", seed=32)
    b = dict(a)
    b["init"] = torch.zeros(1, 2, 64, 64)
    ya, fa = gpu_fwd(ssd, a, 128)
    yb, fb = gpu_fwd(ssd, b, 128)
    assert torch.equal(ya, yb) and torch.equal(fa, fb)


def test_fwd_deterministic():
    inp = inputs.make_inputs(2, 700, 4, 64, 128, 2, io="bf16", init="randn", seed=33)
    y1, f1 = gpu_fwd(ssd, inp, 256)
    y2, f2 = gpu_fwd(ssd, inp, 256)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


def test_fwd_empty_sequence_batch():
    inp = inputs.make_inputs(2, 0, 2, 64, 64, 1, io="bf16", init="randn", seed=34)
    y, final = gpu_fwd(ssd, inp, 64)
    torch.cuda.synchronize()
    assert y.numel() == 0 and torch.equal(final.cpu(), inp["init"])


def test_fwd_no_nan_inf_full_decay_range():
    # strong decays (large A * delta) must underflow cleanly to zero, never overflow
    inp = inputs.make_inputs(1, 512, 4, 64, 128, 2, io="bf16", init="randn", seed=35)
    inp["dt"] = inp["dt"] + 6.0  # delta ~ 2-10, chunk decays far below fp32 range
    y, final = gpu_fwd(ssd, inp, 256)
    assert torch.isfinite(y.float()).all() and torch.isfinite(final).all()
    check_fwd(inp, y, final, "bf16", "strong decay")


# ------------------------------------------------------------ stage parity ----
def stage_case(kw, lengths=None, Q=128):
    if lengths is not None:
        inp = inputs.make_inputs(batch=1, seqlen=sum(lengths), lengths=lengths, **kw)
    else:
        inp = inputs.make_inputs(**kw)
    o = oracle_args(inp)
    y, final, mid = chunked.fwd(**o, chunk_size=Q)
    st = ssd.Stages(inp["x"].cuda(), inp["B"].cuda(),
                    None if inp["cu_seqlens"] is None else inp["cu_seqlens"].cuda(), Q,
                    inp["dt_softplus"])
    return inp, o, mid, st, len(mid["chunks"])


STAGE_KW = [
    (dict(batch=2, seqlen=700, nheads=4, headdim=64, dstate=128, ngroups=2, io="bf16",
          init="randn", seed=41), None, 256),
    (dict(nheads=4, headdim=64, dstate=128, ngroups=2, io="bf16", init="randn", seed=42),
     [1, 0, 300, 513, 77], 128),
    (dict(batch=1, seqlen=200, nheads=2, headdim=16, dstate=16, ngroups=1, io="f32",
          init="randn", seed=43), None, 64),
    (dict(batch=1, seqlen=200, nheads=2, headdim=16, dstate=32, ngroups=1, io="bf16",
          init="randn", seed=44), None, 64),
]


@pytest.mark.parametrize("kw,lengths,Q", STAGE_KW)
def test_stages(kw, lengths, Q):
    inp, o, mid, st, nk = stage_case(kw, lengths, Q)
    d = to_dev(inp)
    f32 = lambda a: torch.tensor(a, dtype=torch.float32, device="cuda")
    # stage 1: cumsum
    delta, acs, decay = st.chunk_cumsum(d["dt"], d["A"], d["dt_bias"])
    torch.cuda.synchronize()
    assert normwise(np64(delta)[:nk], mid["delta"]) <= 1e-5
    assert normwise(np64(acs)[:nk] / LOG2E, mid["acs"]) <= 1e-5
    last = np.array([mid["acs"][k, :, ch["len"] - 1] for k, ch in enumerate(mid["chunks"])])
    if nk:
        assert normwise(np64(decay)[:nk] / LOG2E, last) <= 1e-5
    # oracle intermediates as stage inputs
    nck = delta.shape[0]
    pad = lambda a: np.concatenate([a, np.zeros((nck - nk,) + a.shape[1:])]) if nck > nk else a
    o_delta, o_acs = f32(pad(mid["delta"])), f32(pad(mid["acs"]) * LOG2E)
    o_decay = f32(pad(last * LOG2E)) if nk else decay
    # stage 2: chunk states
    T = st.chunk_state(d["x"], d["B"], o_delta, o_acs)
    torch.cuda.synchronize()
    assert normwise(np64(T)[:nk], mid["T"]) <= (1e-5 if kw["io"] == "f32" else 1e-4)
    # stage 3: state passing
    Hp, final = st.state_passing(f32(pad(mid["T"])), o_decay, d["init"])
    torch.cuda.synchronize()
    _, f_ref = chunked.state_passing(mid["T"], mid["acs"], mid["chunks"],
                                     len(lengths) if lengths else kw["batch"], o["init"])
    assert normwise(np64(Hp)[:nk], mid["Hin"]) <= 1e-5
    assert normwise(np64(final), f_ref) <= 1e-5
    # stage 4: C B^T (lower triangle; fragment order on the bf16 kernels, include/ssd.h)
    frag = bf16_kernels(kw["io"], kw["headdim"], kw["dstate"])
    CB = np64(st.bmm_chunk(d["B"], d["C"]))[:nk]
    CB = cb_rows(CB, Q) if frag else CB
    mask = np.tril(np.ones((Q, Q), dtype=bool))
    lim = 1e-5 if kw["io"] == "f32" else 4e-3
    for k, ch in enumerate(mid["chunks"]):
        n = ch["len"]
        m = mask[:n, :n]
        assert normwise(CB[k][:, :n, :n][:, m], mid["CB"][k][:, :n, :n][:, m]) <= lim
    # stage 5: output from the oracle's intermediates
    CBt = torch.tensor(pad(mid["CB"]), dtype=d["x"].dtype, device="cuda")
    y = st.chunk_scan(d["x"], d["C"], cb_frag(CBt, Q).contiguous() if frag else CBt, o_delta, o_acs,
                      f32(pad(mid["Hin"])), d["D"])
    torch.cuda.synchronize()
    y_ref = chunked.chunk_scan(o["x"], o["C"], np64(CBt.float()), mid["delta"], mid["acs"],
                               mid["Hin"], mid["chunks"], o["D"])
    if kw["io"] == "f32":
        assert normwise(np64(y), y_ref) <= 1e-5
    else:
        assert bf16_excess(np64(y), y_ref) <= 2e-2


# ------------------------------------------------- full sizes, sampled heads ----
@pytest.mark.parametrize("cfg,heads", [(1, [0, 21, 63]), (3, [5, 30]), (4, [7, 50])])
def test_full_size_sampled(cfg, heads):
    inp = inputs.config_inputs(cfg)
    y, final = gpu_fwd(ssd, inp, inputs.CONFIGS[cfg]["chunk"])
    torch.cuda.synchronize()
    o = oracle_args(inp)
    y_ref, f_ref = recurrence.fwd(**o, heads=heads)
    ys = np64(y[:, :, heads])
    fs = np64(final[:, heads])
    assert bf16_excess(ys, y_ref) <= 2e-2
    assert normwise(fs, f_ref) <= 1e-3
    assert torch.isfinite(y.float()).all()


def _up256(n):
    return (n + 255) // 256 * 256


@pytest.mark.gpu
@pytest.mark.parametrize("kw,lengths,Q", STAGE_KW)
def test_fused_cumsum_matches_stage(kw, lengths, Q):
    """ssd_fwd forms delta, acs and the chunk decays inside the chunk-state kernel
    (bf16 path): they must equal the stage-1 kernel's outputs bit for bit (the
    saved context of a forward is what a recomputing backward would build).
    Offsets follow the workspace layout: [chunk table, sequence offsets when
    packed], delta, acs, decays, each piece 256-byte aligned."""
    inp, o, mid, st, nk = stage_case(kw, lengths, Q)
    d = to_dev(inp)
    p = st.prob
    ws = torch.empty(ssd.lib().ssd_bwd_workspace_bytes(ctypes.byref(p), Q, st.packed),
                     dtype=torch.uint8, device="cuda")
    gpu_fwd(ssd, inp, Q, workspace=ws, save_for_backward=True)
    delta, acs, decay = st.chunk_cumsum(d["dt"], d["A"], d["dt_bias"])
    torch.cuda.synchronize()
    nck, H = delta.shape[0], p.nheads
    off = _up256(nck * 16) + _up256((p.nseq + 1) * 4) if st.packed else 0
    n_tok = nck * H * Q
    w_delta = ws[off:off + 4 * n_tok].view(torch.float32).view(nck, H, Q)
    off += _up256(4 * n_tok)
    w_acs = ws[off:off + 4 * n_tok].view(torch.float32).view(nck, H, Q)
    off += _up256(4 * n_tok)
    w_decay = ws[off:off + 4 * nck * H].view(torch.float32).view(nck, H)
    live = [k for k in range(nck) if k < nk]  # chunk slots past the last chunk are never written
    assert torch.equal(w_delta[live], delta[live])
    assert torch.equal(w_acs[live], acs[live])
    assert torch.equal(w_decay[live], decay[live])


def _up(n):
    return (n + 255) // 256 * 256


@pytest.mark.parametrize("lengths", [None, [300, 0, 513, 77]], ids=["batched", "packed"])
def test_cb_in_chunk_state_matches_stage_kernel(lengths):
    """Where the chunk-state kernel forms C.B^T (8 heads per group, chunk 256), the
    C.B^T and its transpose that a saving forward leaves in the workspace equal,
    bit for bit, what the separate C.B^T stage kernel computes, on every 64 x 64
    lower tile that starts inside its chunk.  The workspace offsets follow the
    saved-context layout: delta, acs (nck, H, Q), decay (nck, H), chunk states
    (nck, H, P, N) fp32, passed states in bf16, C.B^T (nck, G, Q, Q) bf16, the chained
    forward's 16 + nck * H flag words, then (backward part) its transpose, each rounded
    up to 256 bytes."""
    H, P, N, G, Q = 16, 64, 128, 2, 256
    kw = dict(nheads=H, headdim=P, dstate=N, ngroups=G, io="bf16", init="randn", seed=51)
    if lengths is None:
        inp = inputs.make_inputs(batch=2, seqlen=700, **kw)
    else:
        inp = inputs.make_inputs(batch=1, seqlen=sum(lengths), lengths=lengths, **kw)
    d = to_dev(inp)
    prob = ssd.problem(d["x"], d["B"], d["cu_seqlens"])
    packed = int(lengths is not None)
    assert ssd.lib().ssd_fwd_kernel_mask(ctypes.byref(prob), Q, packed) == 0xB
    nck = ssd.num_chunks(prob, Q, packed)
    ws = torch.zeros(ssd.lib().ssd_bwd_workspace_bytes(ctypes.byref(prob), Q, packed),
                     dtype=torch.uint8, device="cuda")
    ssd.fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], dt_bias=d["dt_bias"], init=d["init"],
            cu_seqlens=d["cu_seqlens"], chunk_size=Q, dt_softplus=inp["dt_softplus"], workspace=ws,
            save_for_backward=True)
    st = ssd.Stages(d["x"], d["B"], d["cu_seqlens"], Q, inp["dt_softplus"])
    ref = st.bmm_chunk(d["B"], d["C"])
    torch.cuda.synchronize()
    o = 0
    if packed:
        o += _up(nck * 16) + _up((len(lengths) + 1) * 4)
    o += 2 * _up(nck * H * Q * 4) + _up(nck * H * 4) + _up(nck * H * P * N * 4) + _up(nck * H * P * N * 2)
    ncb = nck * G * Q * Q
    cb = ws[o:o + ncb * 2].view(torch.int16).view(nck, G, Q, Q).cpu()
    o += _up(ncb * 2)
    o += _up((16 + nck * H) * 4)  # the chained forward's flags (end of the forward part)
    cbt = ws[o:o + ncb * 2].view(torch.int16).view(nck, G, Q, Q).cpu()
    ref = ref.view(torch.int16).cpu()
    # all three in fragment order (include/ssd.h); compared as rows
    cb, cbt, ref = cb_rows(cb, Q), cb_rows(cbt, Q), cb_rows(ref, Q)
    # chunk lengths: batched rows cut from their first token, packed sequences likewise
    lens = []
    if packed:
        for n in lengths:
            lens += [min(Q, n - c * Q) for c in range((n + Q - 1) // Q)]
    else:
        lens = [min(Q, 700 - c * Q) for c in range((700 + Q - 1) // Q)] * 2
    assert len(lens) <= nck
    checked = 0
    for k, n in enumerate(lens):
        for ti in range(Q // 64):
            if ti * 64 >= n:
                continue
            for tj in range(ti + 1):
                rs, cs = slice(ti * 64, ti * 64 + 64), slice(tj * 64, tj * 64 + 64)
                assert torch.equal(cb[k, :, rs, cs], ref[k, :, rs, cs]), (k, ti, tj)
                assert torch.equal(cbt[k, :, cs, rs].transpose(-1, -2), ref[k, :, rs, cs]), (k, ti, tj)
                checked += 1
    assert checked > 0


FUSED_CB = dict(nheads=16, headdim=64, dstate=128, ngroups=2, io="bf16", init="randn")


@pytest.mark.parametrize("lengths", [None, [300, 0, 513, 77]], ids=["batched", "packed"])
def test_fwd_cb_in_chunk_state(lengths):
    """End to end against the oracle on a shape whose chunk-state kernel forms C.B^T."""
    if lengths is None:
        inp = inputs.make_inputs(batch=2, seqlen=700, seed=52, **FUSED_CB)
    else:
        inp = inputs.make_inputs(batch=1, seqlen=sum(lengths), lengths=lengths, seed=53, **FUSED_CB)
    y, final = gpu_fwd(ssd, inp, 256)
    torch.cuda.synchronize()
    check_fwd(inp, y, final, "bf16", "cb_in_chunk_state")


# The skip term D x dominates y (|D x| up to ~11 against an SSM term of ~0.01-0.03),
# so a scan error as large as the SSM term itself could hide under the y gate.
# Without D the output is the scan alone, gated normwise at 1e-2.  Every full-size
# workload here takes the path whose chunk-state kernel also forms C.B^T.
@pytest.mark.parametrize("cfg,heads", [(1, list(range(64))), (3, [5, 16, 17, 30]),
                                       (4, list(range(56, 64)))])
def test_full_size_scan_only(cfg, heads):
    """The layer workload on every head (both batch rows, all 64 heads); the long
    context and packed workloads on a group's worth of sampled heads."""
    inp = inputs.config_inputs(cfg)
    inp["D"] = None
    d = to_dev(inp)
    prob = ssd.problem(d["x"], d["B"], d["cu_seqlens"])
    assert ssd.lib().ssd_fwd_kernel_mask(ctypes.byref(prob), 256, int(d["cu_seqlens"] is not None)) == 0xB
    y, final = gpu_fwd(ssd, inp, inputs.CONFIGS[cfg]["chunk"])
    torch.cuda.synchronize()
    y_ref, f_ref = recurrence.fwd(**oracle_args(inp), heads=heads)
    assert normwise(np64(y[:, :, heads]), y_ref) <= 1e-2, normwise(np64(y[:, :, heads]), y_ref)
    assert normwise(np64(final[:, heads]), f_ref) <= 1e-3


@pytest.mark.parametrize("lengths", [None, [300, 0, 513, 77]], ids=["batched", "packed"])
def test_fwd_cb_in_chunk_state_scan_only(lengths):
    """The scan-only output (no D) on a shape whose chunk-state kernel forms C.B^T."""
    if lengths is None:
        inp = inputs.make_inputs(batch=2, seqlen=700, seed=54, with_D=False, **FUSED_CB)
    else:
        inp = inputs.make_inputs(batch=1, seqlen=sum(lengths), lengths=lengths, seed=55,
                                 with_D=False, **FUSED_CB)
    y, final = gpu_fwd(ssd, inp, 256)
    torch.cuda.synchronize()
    y_ref, f_ref = recurrence.fwd(**oracle_args(inp))
    assert normwise(np64(y), y_ref) <= 1e-2
    assert normwise(np64(final), f_ref) <= 1e-3


# ------------------------------------- sequential-carry state passing (A/B) ----
@pytest.mark.parametrize("variant", range(1, 8))
@pytest.mark.parametrize("kw,lengths,Q", STAGE_KW)
def test_stage_state_passing_variants(kw, lengths, Q, variant):
    """Every state-passing kernel (SSD_FLAG_SCAN_VARIANT 1..7: the associative scan
    at four segment shapes, the sequential carry with 1, 4, 8 chunks in flight) on
    the oracle's chunk states: the gates of the stage test."""
    inp, o, mid, st, nk = stage_case(kw, lengths, Q)
    d = to_dev(inp)
    f32 = lambda a: torch.tensor(a, dtype=torch.float32, device="cuda")
    nck = st.nck
    pad = lambda a: np.concatenate([a, np.zeros((nck - nk,) + a.shape[1:])]) if nck > nk else a
    last = np.array([mid["acs"][k, :, ch["len"] - 1] for k, ch in enumerate(mid["chunks"])])
    o_decay = f32(pad(last * LOG2E)) if nk else torch.zeros(nck, kw["nheads"], device="cuda")
    Hp, final = st.state_passing(f32(pad(mid["T"])), o_decay, d["init"], variant=variant)
    torch.cuda.synchronize()
    _, f_ref = chunked.state_passing(mid["T"], mid["acs"], mid["chunks"],
                                     len(lengths) if lengths else kw["batch"], o["init"])
    assert normwise(np64(Hp)[:nk], mid["Hin"]) <= 1e-5
    assert normwise(np64(final), f_ref) <= 1e-5


@pytest.mark.parametrize("variant", [5, 7, 4])
@pytest.mark.parametrize("case", ["ragged", "packed", "long_context"])
def test_fwd_scan_variants(case, variant):
    """ssd_fwd with the plain sequential carry (5), the streamed one (7) and the
    widest associative scan (4), against the oracle."""
    if case == "ragged":
        inp = inputs.make_inputs(2, 700, 16, 64, 128, 2, io="bf16", init="randn", seed=81)
        heads, Q = None, 256
    elif case == "packed":
        inp = inputs.make_inputs(1, 891, 4, 64, 128, 2, io="bf16", init="randn", seed=82,
                                 lengths=[1, 0, 300, 513, 77])
        heads, Q = None, 128
    else:
        inp = inputs.config_inputs(3)   # 512 chunks: the longest carry chain
        heads, Q = [9, 31], 256
    y, final = gpu_fwd(ssd, inp, Q, scan_variant=variant)
    torch.cuda.synchronize()
    y_ref, f_ref = recurrence.fwd(**oracle_args(inp), heads=heads)
    if heads is not None:
        y, final = y[:, :, heads], final[:, heads]
    assert bf16_excess(np64(y), y_ref) <= 2e-2
    assert normwise(np64(final), f_ref) <= 1e-3
