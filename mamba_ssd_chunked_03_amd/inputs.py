"""Seeded synthetic inputs for the SSD scan (shared by tests, bench and smoke).

This module draws random inputs and nothing else: it holds none of the
scan's arithmetic, imports neither the HIP binding nor the oracle, and is the
one piece of code that both sides consume.

Workloads (the pages measure a Mamba-2 layer of a hybrid model at batch 2,
sequence length 8192, in bf16; the layer's weights and dimensions are not
published, so these seeded shapes and distributions stand in for it):

    id  shape (B, L, H, P, N, G, Q)             io    notes
    0   1, 256, 4, 16, 16, 1, 64                f32   dt = softplus(N(0,1) - 2) fed
                                                      directly (no bias, no softplus)
    1   2, 8192, 64, 64, 128, 8, 256            bf16  raw dt ~ N(0,1), bias U[-4,-2],
                                                      softplus in the kernel; zero init
    2   as 1, forward + backward                bf16  dout ~ N(0,1) bf16
    3   1, 131072, 32, 64, 128, 4, 256          bf16  init ~ 0.1 N(0,1) (fp32)
    4   1 packed row of 65536 tokens, 64, 64,   bf16  lengths U[512, 16384] (integers),
        128, 8, 256                                   per-sequence init ~ 0.1 N(0,1)

Value distributions: x ~ N(0,1); B, C ~ N(0,1)/sqrt(dstate); A = -exp(U[0, ln 16])
per head; D ~ N(0,1) per head.  Draw order is fixed: x, B, C, dt, dt_bias, A, D,
init, dout, all from one ``torch.Generator`` seeded with the seed (config id by
default); packed lengths are drawn first with ``numpy.random.default_rng(seed)``.
Tensors are drawn in fp32 on the CPU and cast to bf16 with round-to-nearest-even.
"""
import math

import numpy as np
import torch

CONFIGS = {
    0: dict(batch=1, seqlen=256, nheads=4, headdim=16, dstate=16, ngroups=1, chunk=64,
            io="f32", dt_mode="direct", init="none", varlen=None, bwd=False),
    1: dict(batch=2, seqlen=8192, nheads=64, headdim=64, dstate=128, ngroups=8, chunk=256,
            io="bf16", dt_mode="softplus", init="zeros", varlen=None, bwd=False),
    2: dict(batch=2, seqlen=8192, nheads=64, headdim=64, dstate=128, ngroups=8, chunk=256,
            io="bf16", dt_mode="softplus", init="zeros", varlen=None, bwd=True),
    3: dict(batch=1, seqlen=131072, nheads=32, headdim=64, dstate=128, ngroups=4, chunk=256,
            io="bf16", dt_mode="softplus", init="randn", varlen=None, bwd=False),
    4: dict(batch=1, seqlen=65536, nheads=64, headdim=64, dstate=128, ngroups=8, chunk=256,
            io="bf16", dt_mode="softplus", init="randn", varlen=(512, 16384), bwd=True),
}


def varlen_lengths(total, lo, hi, seed):
    """Integer lengths uniform on [lo, hi] until they sum to ``total``; the last
    one is clipped to the remainder (and may be shorter than ``lo``)."""
    rng = np.random.default_rng(seed)
    out = []
    while sum(out) < total:
        n = int(rng.integers(lo, hi + 1))
        out.append(min(n, total - sum(out)))
    return out


def cu_from_lengths(lengths):
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def make_inputs(batch, seqlen, nheads, headdim, dstate, ngroups, io="bf16",
                dt_mode="softplus", init="zeros", lengths=None, bwd=False, seed=0,
                with_D=True, d_final=False):
    """Draw one problem's inputs on the CPU.

    ``dt_mode``: "direct" gives dt = softplus(N(0,1) - 2) as the effective step
    (the library then runs with dt_softplus off and no bias); "softplus" gives raw
    dt ~ N(0,1) and dt_bias ~ U[-4,-2] (the library applies softplus(dt + bias)).
    ``init``: "none" (no tensor), "zeros", or "randn" (0.1 * N(0,1)).
    ``lengths``: packed sequence lengths (batch must be 1 and they must sum to
    seqlen); the result then carries ``cu_seqlens``.
    """
    g = torch.Generator().manual_seed(seed)
    io_dtype = torch.float32 if io == "f32" else torch.bfloat16
    nseq = batch if lengths is None else len(lengths)
    if lengths is not None:
        assert batch == 1 and sum(lengths) == seqlen
    x = torch.randn(batch, seqlen, nheads, headdim, generator=g)
    Bm = torch.randn(batch, seqlen, ngroups, dstate, generator=g) / math.sqrt(dstate)
    Cm = torch.randn(batch, seqlen, ngroups, dstate, generator=g) / math.sqrt(dstate)
    dt_raw = torch.randn(batch, seqlen, nheads, generator=g)
    bias = torch.rand(nheads, generator=g) * 2.0 - 4.0
    A = -torch.exp(torch.rand(nheads, generator=g) * math.log(16.0))
    D = torch.randn(nheads, generator=g)
    init_t = 0.1 * torch.randn(nseq, nheads, headdim, dstate, generator=g)
    dout = torch.randn(batch, seqlen, nheads, headdim, generator=g) if bwd else None
    dfin = 0.1 * torch.randn(nseq, nheads, headdim, dstate, generator=g) if (bwd and d_final) else None
    if dt_mode == "direct":
        dt = torch.nn.functional.softplus(dt_raw - 2.0)
        dt_bias, softplus = None, False
    else:
        dt, dt_bias, softplus = dt_raw, bias, True
    if init == "none":
        init_states = None
    elif init == "zeros":
        init_states = torch.zeros(nseq, nheads, headdim, dstate)
    else:
        init_states = init_t
    out = dict(
        x=x.to(io_dtype).contiguous(), B=Bm.to(io_dtype).contiguous(),
        C=Cm.to(io_dtype).contiguous(), dt=dt.float().contiguous(),
        dt_bias=dt_bias, A=A.float(), D=D.float() if with_D else None,
        init=init_states, dt_softplus=softplus,
        cu_seqlens=None if lengths is None else cu_from_lengths(lengths),
        dout=None if dout is None else dout.to(io_dtype).contiguous(),
        d_final=dfin,
    )
    return out


def config_inputs(cfg_id, seed=None, **over):
    """Inputs of one named workload (see the table above)."""
    c = dict(CONFIGS[cfg_id])
    c.update(over)
    seed = cfg_id if seed is None else seed
    lengths = None
    if c["varlen"] is not None:
        lo, hi = c["varlen"]
        lengths = varlen_lengths(c["seqlen"], lo, hi, seed)
    return make_inputs(c["batch"], c["seqlen"], c["nheads"], c["headdim"], c["dstate"],
                       c["ngroups"], io=c["io"], dt_mode=c["dt_mode"], init=c["init"],
                       lengths=lengths, bwd=c["bwd"], seed=seed)


def to_f64(inp):
    """numpy float64 copies of a problem's tensors (exact widening)."""
    out = {}
    for k, v in inp.items():
        if isinstance(v, torch.Tensor):
            out[k] = v.detach().cpu().double().numpy() if v.is_floating_point() else v.cpu().numpy()
        else:
            out[k] = v
    return out
