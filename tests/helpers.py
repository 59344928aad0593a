"""Shared test helpers: error measures and oracle/GPU plumbing."""
import math

import numpy as np
import torch

from mamba_ssd_chunked_03_amd import inputs

LOG2E = 1.0 / math.log(2.0)


def has_gpu():
    return torch.cuda.is_available()


def to_dev(inp, dev="cuda"):
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def np64(t):
    return None if t is None else t.detach().cpu().double().numpy()


def normwise(got, ref):
    """max |got - ref| / max |ref| (normwise relative error)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    if den == 0.0:
        return float(np.max(np.abs(got))) if got.size else 0.0
    return float(np.max(np.abs(got - ref)) / den)


def half_ulp_bf16(ref):
    """Half a bf16 ulp at each reference value (the output rounding alone)."""
    a = np.abs(np.asarray(ref, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 1e-38)))
    return 0.5 * np.exp2(e - 7)


def bf16_excess(got, ref):
    """max(|got - ref| - half_ulp_bf16(ref)): error beyond the output rounding."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref) - half_ulp_bf16(ref))) if ref.size else 0.0


def oracle_args(inp):
    a = inputs.to_f64(inp)
    return dict(x=a["x"], dt=a["dt"], A=a["A"], B=a["B"], C=a["C"], D=a["D"],
                dt_bias=a["dt_bias"], init=a["init"], dt_softplus=inp["dt_softplus"],
                cu_seqlens=a["cu_seqlens"])


def gpu_fwd(ssd, inp, chunk_size, **kw):
    d = to_dev(inp)
    return ssd.fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], dt_bias=d["dt_bias"],
                   init=d["init"], cu_seqlens=d["cu_seqlens"], chunk_size=chunk_size,
                   dt_softplus=inp["dt_softplus"], **kw)


def gpu_bwd(ssd, inp, chunk_size, **kw):
    d = to_dev(inp)
    return ssd.bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["dout"], D=d["D"],
                   dt_bias=d["dt_bias"], init=d["init"], d_final=d["d_final"],
                   cu_seqlens=d["cu_seqlens"], chunk_size=chunk_size,
                   dt_softplus=inp["dt_softplus"], **kw)


def batch_rows(inp, rows):
    """The inputs of some batch rows alone (each row is an independent problem)."""
    out = dict(inp)
    for k in ("x", "B", "C", "dt", "dout", "init", "d_final"):
        if out.get(k) is not None:
            out[k] = out[k][rows].contiguous()
    return out


def packed_sequences(inp, seqs):
    """The inputs of some packed sequences alone, re-packed into one row (each
    sequence is an independent problem).  Returns (inputs, token index list)."""
    cu = [int(v) for v in inp["cu_seqlens"]]
    toks = [t for s in seqs for t in range(cu[s], cu[s + 1])]
    idx = torch.tensor(toks, dtype=torch.long)
    out = dict(inp)
    for k in ("x", "B", "C", "dt", "dout"):
        if out.get(k) is not None:
            out[k] = out[k][:, idx].contiguous()
    for k in ("init", "d_final"):
        if out.get(k) is not None:
            out[k] = out[k][list(seqs)].contiguous()
    lens = [cu[s + 1] - cu[s] for s in seqs]
    out["cu_seqlens"] = inputs.cu_from_lengths(lens)
    return out, toks


def bf16_kernels(io, headdim, dstate):
    """Whether a problem runs on the bf16 matrix-core kernels (the rest run on the
    fp32 ones): they store C.B^T in fragment order (include/ssd.h)."""
    return io == "bf16" and headdim >= 32 and dstate >= 32


def cb_rows(cb, Q):
    """C.B^T (..., Q, Q) in fragment order -> row-major (a tensor or an array)."""
    lead = tuple(cb.shape[:-2])
    f = cb.reshape(lead + (Q // 16, Q // 32, 4, 16, 8))  # (R, S, q, r, e) = [16R + r][32S + 8q + e]
    n = len(lead)
    perm = tuple(range(n)) + (n, n + 3, n + 1, n + 2, n + 4)  # -> (R, r, S, q, e)
    f = f.permute(perm) if hasattr(f, "permute") else f.transpose(perm)
    return f.reshape(lead + (Q, Q))


def cb_frag(cb, Q):
    """Row-major C.B^T (..., Q, Q) -> fragment order (the inverse of cb_rows)."""
    lead = tuple(cb.shape[:-2])
    f = cb.reshape(lead + (Q // 16, 16, Q // 32, 4, 8))  # (R, r, S, q, e)
    n = len(lead)
    perm = tuple(range(n)) + (n, n + 2, n + 3, n + 1, n + 4)  # -> (R, S, q, r, e)
    f = f.permute(perm) if hasattr(f, "permute") else f.transpose(perm)
    return f.reshape(lead + (Q, Q))

