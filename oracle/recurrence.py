"""Token-by-token fp64 recurrence: the SSD oracle (test infrastructure only).

What it computes (gigipick.blogspot.com "LLM Mamba ...", section 1: the
selective SSM is a linear recurrence in which h_t needs h_{t-1} and the decay
and input matrices change with the input; the printed equation was lost, so
the Mamba-2 form is used).  Per sequence and head h, with state S = h^T of
shape (headdim P, dstate N) and group g = h // (nheads // ngroups):

    z_t     = dt[t, h] + dt_bias[h]                (dt_bias absent -> 0)
    delta_t = softplus(z_t) if dt_softplus else z_t
    a_t     = exp(delta_t * A[h])
    S_t     = a_t * S_{t-1} + delta_t * x_t B_t^T  (x_t: P-vector, B_t: N-vector)
    y_t     = S_t C_t + D[h] * x_t                 (D absent -> 0)
    S_{-1}  = init (zeros when absent);  final = S after the last token.

The chunked form reaches exactly this result up to rounding order, so the
oracle is this plain definition, written one token at a time.  All
arithmetic is float64; inputs are converted exactly (bf16 and fp32 values are
representable in fp64).

Layout (dense, last index fastest):
    x, y, dout     (batch, seqlen, nheads, headdim)
    dt, ddt        (batch, seqlen, nheads)
    B, C, dB, dC   (batch, seqlen, ngroups, dstate)
    A, D, dt_bias  (nheads,)
    init, final    (nseq, nheads, headdim, dstate); nseq = batch, or the number
                   of packed sequences when ``cu_seqlens`` is given (batch 1).

Packed sequences (``cu_seqlens``): sequence s covers tokens
[cu_seqlens[s], cu_seqlens[s+1]) of the single batch row; the state starts
from init[s] at its first token and nothing crosses a boundary.

The backward is the adjoint of the same loop (reverse-mode differentiation of
the recurrence written out by hand), with the state re-computed segment by
segment from checkpoints so memory stays bounded.
"""
import numpy as np


def softplus(z):
    """softplus(z) = log(1 + e^z), evaluated as max(z, 0) + log1p(e^-|z|)."""
    z = np.asarray(z, dtype=np.float64)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def sigmoid(z):
    """Logistic function, d softplus / dz, in a form that never overflows."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def effective_dt(dt, dt_bias=None, dt_softplus=False):
    """Return (delta, z): z = dt + dt_bias, delta = softplus(z) or z."""
    z = np.asarray(dt, dtype=np.float64)
    if dt_bias is not None:
        z = z + np.asarray(dt_bias, dtype=np.float64)
    delta = softplus(z) if dt_softplus else z
    return delta, z


def sequences(batch, seqlen, cu_seqlens=None):
    """List of (seq index, batch row, first token, end token)."""
    if cu_seqlens is None:
        return [(b, b, 0, seqlen) for b in range(batch)]
    cu = [int(v) for v in np.asarray(cu_seqlens).reshape(-1)]
    if batch != 1:
        raise ValueError("packed sequences need batch == 1")
    if cu[0] != 0 or cu[-1] != seqlen or any(cu[i] > cu[i + 1] for i in range(len(cu) - 1)):
        raise ValueError("cu_seqlens must rise from 0 to seqlen")
    return [(s, 0, cu[s], cu[s + 1]) for s in range(len(cu) - 1)]


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def _prep(x, dt, A, B, C, D, dt_bias, dt_softplus, heads):
    x, A, B, C, D = _f64(x), _f64(A), _f64(B), _f64(C), _f64(D)
    nbatch, seqlen, nheads, headdim = x.shape
    ngroups, dstate = B.shape[2], B.shape[3]
    if nheads % ngroups:
        raise ValueError("nheads must be a multiple of ngroups")
    heads = np.arange(nheads) if heads is None else np.asarray(heads, dtype=np.int64)
    group_of = heads // (nheads // ngroups)
    delta, z = effective_dt(dt, dt_bias, dt_softplus)
    return x, A, B, C, D, delta, z, heads, group_of


def fwd(x, dt, A, B, C, D=None, dt_bias=None, init=None, dt_softplus=False,
        cu_seqlens=None, heads=None):
    """Forward recurrence.  Returns (y, final) in float64.

    ``heads`` (optional) restricts the computation to those head indices; the
    returned arrays then carry only those heads, in the given order.
    """
    x, A, B, C, D, delta, z, heads, group_of = _prep(x, dt, A, B, C, D, dt_bias,
                                                     dt_softplus, heads)
    nbatch, seqlen, _, headdim = x.shape
    dstate = B.shape[3]
    nh = len(heads)
    seqs = sequences(nbatch, seqlen, cu_seqlens)
    y = np.zeros((nbatch, seqlen, nh, headdim))
    final = np.zeros((len(seqs), nh, headdim, dstate))
    Ah = A[heads]
    Dh = np.zeros(nh) if D is None else D[heads]
    for s, b, t0, t1 in seqs:
        S = np.zeros((nh, headdim, dstate)) if init is None else _f64(init)[s][heads].copy()
        for t in range(t0, t1):
            d = delta[b, t, heads]
            a = np.exp(d * Ah)
            xt = x[b, t, heads]
            Bt = B[b, t, group_of]
            Ct = C[b, t, group_of]
            S = a[:, None, None] * S + (d[:, None] * xt)[:, :, None] * Bt[:, None, :]
            y[b, t] = np.einsum("hpn,hn->hp", S, Ct) + Dh[:, None] * xt
        final[s] = S
    return y, final


def bwd(x, dt, A, B, C, dout, D=None, dt_bias=None, init=None, d_final=None,
        dt_softplus=False, cu_seqlens=None, heads=None, checkpoint=256):
    """Adjoint of ``fwd``.  Returns a dict of float64 gradients.

    Keys: dx, ddt (w.r.t. the raw dt input), dA, dB, dC, dD (None when D is
    None), d_dt_bias, d_init.  With ``heads`` given, dB and dC hold only the
    contributions of those heads, and per-head outputs carry only those heads.
    Also dA_abs, per head the sum of the absolute values of the terms that dA
    sums: a diagnostic, not a gradient.  dA is a sum over tokens whose terms
    can cancel to a small fraction of their size; the error of a computed sum
    is naturally measured against the sum of its terms' magnitudes.

    Let G_t = dL/dS_t (total).  Walking tokens backwards:
        G_t   = dy_t C_t^T + a_{t+1} G_{t+1}    (G_last adds d_final)
        dx_t  = delta_t G_t B_t + D dy_t
        dB_t += delta_t G_t^T x_t               (summed over the group's heads)
        dC_t += S_t^T dy_t
        ddelta_t = x_t^T G_t B_t + A a_t <G_t, S_{t-1}>
        dA   += delta_t a_t <G_t, S_{t-1}>
        dD   += dy_t . x_t
        d_init = a_first G_first
        ddt  = ddelta * sigmoid(z) if dt_softplus else ddelta;  d_dt_bias = sum ddt
    """
    x, A, B, C, D, delta, z, heads, group_of = _prep(x, dt, A, B, C, D, dt_bias,
                                                     dt_softplus, heads)
    dout = _f64(dout)
    nbatch, seqlen, _, headdim = x.shape
    ngroups, dstate = B.shape[2], B.shape[3]
    nh = len(heads)
    seqs = sequences(nbatch, seqlen, cu_seqlens)
    Ah = A[heads]
    Dh = np.zeros(nh) if D is None else D[heads]
    dx = np.zeros((nbatch, seqlen, nh, headdim))
    ddelta = np.zeros((nbatch, seqlen, nh))
    dB = np.zeros_like(B)
    dC = np.zeros_like(C)
    dA = np.zeros(nh)
    dA_abs = np.zeros(nh)
    dD = np.zeros(nh)
    d_init = np.zeros((len(seqs), nh, headdim, dstate))
    onehot = np.zeros((nh, ngroups))
    onehot[np.arange(nh), group_of] = 1.0  # sums per-head terms into their group

    for s, b, t0, t1 in seqs:
        S0 = np.zeros((nh, headdim, dstate)) if init is None else _f64(init)[s][heads].copy()
        # forward sweep: checkpoint the state entering every segment
        starts = list(range(t0, t1, checkpoint))
        ckpt = {}
        S = S0
        for t in range(t0, t1):
            if (t - t0) % checkpoint == 0:
                ckpt[t] = S
            d = delta[b, t, heads]
            S = np.exp(d * Ah)[:, None, None] * S + \
                (d[:, None] * x[b, t, heads])[:, :, None] * B[b, t, group_of][:, None, :]
        G = np.zeros((nh, headdim, dstate)) if d_final is None else _f64(d_final)[s][heads].copy()
        for seg0 in reversed(starts):
            seg1 = min(seg0 + checkpoint, t1)
            # re-run the segment forward with the same arithmetic as above
            before, after, decay = [], [], []
            S = ckpt[seg0]
            for t in range(seg0, seg1):
                d = delta[b, t, heads]
                a = np.exp(d * Ah)
                before.append(S)
                S = a[:, None, None] * S + \
                    (d[:, None] * x[b, t, heads])[:, :, None] * B[b, t, group_of][:, None, :]
                after.append(S)
                decay.append(a)
            for k in range(seg1 - seg0 - 1, -1, -1):
                t = seg0 + k
                d = delta[b, t, heads]
                a = decay[k]
                xt = x[b, t, heads]
                dyt = dout[b, t, heads]
                Bt = B[b, t, group_of]
                Ct = C[b, t, group_of]
                G = G + dyt[:, :, None] * Ct[:, None, :]
                GB = np.einsum("hpn,hn->hp", G, Bt)
                dx[b, t] = d[:, None] * GB + Dh[:, None] * dyt
                dB[b, t] += onehot.T @ (d[:, None] * np.einsum("hpn,hp->hn", G, xt))
                dC[b, t] += onehot.T @ np.einsum("hpn,hp->hn", after[k], dyt)
                gs = np.einsum("hpn,hpn->h", G, before[k])
                ddelta[b, t] = np.einsum("hp,hp->h", xt, GB) + Ah * a * gs
                dA += d * a * gs
                dA_abs += np.abs(d * a * gs)
                dD += np.einsum("hp,hp->h", dyt, xt)
                G = a[:, None, None] * G
        d_init[s] = G
    ddt = ddelta * sigmoid(z[:, :, heads]) if dt_softplus else ddelta
    return {
        "dx": dx, "ddt": ddt, "dA": dA, "dB": dB, "dC": dC,
        "dD": None if D is None else dD,
        "d_dt_bias": ddt.sum(axis=(0, 1)), "d_init": d_init, "dA_abs": dA_abs,
    }
