"""Gated RMSNorm of the Mamba-2 layer, forward and backward: fp64 oracle (test
infrastructure only; the GPU path shares no code with it).

What it computes.  The aitrends.kr/articles/109906 page ("B200에 맞춘 Helion
Mamba-2 커널 최적화", its key-figures list and results section) names the
layer's normalisation backward kernel, _layer_norm_bwd, as the largest single
gain (one B200, batch 2, seqlen 8192, bf16) but prints no formula.  The plainest reading, the Mamba-2 layer's
gated RMSNorm applied to the SSD output y with the gate z (normalised after
gating), is taken here.  Per row t (a token) of D columns, split into groups of
`group` consecutive columns, and per column i with group g(i):

    s_i    = z_i * sigmoid(z_i)                 (silu; s = 1 when there is no gate)
    v_i    = y_i * s_i
    r_g    = 1 / sqrt(mean_{j in g} v_j^2 + eps)
    out_i  = v_i * r_g(i) * w_i

Backward, for an upstream gradient dout (derived from the definition above):

    c_g    = sum_{j in g} w_j dout_j v_j
    dv_i   = r * w_i dout_i - (r^3 / |g|) c_g(i) v_i
    dy_i   = dv_i s_i
    dz_i   = dv_i y_i sigmoid(z_i) (1 + z_i (1 - sigmoid(z_i)))
    dw_i   = sum_t dout_{t,i} v_{t,i} r_{t,g(i)}

All arithmetic is float64.  Layout: y, z, out, dout, dy, dz (rows, D) with D
fastest; w, dw (D,); r (rows, D // group).
"""
import numpy as np


def sigmoid(z):
    return 0.5 * (1.0 + np.tanh(0.5 * z))  # the logistic function, overflow-free


def fwd(y, z, w, group, eps):
    """Returns (out, r).  z may be None (no gate)."""
    y = np.asarray(y, np.float64)
    rows, D = y.shape
    assert D % group == 0
    s = np.ones_like(y) if z is None else np.asarray(z, np.float64) * sigmoid(np.asarray(z, np.float64))
    v = y * s
    vg = v.reshape(rows, D // group, group)
    r = 1.0 / np.sqrt(np.mean(vg * vg, axis=2) + eps)
    out = (vg * r[:, :, None]).reshape(rows, D) * np.asarray(w, np.float64)[None, :]
    return out, r


def bwd(dout, y, z, w, group, eps):
    """Returns (dy, dz, dw); dz is None without a gate."""
    y = np.asarray(y, np.float64)
    dout = np.asarray(dout, np.float64)
    w = np.asarray(w, np.float64)
    rows, D = y.shape
    ng = D // group
    if z is None:
        s = np.ones_like(y)
    else:
        z = np.asarray(z, np.float64)
        sg = sigmoid(z)
        s = z * sg
    v = y * s
    _, r = fwd(y, z, w, group, eps)
    wd = (w[None, :] * dout).reshape(rows, ng, group)
    vg = v.reshape(rows, ng, group)
    c = np.sum(wd * vg, axis=2)
    dv = (r[:, :, None] * wd - (r ** 3 / group)[:, :, None] * c[:, :, None] * vg).reshape(rows, D)
    dy = dv * s
    dz = None if z is None else dv * y * sg * (1.0 + z * (1.0 - sg))
    dw = np.sum(dout * v * np.repeat(r, group, axis=1), axis=0)
    return dy, dz, dw
