"""Pins for the backward oracle (oracle.recurrence.bwd and oracle.chunked.bwd).

The loss is L = <dout, y> + <d_final, final>.  Every gradient is checked by
central finite differences of the forward oracle, and by torch.autograd
(float64, CPU) through a token loop written here independently of the
oracle.  The adjoint identity <dy, J v> = <J^T dy, v> checks the linear part.
"""
import math

import numpy as np
import pytest
import torch

from oracle import chunked, recurrence
from test_oracle_recurrence import rand_problem

GRADS = ["dx", "ddt", "dA", "dB", "dC", "dD", "d_dt_bias", "d_init"]
WRT = {"dx": "x", "ddt": "dt", "dA": "A", "dB": "B", "dC": "C", "dD": "D",
       "d_dt_bias": "dt_bias", "d_init": "init"}


def loss(p, dout, d_final, cu=None):
    y, f = recurrence.fwd(**p, cu_seqlens=cu)
    return float(np.sum(dout * y) + np.sum(d_final * f))


def tiny(seed, softplus=True):
    rng = np.random.default_rng(seed)
    p = rand_problem(rng, batch=1, L=13, H=2, P=3, N=4, G=1, softplus=softplus)
    dout = rng.standard_normal(p["x"].shape)
    d_final = rng.standard_normal(p["init"].shape)
    return p, dout, d_final


@pytest.mark.parametrize("softplus", [True, False])
def test_finite_differences(softplus):
    p, dout, d_final = tiny(20, softplus)
    if not softplus:
        p["dt_bias"] = np.array([0.05, -0.02])   # the bias still enters z = dt + bias
    g = recurrence.bwd(**p, dout=dout, d_final=d_final, checkpoint=5)
    h = 1e-6
    for key in GRADS:
        name = WRT[key]
        base = p[name]
        num = np.zeros_like(base)
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            pp = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
            pp[name][idx] += h
            lp = loss(pp, dout, d_final)
            pp[name][idx] -= 2 * h
            lm = loss(pp, dout, d_final)
            num[idx] = (lp - lm) / (2 * h)
        scale = max(1.0, np.max(np.abs(num)))
        assert np.max(np.abs(g[key] - num)) <= 1e-7 * scale, key


def torch_loop_loss(x, dt, A, B, C, D, bias, init, dout, d_final, softplus):
    """Independent token loop in torch (float64) for autograd."""
    L, H = x.shape[1], x.shape[2]
    G = B.shape[2]
    hpg = H // G
    z = dt + bias
    delta = torch.nn.functional.softplus(z) if softplus else z
    S = init[0]
    total = torch.zeros((), dtype=torch.float64)
    for t in range(L):
        rows = []
        newS = []
        for h in range(H):
            g = h // hpg
            a = torch.exp(delta[0, t, h] * A[h])
            Sh = a * S[h] + delta[0, t, h] * torch.outer(x[0, t, h], B[0, t, g])
            newS.append(Sh)
            rows.append(Sh @ C[0, t, g] + D[h] * x[0, t, h])
        S = torch.stack(newS)
        total = total + torch.sum(dout[0, t] * torch.stack(rows))
    return total + torch.sum(d_final[0] * S)


@pytest.mark.parametrize("softplus", [True, False])
def test_autograd_independent_loop(softplus):
    p, dout, d_final = tiny(21, softplus)
    bias = p["dt_bias"] if p["dt_bias"] is not None else np.array([0.05, -0.02])
    p["dt_bias"] = bias
    t = {k: torch.tensor(p[k], dtype=torch.float64, requires_grad=True)
         for k in ["x", "dt", "A", "B", "C", "D", "dt_bias", "init"]}
    L = torch_loop_loss(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["dt_bias"], t["init"],
                        torch.tensor(dout), torch.tensor(d_final), softplus)
    L.backward()
    g = recurrence.bwd(**p, dout=dout, d_final=d_final)
    for key in GRADS:
        ref = t[WRT[key]].grad.numpy()
        assert np.allclose(g[key], ref, rtol=1e-10, atol=1e-11), key


def test_adjoint_identity():
    # y and final are linear in (x, init) jointly: <dy, y(v, s)> + <df, final(v, s)>
    # equals <dx, v> + <d_init, s> where (dx, d_init) is the adjoint applied to (dy, df).
    rng = np.random.default_rng(22)
    p = rand_problem(rng, batch=2, L=31, H=4, P=3, N=5, G=2)
    dout = rng.standard_normal(p["x"].shape)
    d_final = rng.standard_normal(p["init"].shape)
    g = recurrence.bwd(**p, dout=dout, d_final=d_final, checkpoint=7)
    q = dict(p)
    q["x"] = rng.standard_normal(p["x"].shape)
    q["init"] = rng.standard_normal(p["init"].shape)
    q["D"] = None                                       # D x is linear too, but isolate the scan
    gq = recurrence.bwd(**q, dout=dout, d_final=d_final)
    y, f = recurrence.fwd(**q)
    lhs = np.sum(dout * y) + np.sum(d_final * f)
    rhs = np.sum(gq["dx"] * q["x"]) + np.sum(gq["d_init"] * q["init"])
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))
    assert g["dD"] is not None and gq["dD"] is None


@pytest.mark.parametrize("ck", [1, 4, 256])
def test_checkpoint_interval_invariance(ck):
    p, dout, d_final = tiny(23)
    ref = recurrence.bwd(**p, dout=dout, d_final=d_final, checkpoint=1000)
    g = recurrence.bwd(**p, dout=dout, d_final=d_final, checkpoint=ck)
    for key in GRADS:
        assert np.array_equal(g[key], ref[key]), key


@pytest.mark.parametrize("Q", [1, 3, 8, 64])
def test_chunked_bwd_equals_token_adjoint(Q):
    rng = np.random.default_rng(24 + Q)
    p = rand_problem(rng, batch=2, L=21, H=4, P=3, N=5, G=2)
    dout = rng.standard_normal(p["x"].shape)
    d_final = rng.standard_normal(p["init"].shape)
    ref = recurrence.bwd(**p, dout=dout, d_final=d_final)
    g = chunked.bwd(**p, dout=dout, d_final=d_final, chunk_size=Q)
    for key in GRADS:
        assert np.allclose(g[key], ref[key], rtol=1e-10, atol=1e-11), key


def test_chunked_bwd_packed_and_optional_inputs():
    rng = np.random.default_rng(25)
    lengths = [6, 0, 11, 1, 9]
    p = rand_problem(rng, batch=1, L=sum(lengths), H=4, P=3, N=5, G=2, D=False)
    p["init"] = 0.3 * rng.standard_normal((len(lengths), 4, 3, 5))
    cu = np.cumsum([0] + lengths)
    dout = rng.standard_normal(p["x"].shape)
    for d_final in (None, rng.standard_normal(p["init"].shape)):
        ref = recurrence.bwd(**p, dout=dout, d_final=d_final, cu_seqlens=cu)
        g = chunked.bwd(**p, dout=dout, d_final=d_final, cu_seqlens=cu, chunk_size=4)
        for key in GRADS:
            if key == "dD":
                assert ref[key] is None and g[key] is None
                continue
            assert np.allclose(g[key], ref[key], rtol=1e-10, atol=1e-11), key
        # the empty sequence's d_init is d_final (or zero)
        exp1 = np.zeros((4, 3, 5)) if d_final is None else d_final[1]
        assert np.array_equal(ref["d_init"][1], exp1)


def test_packed_bwd_equals_separate():
    rng = np.random.default_rng(26)
    lengths = [7, 12]
    p = rand_problem(rng, batch=1, L=19, H=2, P=2, N=3, G=1)
    p["init"] = 0.3 * rng.standard_normal((2, 2, 2, 3))
    cu = np.cumsum([0] + lengths)
    dout = rng.standard_normal(p["x"].shape)
    g = recurrence.bwd(**p, dout=dout, cu_seqlens=cu)
    dA = np.zeros(2)
    for s in range(2):
        sl = slice(cu[s], cu[s + 1])
        q = {k: (v[:, sl] if k in ("x", "dt", "B", "C") else v) for k, v in p.items()}
        q["init"] = p["init"][s:s + 1]
        gs = recurrence.bwd(**q, dout=dout[:, sl])
        assert np.allclose(g["dx"][:, sl], gs["dx"], rtol=1e-12, atol=1e-13)
        assert np.allclose(g["d_init"][s], gs["d_init"][0], rtol=1e-12, atol=1e-13)
        dA += gs["dA"]
    assert np.allclose(g["dA"], dA, rtol=1e-12, atol=1e-13)


def test_dA_abs_is_the_sum_of_the_terms_magnitudes():
    """dA_abs (a diagnostic: per head, the sum over tokens of |delta a <G, S_prev>|,
    the terms whose signed sum is dA) equals dA where every term has the same
    sign, exceeds |dA| where they have both signs, and is never below |dA|."""
    rng = np.random.default_rng(31)
    # one head, headdim = dstate = 1, positive inputs and upstream gradient:
    # G_t, S_t, the decays and delta are all positive, so every term is positive
    L = 9
    p = dict(x=rng.uniform(0.5, 1.5, (1, L, 1, 1)), dt=rng.uniform(-1.0, 0.5, (1, L, 1)),
             A=np.array([-0.7]), B=rng.uniform(0.5, 1.5, (1, L, 1, 1)),
             C=rng.uniform(0.5, 1.5, (1, L, 1, 1)), D=None, dt_bias=None,
             init=rng.uniform(0.5, 1.5, (1, 1, 1, 1)), dt_softplus=True)
    dout = rng.uniform(0.5, 1.5, (1, L, 1, 1))
    g = recurrence.bwd(**p, dout=dout)
    assert g["dA"][0] > 0
    assert math.isclose(g["dA_abs"][0], g["dA"][0], rel_tol=1e-12)
    # the upstream gradient alternating in sign: terms of both signs
    dalt = dout * np.array([1.0, -1.0] * L)[:L, None, None][None]
    g2 = recurrence.bwd(**p, dout=dalt)
    assert g2["dA_abs"][0] > abs(g2["dA"][0]) * (1 + 1e-6)
    # any problem: the triangle inequality, per head
    q, dq, dfq = tiny(32)
    g3 = recurrence.bwd(**q, dout=dq, d_final=dfq)
    assert np.all(g3["dA_abs"] >= np.abs(g3["dA"]) * (1 - 1e-12))
