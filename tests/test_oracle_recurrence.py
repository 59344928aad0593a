"""Pins for the forward oracle (oracle.recurrence.fwd and oracle.chunked.fwd).

Nothing here re-types the oracle: closed forms (geometric series), a textbook
IIR filter (scipy.signal.lfilter), an O(L^2) brute-force sum, a hand-worked
golden example, and invariants that hold for the recurrence whatever its
implementation (causality, linearity, chunk-size invariance, resume, packing).
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.signal import lfilter

from oracle import chunked, recurrence

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_problem(rng, batch=1, L=37, H=4, P=3, N=5, G=2, init=True, D=True, softplus=True):
    x = rng.standard_normal((batch, L, H, P))
    B = rng.standard_normal((batch, L, G, N)) / math.sqrt(N)
    C = rng.standard_normal((batch, L, G, N)) / math.sqrt(N)
    dt = rng.standard_normal((batch, L, H))
    bias = rng.uniform(-4, -2, H) if softplus else None
    if not softplus:
        dt = np.log1p(np.exp(dt - 2.0))
    A = -np.exp(rng.uniform(0, math.log(16), H))
    Dv = rng.standard_normal(H) if D else None
    init_s = 0.3 * rng.standard_normal((batch, H, P, N)) if init else None
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=Dv, dt_bias=bias, init=init_s, dt_softplus=softplus)


def test_softplus_matches_definition():
    z = np.concatenate([np.linspace(-40, 40, 801), [-700.0, 0.0, 700.0]])
    ref = np.array([math.log1p(math.exp(v)) if v < 30 else v + math.log1p(math.exp(-v)) for v in z])
    assert np.allclose(recurrence.softplus(z), ref, rtol=1e-15, atol=1e-300)
    s = recurrence.sigmoid(z)
    ref_s = np.array([1.0 / (1.0 + math.exp(-v)) if v > -700 else 0.0 for v in z])
    assert np.allclose(s, ref_s, rtol=1e-14, atol=1e-300)


@pytest.mark.parametrize("A", [-1.7, -0.05, 0.0])
@pytest.mark.parametrize("softplus", [False, True])
def test_closed_form_constant_inputs(A, softplus):
    # Constant delta, x, B, C and scalar A: the state is a geometric series,
    #   S_t = a^{t+1} S0 + delta x B^T (1 - a^{t+1}) / (1 - a),   a = e^{delta A},
    # and S_t = S0 + (t+1) delta x B^T when A = 0 (a = 1).
    L, P, N = 50, 3, 4
    rng = np.random.default_rng(7)
    xv, Bv, Cv = rng.standard_normal(P), rng.standard_normal(N), rng.standard_normal(N)
    S0 = rng.standard_normal((P, N))
    Dv = 0.7
    z = -1.3
    delta = math.log1p(math.exp(z)) if softplus else 0.4
    dtv = z if softplus else delta
    x = np.broadcast_to(xv, (1, L, 1, P)).copy()
    B = np.broadcast_to(Bv, (1, L, 1, N)).copy()
    C = np.broadcast_to(Cv, (1, L, 1, N)).copy()
    dt = np.full((1, L, 1), dtv)
    y, final = recurrence.fwd(x, dt, np.array([A]), B, C, D=np.array([Dv]),
                              init=S0[None, None], dt_softplus=softplus)
    a = math.exp(delta * A)
    for t in range(L):
        if A == 0.0:
            S = S0 + (t + 1) * delta * np.outer(xv, Bv)
        else:
            S = a ** (t + 1) * S0 + delta * np.outer(xv, Bv) * (1 - a ** (t + 1)) / (1 - a)
        assert np.allclose(y[0, t, 0], S @ Cv + Dv * xv, rtol=1e-12, atol=1e-12)
    assert np.allclose(final[0, 0], S, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("A", [-2.5, -0.1])
def test_scalar_lti_equals_lfilter(A):
    # P = N = 1 with constant delta, B, C: the scan is the first-order IIR filter
    # y = (delta B C) x + a y[-1], i.e. lfilter([delta B C], [1, -a]) plus D x;
    # the initial state enters as the filter state zi = a C S0.
    rng = np.random.default_rng(8)
    L = 200
    delta, Bv, Cv, Dv, S0 = 0.3, 0.8, -1.1, 0.25, 0.6
    xs = rng.standard_normal(L)
    a = math.exp(delta * A)
    ref, _ = lfilter([delta * Bv * Cv], [1.0, -a], xs, zi=[a * Cv * S0])
    ref = ref + Dv * xs
    y, final = recurrence.fwd(xs.reshape(1, L, 1, 1), np.full((1, L, 1), delta), np.array([A]),
                              np.full((1, L, 1, 1), Bv), np.full((1, L, 1, 1), Cv),
                              D=np.array([Dv]), init=np.full((1, 1, 1, 1), S0))
    assert np.allclose(y[0, :, 0, 0], ref, rtol=1e-12, atol=1e-12)


def test_scalar_time_varying_brute_force():
    # y_t = sum_{s<=t} C_t (prod_{r=s+1..t} a_r) delta_s B_s x_s
    #       + C_t (prod_{r<=t} a_r) S0 + D x_t          (O(L^2) sum, no recursion)
    rng = np.random.default_rng(9)
    L = 60
    x = rng.standard_normal(L)
    Bv, Cv = rng.standard_normal(L), rng.standard_normal(L)
    dt = rng.standard_normal(L)
    bias, A, Dv, S0 = -2.5, -3.0, 0.4, 0.9
    delta = np.log1p(np.exp(dt + bias))
    a = np.exp(delta * A)
    ref = np.zeros(L)
    for t in range(L):
        acc = Cv[t] * np.prod(a[:t + 1]) * S0 + Dv * x[t]
        for s in range(t + 1):
            acc += Cv[t] * np.prod(a[s + 1:t + 1]) * delta[s] * Bv[s] * x[s]
        ref[t] = acc
    y, _ = recurrence.fwd(x.reshape(1, L, 1, 1), dt.reshape(1, L, 1), np.array([A]),
                          Bv.reshape(1, L, 1, 1), Cv.reshape(1, L, 1, 1), D=np.array([Dv]),
                          dt_bias=np.array([bias]), init=np.full((1, 1, 1, 1), S0),
                          dt_softplus=True)
    assert np.allclose(y[0, :, 0, 0], ref, rtol=1e-12, atol=1e-13)


def test_golden_hand_worked():
    # tests/golden/recurrence_hand.json: a 4-token, 2-head example worked by hand
    # from the recurrence's definition (decays chosen as 1 and 1/2 so that the
    # arithmetic is exact in binary fractions).
    with open(os.path.join(GOLDEN, "recurrence_hand.json")) as f:
        g = json.load(f)
    arr = {k: np.array(v, dtype=np.float64) for k, v in g["inputs"].items()}
    y, final = recurrence.fwd(arr["x"], arr["dt"], arr["A"], arr["B"], arr["C"], D=arr["D"],
                              init=arr["init"], dt_softplus=False)
    assert np.allclose(y, np.array(g["expected"]["y"]), rtol=1e-14, atol=1e-14)
    assert np.allclose(final, np.array(g["expected"]["final"]), rtol=1e-14, atol=1e-14)
    yc, fc, _ = chunked.fwd(arr["x"], arr["dt"], arr["A"], arr["B"], arr["C"], D=arr["D"],
                            init=arr["init"], dt_softplus=False, chunk_size=3)
    assert np.allclose(yc, np.array(g["expected"]["y"]), rtol=1e-14, atol=1e-14)
    assert np.allclose(fc, np.array(g["expected"]["final"]), rtol=1e-14, atol=1e-14)


def test_group_mapping_contiguous():
    # Head h reads group h // (H/G): changing group 1's B must leave heads 0, 1
    # (group 0) untouched and move heads 2, 3.
    rng = np.random.default_rng(10)
    p = rand_problem(rng, H=4, G=2)
    y0, _ = recurrence.fwd(**p)
    p2 = dict(p)
    p2["B"] = p["B"].copy()
    p2["B"][:, :, 1] += 1.0
    y1, _ = recurrence.fwd(**p2)
    assert np.array_equal(y0[:, :, :2], y1[:, :, :2])
    assert not np.allclose(y0[:, :, 2:], y1[:, :, 2:])


@pytest.mark.parametrize("Q", [1, 2, 7, 16, 64, 37])
def test_chunked_equals_sequential(Q):
    rng = np.random.default_rng(11 + Q)
    p = rand_problem(rng, batch=2, L=37)
    y_ref, f_ref = recurrence.fwd(**p)
    y, f, mid = chunked.fwd(**p, chunk_size=Q)
    assert np.allclose(y, y_ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(f, f_ref, rtol=1e-12, atol=1e-12)


def test_chunked_no_init_no_D_direct_dt():
    rng = np.random.default_rng(12)
    p = rand_problem(rng, L=40, init=False, D=False, softplus=False)
    y_ref, f_ref = recurrence.fwd(**p)
    y, f, _ = chunked.fwd(**p, chunk_size=16)
    assert np.allclose(y, y_ref, rtol=1e-12, atol=1e-12) and np.allclose(f, f_ref, rtol=1e-12, atol=1e-12)


def test_chunk_states_are_zero_init_states():
    # T_c is the state a chunk reaches from a zero state; H_c the state entering it.
    rng = np.random.default_rng(13)
    p = rand_problem(rng, L=30)
    _, _, mid = chunked.fwd(**p, chunk_size=8)
    for k, ch in enumerate(mid["chunks"]):
        s, n = ch["start"], ch["len"]
        sub = {kk: (v[:, s:s + n] if kk in ("x", "dt", "B", "C") else v) for kk, v in p.items()}
        sub["init"] = None
        _, fT = recurrence.fwd(**sub)
        assert np.allclose(mid["T"][k], fT[0], rtol=1e-12, atol=1e-13)
        _, fH = recurrence.fwd(**{kk: (v[:, :s] if kk in ("x", "dt", "B", "C") else v)
                                  for kk, v in p.items()}) if s > 0 else (None, p["init"])
        assert np.allclose(mid["Hin"][k], fH[0], rtol=1e-12, atol=1e-13)


def test_causality():
    rng = np.random.default_rng(14)
    p = rand_problem(rng, L=30)
    y0, _ = recurrence.fwd(**p)
    t = 17
    p2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
    p2["x"][:, t + 1:] += rng.standard_normal(p2["x"][:, t + 1:].shape)
    p2["B"][:, t + 1:] += 1.0
    p2["dt"][:, t + 1:] -= 1.0
    y1, _ = recurrence.fwd(**p2)
    assert np.array_equal(y0[:, :t + 1], y1[:, :t + 1])
    assert not np.allclose(y0[:, t + 1:], y1[:, t + 1:])


def test_linearity_in_x_and_init():
    rng = np.random.default_rng(15)
    p = rand_problem(rng, L=25)
    q = dict(p)
    q["x"] = rng.standard_normal(p["x"].shape)
    q["init"] = rng.standard_normal(p["init"].shape)
    r = dict(p)
    r["x"] = 2.0 * p["x"] - 3.0 * q["x"]
    r["init"] = 2.0 * p["init"] - 3.0 * q["init"]
    yp, fp = recurrence.fwd(**p)
    yq, fq = recurrence.fwd(**q)
    yr, fr = recurrence.fwd(**r)
    assert np.allclose(yr, 2 * yp - 3 * yq, rtol=1e-11, atol=1e-11)
    assert np.allclose(fr, 2 * fp - 3 * fq, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("split", [8, 13, 1])
def test_resume_split(split):
    rng = np.random.default_rng(16)
    p = rand_problem(rng, L=32)
    y, f = recurrence.fwd(**p)
    a = {k: (v[:, :split] if k in ("x", "dt", "B", "C") else v) for k, v in p.items()}
    b = {k: (v[:, split:] if k in ("x", "dt", "B", "C") else v) for k, v in p.items()}
    ya, fa = recurrence.fwd(**a)
    b["init"] = fa
    yb, fb = recurrence.fwd(**b)
    assert np.allclose(np.concatenate([ya, yb], axis=1), y, rtol=1e-12, atol=1e-12)
    assert np.allclose(fb, f, rtol=1e-12, atol=1e-12)


def test_packed_equals_separate():
    rng = np.random.default_rng(17)
    lengths = [5, 0, 19, 1, 12]
    L = sum(lengths)
    p = rand_problem(rng, L=L)
    p["init"] = 0.3 * rng.standard_normal((len(lengths), 4, 3, 5))
    cu = np.cumsum([0] + lengths)
    y, f = recurrence.fwd(**p, cu_seqlens=cu)
    yc, fc, _ = chunked.fwd(**p, cu_seqlens=cu, chunk_size=4)
    assert np.allclose(yc, y, rtol=1e-12, atol=1e-12) and np.allclose(fc, f, rtol=1e-12, atol=1e-12)
    for s in range(len(lengths)):
        sl = slice(cu[s], cu[s + 1])
        q = {k: (v[:, sl] if k in ("x", "dt", "B", "C") else v) for k, v in p.items()}
        q["init"] = p["init"][s:s + 1]
        ys, fs = recurrence.fwd(**q)
        assert np.allclose(y[:, sl], ys, rtol=1e-12, atol=1e-12)
        assert np.allclose(f[s], fs[0], rtol=1e-12, atol=1e-12)
    # an empty sequence passes its init through unchanged
    assert np.array_equal(f[1], p["init"][1])


def test_head_subset_matches_full():
    rng = np.random.default_rng(18)
    p = rand_problem(rng, L=20, H=4, G=2)
    y, f = recurrence.fwd(**p)
    ys, fs = recurrence.fwd(**p, heads=[3, 1])
    assert np.array_equal(ys, y[:, :, [3, 1]]) and np.array_equal(fs, f[:, [3, 1]])
