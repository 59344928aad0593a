"""Pins for oracle.scan: the combine is associative and every host scan equals
the sequential fold (scan page, section 2, and its Hillis-Steele pseudo-code)."""
import numpy as np
import pytest

from oracle import scan


def _rand_elem(rng, shape, zero=False):
    a = 0.0 if zero else float(rng.uniform(1e-3, 1.0))
    return (a, rng.standard_normal(shape))


def _close(e1, e2, tol=1e-14):
    a1, b1 = e1
    a2, b2 = e2
    scale = max(1.0, float(np.max(np.abs(b2))))
    return abs(a1 - a2) <= tol * max(1.0, abs(a2)) and np.max(np.abs(b1 - b2)) <= tol * scale


@pytest.mark.parametrize("zero_mask", [0, 1, 2, 4, 7])
def test_combine_associative(zero_mask):
    rng = np.random.default_rng(zero_mask)
    for _ in range(200):
        e = [_rand_elem(rng, (3, 5), zero=bool(zero_mask >> i & 1)) for i in range(3)]
        left = scan.combine(scan.combine(e[0], e[1]), e[2])
        right = scan.combine(e[0], scan.combine(e[1], e[2]))
        assert _close(left, right)


def test_combine_is_affine_composition():
    # (a1,b1)(+)(a2,b2) must equal applying S -> a1 S + b1, then S -> a2 S + b2.
    rng = np.random.default_rng(1)
    for _ in range(50):
        e1, e2 = _rand_elem(rng, (4,)), _rand_elem(rng, (4,))
        S = rng.standard_normal(4)
        a, b = scan.combine(e1, e2)
        assert np.allclose(a * S + b, e2[0] * (e1[0] * S + e1[1]) + e2[1], rtol=1e-14, atol=1e-14)


def test_combine_not_commutative():
    # A mistake that swaps operands must be caught: the operator is order-sensitive.
    e1, e2 = (0.5, np.array([1.0])), (0.25, np.array([2.0]))
    assert not _close(scan.combine(e1, e2), scan.combine(e2, e1))


def test_log_combine_matches_linear():
    rng = np.random.default_rng(2)
    for _ in range(100):
        (a1, b1), (a2, b2) = _rand_elem(rng, (3,)), _rand_elem(rng, (3,))
        l, b = scan.combine_log((np.log(a1), b1), (np.log(a2), b2))
        a_ref, b_ref = scan.combine((a1, b1), (a2, b2))
        assert abs(np.exp(l) - a_ref) < 1e-14 and np.allclose(b, b_ref, rtol=1e-13, atol=1e-14)


def test_identity():
    rng = np.random.default_rng(3)
    e = _rand_elem(rng, (2, 2))
    i = scan.identity_like(e[1])
    assert _close(scan.combine(i, e), e) and _close(scan.combine(e, i), e)


@pytest.mark.parametrize("n", list(range(1, 34)) + [63, 64, 65, 127, 128, 129, 130])
def test_parallel_scans_equal_fold(n):
    rng = np.random.default_rng(100 + n)
    elems = [_rand_elem(rng, (2, 3), zero=(rng.uniform() < 0.05)) for _ in range(n)]
    ref = scan.fold(elems)
    hs = scan.hillis_steele(elems)
    bl = scan.blelloch(elems, scan.identity_like(elems[0][1]))
    assert len(hs) == len(bl) == n
    for r, h, b in zip(ref, hs, bl):
        assert _close(h, r, 1e-13) and _close(b, r, 1e-13)


def test_inplace_hillis_steele_races():
    # The pseudo-code's in-place update, run in the natural ascending order
    # without double buffering, reads values already overwritten in the same
    # step; show that this differs from the fold, which is why the oracle and
    # the kernels double-buffer (or read into registers, sync, then write).
    rng = np.random.default_rng(5)
    elems = [_rand_elem(rng, (1,)) for _ in range(8)]
    V = list(elems)
    d = 1
    while d < len(V):
        for i in range(d, len(V)):
            V[i] = scan.combine(V[i - d], V[i])
        d *= 2
    ref = scan.fold(elems)
    assert not all(_close(v, r, 1e-12) for v, r in zip(V, ref))


def test_fold_gives_recurrence_states():
    # The inclusive prefix of (a_t, delta_t x_t B_t^T) from the identity is the
    # state S_t of S_t = a_t S_{t-1} + delta_t x_t B_t^T with S_{-1} = 0.
    rng = np.random.default_rng(6)
    L, P, N = 20, 3, 4
    a = rng.uniform(0.3, 1.0, L)
    u = rng.standard_normal((L, P, N))
    pref = scan.fold(list(zip(a, u)))
    S = np.zeros((P, N))
    for t in range(L):
        S = a[t] * S + u[t]
        assert np.allclose(pref[t][1], S, rtol=1e-13, atol=1e-14)
        assert abs(pref[t][0] - np.prod(a[:t + 1])) < 1e-14
