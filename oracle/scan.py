"""Scan element, associative combine and host scans (oracle; test infrastructure).

Follows gigipick.blogspot.com "LLM Mamba ...", section 2: each time step
contributes a pair (decay, input term); pairs are merged by an associative
operator, and the state after step t is the inclusive prefix of the pairs.
The page's formula for the operator was lost in extraction; the reading used
is the composition of affine maps S -> a*S + b applied left to right:

    (a1, b1) (+) (a2, b2) = (a1 * a2,  a2 * b1 + b2)

``a`` is a scalar (one decay per head, Mamba-2), ``b`` an array of any shape.
The page's Hillis-Steele pseudo-code updates V[i] in place after reading
V[i-d]; with one barrier per step that is a read-after-write race, so the
version here is double-buffered (every step reads the previous buffer only).

Log-domain elements (l, b) with l = log(a) use
    (l1, b1) (+) (l2, b2) = (l1 + l2,  exp(l2) * b1 + b2).
"""
import numpy as np


def combine(e1, e2):
    """(a1, b1) (+) (a2, b2) = (a1*a2, a2*b1 + b2): apply e1 first, then e2."""
    a1, b1 = e1
    a2, b2 = e2
    return (a1 * a2, a2 * b1 + b2)


def combine_log(e1, e2):
    """Log-domain combine: (l1 + l2, exp(l2) * b1 + b2)."""
    l1, b1 = e1
    l2, b2 = e2
    return (l1 + l2, np.exp(l2) * b1 + b2)


def identity_like(b):
    """Identity element (1, 0) of ``combine``."""
    return (1.0, np.zeros_like(np.asarray(b, dtype=np.float64)))


def fold(elems, op=combine):
    """Sequential inclusive prefix: out[i] = e0 (+) e1 (+) ... (+) ei."""
    out = []
    acc = None
    for e in elems:
        acc = e if acc is None else op(acc, e)
        out.append(acc)
    return out


def hillis_steele(elems, op=combine):
    """Double-buffered Hillis-Steele inclusive scan (section 2 of the scan page).

    Step d = 1, 2, 4, ...: element i (i >= d) becomes V[i-d] (+) V[i], where both
    operands come from the previous step's buffer.
    """
    cur = list(elems)
    n = len(cur)
    d = 1
    while d < n:
        nxt = list(cur)
        for i in range(d, n):
            nxt[i] = op(cur[i - d], cur[i])
        cur = nxt
        d *= 2
    return cur


def blelloch(elems, identity, op=combine):
    """Work-efficient (Blelloch) scan, returned as an inclusive prefix.

    Up-sweep builds subtree totals; down-sweep turns them into exclusive
    prefixes (parent prefix (+) left-subtree total for the right child).  The
    operator is not commutative, so operand order is kept explicit.
    """
    n = len(elems)
    if n == 0:
        return []
    size = 1
    while size < n:
        size *= 2
    x = list(elems) + [identity] * (size - n)
    d = 1
    while d < size:
        for i in range(2 * d - 1, size, 2 * d):
            x[i] = op(x[i - d], x[i])
        d *= 2
    x[size - 1] = identity
    d = size // 2
    while d >= 1:
        for i in range(2 * d - 1, size, 2 * d):
            left = x[i - d]
            x[i - d] = x[i]
            x[i] = op(x[i], left)
        d //= 2
    # x is now the exclusive scan; make it inclusive.
    return [op(x[i], elems[i]) for i in range(n)]
