"""Four-stage chunked SSD in fp64 (oracle; test infrastructure only).

This is the chunked form of the recurrence in ``oracle.recurrence``: it must
give the same result up to rounding order, and ``tests/test_oracle_*.py``
pins it against the token loop.  It exists for two reasons: to check the
chunked equations (and their backward) before any kernel uses them, and to
give per-stage intermediates that single GPU stages can be compared with.

Chunking follows gigipick.blogspot.com "LLM Mamba ...", section 3 (memory
hierarchy): the sequence is cut into chunks and the final (carry-out) state of
each chunk is passed on as the initial (carry-in) state of the next.  The
cross-chunk pass is the sequential state-passing loop that
aitrends.kr/articles/109906 ("Helion-based B200 kernel redesign") turns into an
associative scan; here it stays the plain loop (the definition).

Notation per sequence, head h (group g), chunk c holding positions i, j in
[0, len_c):
    delta_j, dA_j = delta_j * A[h], acs_i = sum_{t<=i} dA_t  (natural log)
    L_ij  = exp(acs_i - acs_j) for i >= j, else 0;  w_j = exp(acs_last - acs_j)
    CB_ij = C_i . B_j;  alpha_c = exp(acs_last)
    T_c   = sum_j w_j delta_j x_j B_j^T                      (chunk state, P x N)
    E_c   = alpha_c H_c + T_c,  H_{c+1} = E_c,  H_first = init,  final = E_last
    y_i   = sum_{j<=i} CB_ij L_ij delta_j x_j + exp(acs_i) H_c C_i + D x_i

Chunks are enumerated flat: batch rows (or packed sequences) in order, each
cut from its own first token; the last chunk of a sequence may be partial.
Per-chunk arrays are padded with zeros past the chunk's length.
"""
import numpy as np

from .recurrence import effective_dt, sequences, sigmoid, _f64


def chunk_list(batch, seqlen, chunk_size, cu_seqlens=None):
    """Flat chunk list: dicts with seq, row, start, len, first, last."""
    out = []
    for s, b, t0, t1 in sequences(batch, seqlen, cu_seqlens):
        starts = list(range(t0, t1, chunk_size))
        for k, c0 in enumerate(starts):
            out.append(dict(seq=s, row=b, start=c0, len=min(chunk_size, t1 - c0),
                            first=(k == 0), last=(k == len(starts) - 1)))
    return out


def chunk_cumsum(dt, A, chunks, chunk_size, dt_bias=None, dt_softplus=False):
    """Stage 1: delta and the within-chunk inclusive cumsum of delta*A.

    Returns delta, acs of shape (nchunks, nheads, chunk_size), natural-log units.
    """
    delta, _ = effective_dt(dt, dt_bias, dt_softplus)
    A = _f64(A)
    nheads = delta.shape[2]
    d_out = np.zeros((len(chunks), nheads, chunk_size))
    a_out = np.zeros((len(chunks), nheads, chunk_size))
    for k, ch in enumerate(chunks):
        d = delta[ch["row"], ch["start"]:ch["start"] + ch["len"]].T  # (H, len)
        d_out[k, :, :ch["len"]] = d
        a_out[k, :, :ch["len"]] = np.cumsum(d * A[:, None], axis=1)
    return d_out, a_out


def chunk_state(x, B, delta, acs, chunks):
    """Stage 2: T_c = sum_j w_j delta_j x_j B_j^T, shape (nchunks, H, P, N)."""
    x, B = _f64(x), _f64(B)
    nheads, headdim = x.shape[2], x.shape[3]
    ngroups, dstate = B.shape[2], B.shape[3]
    grp = np.arange(nheads) // (nheads // ngroups)
    T = np.zeros((len(chunks), nheads, headdim, dstate))
    for k, ch in enumerate(chunks):
        n = ch["len"]
        sl = slice(ch["start"], ch["start"] + n)
        xs = x[ch["row"], sl]                      # (n, H, P)
        Bs = B[ch["row"], sl][:, grp]              # (n, H, N)
        w = np.exp(acs[k, :, n - 1:n] - acs[k, :, :n])  # (H, n)
        scale = (w * delta[k, :, :n]).T            # (n, H)
        T[k] = np.einsum("jh,jhp,jhn->hpn", scale, xs, Bs)
    return T


def state_passing(T, acs, chunks, nseq, init=None):
    """Stage 3: sequential state passing over each sequence's chunks.

    Returns Hin (nchunks, H, P, N), the state entering each chunk, and final
    (nseq, H, P, N).  A sequence with no tokens keeps its init as final.
    """
    nchunks, nheads, headdim, dstate = T.shape
    Hin = np.zeros_like(T)
    final = np.zeros((nseq, nheads, headdim, dstate)) if init is None else _f64(init).copy()
    state = None
    for k, ch in enumerate(chunks):
        if ch["first"]:
            state = np.zeros((nheads, headdim, dstate)) if init is None else _f64(init)[ch["seq"]].copy()
        Hin[k] = state
        alpha = np.exp(acs[k, :, ch["len"] - 1])
        state = alpha[:, None, None] * state + T[k]
        if ch["last"]:
            final[ch["seq"]] = state
    return Hin, final


def bmm_chunk(B, C, chunks, chunk_size):
    """Stage 4: CB_ij = C_i . B_j per chunk and group, (nchunks, G, Q, Q)."""
    B, C = _f64(B), _f64(C)
    ngroups = B.shape[2]
    CB = np.zeros((len(chunks), ngroups, chunk_size, chunk_size))
    for k, ch in enumerate(chunks):
        n = ch["len"]
        sl = slice(ch["start"], ch["start"] + n)
        CB[k, :, :n, :n] = np.einsum("ign,jgn->gij", C[ch["row"], sl], B[ch["row"], sl])
    return CB


def decay_matrix(acs_k, n):
    """L_ij = exp(acs_i - acs_j) for i >= j, 0 above the diagonal; (H, n, n)."""
    a = acs_k[:, :n]
    diff = a[:, :, None] - a[:, None, :]
    mask = np.tril(np.ones((n, n), dtype=bool))
    return np.where(mask, np.exp(np.where(mask, diff, 0.0)), 0.0)


def chunk_scan(x, C, CB, delta, acs, Hin, chunks, D=None):
    """Stage 5: y_i = sum_{j<=i} CB_ij L_ij delta_j x_j + exp(acs_i) H_c C_i + D x_i."""
    x, C = _f64(x), _f64(C)
    nbatch, seqlen, nheads, headdim = x.shape
    ngroups = C.shape[2]
    grp = np.arange(nheads) // (nheads // ngroups)
    Dh = np.zeros(nheads) if D is None else _f64(D)
    y = np.zeros_like(x)
    for k, ch in enumerate(chunks):
        n = ch["len"]
        sl = slice(ch["start"], ch["start"] + n)
        xs = x[ch["row"], sl]                         # (n, H, P)
        Cs = C[ch["row"], sl][:, grp]                 # (n, H, N)
        L = decay_matrix(acs[k], n)                   # (H, n, n)
        cb = CB[k][grp][:, :n, :n]                    # (H, n, n)
        intra = np.einsum("hij,hj,jhp->ihp", cb * L, delta[k, :, :n], xs)
        inter = np.exp(acs[k, :, :n]).T[:, :, None] * np.einsum("hpn,ihn->ihp", Hin[k], Cs)
        y[ch["row"], sl] = intra + inter + Dh[None, :, None] * xs
    return y


def fwd(x, dt, A, B, C, D=None, dt_bias=None, init=None, dt_softplus=False,
        cu_seqlens=None, chunk_size=64):
    """Chunked forward.  Returns (y, final, intermediates dict)."""
    nbatch, seqlen = np.shape(x)[0], np.shape(x)[1]
    chunks = chunk_list(nbatch, seqlen, chunk_size, cu_seqlens)
    nseq = len(sequences(nbatch, seqlen, cu_seqlens))
    delta, acs = chunk_cumsum(dt, A, chunks, chunk_size, dt_bias, dt_softplus)
    T = chunk_state(x, B, delta, acs, chunks)
    Hin, final = state_passing(T, acs, chunks, nseq, init)
    CB = bmm_chunk(B, C, chunks, chunk_size)
    y = chunk_scan(x, C, CB, delta, acs, Hin, chunks, D)
    return y, final, dict(chunks=chunks, delta=delta, acs=acs, T=T, Hin=Hin, CB=CB)


def state_passing_bwd(U, acs, chunks, nseq, d_final=None):
    """Reverse state passing: dE_c = dL/dE_c, d_init = dL/dH_first.

    Walking each sequence's chunks backwards from dE_last = d_final (0 when
    absent):  dE_c stored, then the running value becomes alpha_c dE_c + U_c,
    which is dE_{c-1} (= dL/dH_c).  After the first chunk it is d_init.
    """
    nchunks, nheads, headdim, dstate = U.shape
    dE = np.zeros_like(U)
    d_init = np.zeros((nseq, nheads, headdim, dstate)) if d_final is None else _f64(d_final).copy()
    g = None
    for k in range(nchunks - 1, -1, -1):
        ch = chunks[k]
        if ch["last"]:
            g = np.zeros((nheads, headdim, dstate)) if d_final is None else _f64(d_final)[ch["seq"]].copy()
        dE[k] = g
        alpha = np.exp(acs[k, :, ch["len"] - 1])
        g = alpha[:, None, None] * g + U[k]
        if ch["first"]:
            d_init[ch["seq"]] = g
    return dE, d_init


def bwd(x, dt, A, B, C, dout, D=None, dt_bias=None, init=None, d_final=None,
        dt_softplus=False, cu_seqlens=None, chunk_size=64):
    """Chunked backward.  Same gradient keys as ``recurrence.bwd`` plus
    intermediates (U, dE, ddA_last) for stage-level comparison.

    Per chunk and head, with M_ij = (dy_i . x_j) CB_ij L_ij delta_j and
    dCB_ij = (dy_i . x_j) L_ij delta_j (i >= j), dT = dE_c:
        U_c   = sum_i exp(acs_i) dy_i C_i^T
        dx_j  = delta_j sum_i CB_ij L_ij dy_i + w_j delta_j dT B_j + D dy_j
        dC_i += exp(acs_i) H_c^T dy_i + sum_j dCB_ij B_j
        dB_j += sum_i dCB_ij C_i + w_j delta_j dT^T x_j
        ddelta_j(direct) = sum_i (dy_i . x_j) CB_ij L_ij + w_j x_j^T dT B_j
        r_i = exp(acs_i) dy_i^T H_c C_i,  s_j = w_j delta_j x_j^T dT B_j
        ddA_t = sum_{i>=t} r_i + sum_{j<t} s_j + alpha <dE_c, H_c>
                + sum_{i>=t, j<t} M_ij
        ddelta_t = ddelta_t(direct) + A ddA_t;  dA += sum_t delta_t ddA_t
    """
    x, B, C, dout = _f64(x), _f64(B), _f64(C), _f64(dout)
    A = _f64(A)
    nbatch, seqlen, nheads, headdim = x.shape
    ngroups, dstate = B.shape[2], B.shape[3]
    grp = np.arange(nheads) // (nheads // ngroups)
    Dh = np.zeros(nheads) if D is None else _f64(D)
    y, final, mid = fwd(x, dt, A, B, C, D, dt_bias, init, dt_softplus, cu_seqlens, chunk_size)
    chunks, delta, acs, Hin, CB = mid["chunks"], mid["delta"], mid["acs"], mid["Hin"], mid["CB"]
    nseq = len(sequences(nbatch, seqlen, cu_seqlens))
    _, z = effective_dt(dt, dt_bias, dt_softplus)

    U = np.zeros_like(Hin)
    for k, ch in enumerate(chunks):
        n = ch["len"]
        sl = slice(ch["start"], ch["start"] + n)
        e = np.exp(acs[k, :, :n]).T                       # (n, H)
        U[k] = np.einsum("ih,ihp,ihn->hpn", e, dout[ch["row"], sl], C[ch["row"], sl][:, grp])
    dE, d_init = state_passing_bwd(U, acs, chunks, nseq, d_final)

    dx = np.zeros_like(x)
    dB = np.zeros_like(B)
    dC = np.zeros_like(C)
    ddelta = np.zeros((nbatch, seqlen, nheads))
    dA = np.zeros(nheads)
    ddA_last = np.zeros((len(chunks), nheads))
    for k, ch in enumerate(chunks):
        n = ch["len"]
        r0 = ch["row"]
        sl = slice(ch["start"], ch["start"] + n)
        xs, dys = x[r0, sl], dout[r0, sl]                  # (n, H, P)
        Bs, Cs = B[r0, sl][:, grp], C[r0, sl][:, grp]      # (n, H, N)
        d = delta[k, :, :n]                                # (H, n)
        a = acs[k, :, :n]
        L = decay_matrix(acs[k], n)                        # (H, n, n)
        cb = CB[k][grp][:, :n, :n]
        w = np.exp(a[:, n - 1:n] - a)                      # (H, n)
        alpha = np.exp(a[:, n - 1])
        dT = dE[k]
        DX = np.einsum("ihp,jhp->hij", dys, xs)            # dy_i . x_j
        M = DX * cb * L * d[:, None, :]
        dCB = DX * L * d[:, None, :]
        dTB = np.einsum("hpn,jhn->jhp", dT, Bs)             # dT B_j
        dx[r0, sl] = (d.T[:, :, None] * np.einsum("hij,ihp->jhp", cb * L, dys)
                      + (w * d).T[:, :, None] * dTB + Dh[None, :, None] * dys)
        HtDy = np.einsum("hpn,ihp->ihn", Hin[k], dys)      # H_c^T dy_i
        dC_h = np.exp(a).T[:, :, None] * HtDy + np.einsum("hij,jhn->ihn", dCB, Bs)
        dB_h = (np.einsum("hij,ihn->jhn", dCB, Cs)
                + (w * d).T[:, :, None] * np.einsum("hpn,jhp->jhn", dT, xs))
        for g in range(ngroups):
            dC[r0, sl, g] += dC_h[:, grp == g].sum(axis=1)
            dB[r0, sl, g] += dB_h[:, grp == g].sum(axis=1)
        xdTB = np.einsum("jhp,jhp->hj", xs, dTB)            # x_j^T dT B_j
        dd_direct = np.einsum("hij,hij->hj", DX * cb, L) + w * xdTB
        r = np.exp(a) * np.einsum("ihn,ihn->hi", HtDy, Cs)
        s = w * d * xdTB
        ddA_last[k] = alpha * np.einsum("hpn,hpn->h", dT, Hin[k])
        ddA = np.zeros((nheads, n))
        for t in range(n):
            ddA[:, t] = (r[:, t:].sum(axis=1) + s[:, :t].sum(axis=1) + ddA_last[k]
                         + M[:, t:, :t].sum(axis=(1, 2)))
        ddelta[r0, sl] = (dd_direct + A[:, None] * ddA).T
        dA += (d * ddA).sum(axis=1)
    dD = None if D is None else np.einsum("bthp,bthp->h", dout, x)
    ddt = ddelta * sigmoid(z) if dt_softplus else ddelta
    return {
        "dx": dx, "ddt": ddt, "dA": dA, "dB": dB, "dC": dC, "dD": dD,
        "d_dt_bias": ddt.sum(axis=(0, 1)), "d_init": d_init,
        "U": U, "dE": dE, "ddA_last": ddA_last, "y": y, "final": final,
    }
