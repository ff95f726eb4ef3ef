"""Dense fp64 forward and backward of relative-position attention.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: "Fast and Exact Relative-Position Attention via Structure-Aware
Kernels" (nanless.github.io digest), section on the score formula, Eq. (1):
each score adds to the content product q_i.k_j the relation terms of the row
r = phi(i, j): a query-side product q_i.aQ[r], a key-side product k_j.aK[r]
and a scalar b[r]; the sum is scaled by tau and an additive mask M_ij (0 or
-inf here) is added.  A row softmax gives P and the output is O = P V (the
scaled-dot-product form on the auturnal.com attention primer).

Readings adopted where the page is silent:
* tau multiplies the whole bracket, b included (Eq. (1) puts b inside).
* masks: causal means M_ij = -inf for j > i; key padding means M_ij = -inf for
  j >= key_len[batch].  A row with every key masked has O = 0, LSE = -inf and
  contributes no gradient.
* LSE_i = log sum_j exp(S_ij) (natural log).

Gradients (chain rule through Eq. (1); the per-row sums match Eq. (4) of the
page's backward section, dZ^Q_ir = tau * sum_{j: phi(i,j)=r} dS_ij and the
key-side analogue):
    dV = P^T dO,   dP = dO V^T,   D_i = sum_j P_ij dP_ij,   dS = P * (dP - D)
    G  = tau * dS
    CQ[i, r] = sum_{j: phi=r} G_ij,     CK[j, r] = sum_{i: phi=r} G_ij
    dQ = G K + CQ aQ,   dK = G^T Q + CK aK
    daQ = CQ^T Q,       daK = CK^T K,   db_r = sum_i CQ[i, r]

Tables may be per head (aQ, aK: [H, R, d]; b: [H, R]) or shared by all heads
(aQ, aK: [R, d]; b: [R]); the gradient has the shape of its table.
Everything is computed in float64 one (batch, head) pair and one block of
query rows at a time, with library matmuls, exp and bincount as the steps.

Optional attention dropout (``dropout`` = (t, seed, offset), drop probability
t / 256; the readings are in ``oracle/dropout.py``): the weights P are
replaced by P * K / (1 - p) in O = P V, and in the backward dV uses the same
weights while dP = (dO V^T) * K / (1 - p); D_i and dS = P * (dP - D) keep
their form.
"""

import numpy as np

from .dropout import keep_mask, keep_scale
from .phi import num_rows, phi_rows


def _vec_table(t, h, shared_ndim):
    """Per-head slice of a table whose shared form has ``shared_ndim`` dims."""
    if t is None:
        return None
    return t if t.ndim == shared_ndim else t[h]


def _scores(qh, kh, ZQ, ZK, bh, rows_of, N, i0, i1, tau, causal, kl):
    """tau * (q.k + ZQ[i, r] + ZK[j, r] + b[r]) + M for query rows i0..i1-1."""
    ii = np.arange(i0, i1, dtype=np.int64)[:, None]
    jj = np.arange(N, dtype=np.int64)[None, :]
    r = rows_of[jj - ii + (N - 1)]
    raw = qh[i0:i1] @ kh.T
    if ZQ is not None:
        raw = raw + np.take_along_axis(ZQ[i0:i1], r, axis=1)
    if ZK is not None:
        raw = raw + ZK[jj, r]
    if bh is not None:
        raw = raw + bh[r]
    S = tau * raw
    masked = np.zeros(S.shape, dtype=bool)
    if causal:
        masked |= jj > ii
    if kl is not None:
        masked |= jj >= kl
    S[masked] = -np.inf
    return S, r


def _softmax_rows(S):
    m = S.max(axis=1)
    dead = ~np.isfinite(m)
    m_safe = np.where(dead, 0.0, m)
    E = np.exp(S - m_safe[:, None])
    l = E.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        P = np.where(dead[:, None], 0.0, E / np.where(dead, 1.0, l)[:, None])
        lse = np.where(dead, -np.inf, m_safe + np.log(np.where(dead, 1.0, l)))
    return P, lse


def _pairs(B, H, bh):
    return [(b_, h_) for b_ in range(B) for h_ in range(H)] if bh is None else list(bh)


def forward(q, k, v, aQ=None, aK=None, b=None, *, phi, tau, causal=False,
            key_len=None, row_block=512, bh=None, query_rows=None, dropout=None):
    """Return (O [B,H,N,d], LSE [B,H,N]) in float64.

    ``bh`` restricts the work to a list of (batch, head) pairs and
    ``query_rows`` to a sorted array of query indices; entries not computed
    are NaN.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, N, d = q.shape
    O = np.full((B, H, N, d), np.nan)
    LSE = np.full((B, H, N), np.nan)
    if N == 0:
        return O, LSE
    rows_of = phi_rows(phi, N)
    blocks = _row_blocks(N, row_block, query_rows)
    for bi, h in _pairs(B, H, bh):
        qh, kh, vh = q[bi, h], k[bi, h], v[bi, h]
        aQh = _vec_table(aQ, h, 2)
        aKh = _vec_table(aK, h, 2)
        bvec = _vec_table(b, h, 1)
        ZQ = qh @ aQh.T if aQh is not None else None
        ZK = kh @ aKh.T if aKh is not None else None
        kl = None if key_len is None else int(key_len[bi])
        for rows in blocks:
            S, _ = _scores(qh, kh, ZQ, ZK, bvec, rows_of, N, rows[0], rows[-1] + 1,
                           tau, causal, kl)
            sel = rows - rows[0]
            P, lse = _softmax_rows(S[sel])
            if dropout is not None:
                P = P * keep_mask(dropout, bi * H + h, rows, N) * keep_scale(dropout)
            O[bi, h, rows] = P @ vh
            LSE[bi, h, rows] = lse
    return O, LSE


def _row_blocks(N, row_block, query_rows):
    if query_rows is None:
        return [np.arange(i0, min(N, i0 + row_block)) for i0 in range(0, N, row_block)]
    qr = np.unique(np.asarray(query_rows, dtype=np.int64))
    out = []
    for i0 in range(0, N, row_block):
        sel = qr[(qr >= i0) & (qr < i0 + row_block)]
        if sel.size:
            out.append(sel)
    return out


def backward(q, k, v, aQ=None, aK=None, b=None, *, dO, phi, tau, causal=False,
             key_len=None, row_block=512, bh=None, query_rows=None, dropout=None):
    """Exact gradients of sum(O * dO).

    Returns a dict with dq, dk, dv ([B,H,N,d]) and daq, dak, db (shape of
    their table, or None when the table is absent).  With ``query_rows`` only
    dq is computed, for those rows (the rest is NaN); ``bh`` restricts the
    (batch, head) pairs (other entries NaN; table gradients then sum over the
    listed pairs only).
    """
    q, k, v, dO = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dO))
    B, H, N, d = q.shape
    rows_only = query_rows is not None
    dq = np.full((B, H, N, d), np.nan)
    dk = np.full((B, H, N, d), np.nan)
    dv = np.full((B, H, N, d), np.nan)
    daq = None if aQ is None else np.zeros(np.shape(aQ))
    dak = None if aK is None else np.zeros(np.shape(aK))
    db = None if b is None else np.zeros(np.shape(b))
    out = dict(dq=dq, dk=dk, dv=dv, daq=daq, dak=dak, db=db)
    if N == 0:
        return out
    R = num_rows(phi, N)
    rows_of = phi_rows(phi, N)
    blocks = _row_blocks(N, row_block, query_rows)
    for bi, h in _pairs(B, H, bh):
        qh, kh, vh, dOh = q[bi, h], k[bi, h], v[bi, h], dO[bi, h]
        aQh = _vec_table(aQ, h, 2)
        aKh = _vec_table(aK, h, 2)
        bvec = _vec_table(b, h, 1)
        ZQ = qh @ aQh.T if aQh is not None else None
        ZK = kh @ aKh.T if aKh is not None else None
        kl = None if key_len is None else int(key_len[bi])
        dQh = np.zeros((N, d))
        dKh = np.zeros((N, d))
        dVh = np.zeros((N, d))
        CK = np.zeros((N, R)) if (aKh is not None and not rows_only) else None
        for rows in blocks:
            i0, i1 = int(rows[0]), int(rows[-1]) + 1
            S, r = _scores(qh, kh, ZQ, ZK, bvec, rows_of, N, i0, i1, tau, causal, kl)
            sel = rows - i0
            S, r = S[sel], r[sel]
            P, _ = _softmax_rows(S)
            dP = dOh[rows] @ vh.T
            Pv = P  # the weights that multiply V in the forward
            if dropout is not None:
                Km = keep_mask(dropout, bi * H + h, rows, N) * keep_scale(dropout)
                Pv = P * Km
                dP = dP * Km
            Drow = (P * dP).sum(axis=1)
            G = tau * (P * (dP - Drow[:, None]))
            dQh[rows] = G @ kh
            if not rows_only:
                dVh += Pv.T @ dOh[rows]
                dKh += G.T @ qh[rows]
            nb = len(rows)
            if aQh is not None or bvec is not None:
                flat = (np.arange(nb, dtype=np.int64)[:, None] * R + r).ravel()
                CQ = np.bincount(flat, weights=G.ravel(), minlength=nb * R).reshape(nb, R)
                if aQh is not None:
                    dQh[rows] += CQ @ aQh
                if not rows_only:
                    if aQh is not None:
                        _acc(daq, h, CQ.T @ qh[rows])
                    if bvec is not None:
                        _acc(db, h, CQ.sum(axis=0))
            if CK is not None:
                jj = np.arange(N, dtype=np.int64)[None, :]
                flat = (jj * R + r).ravel()
                CK += np.bincount(flat, weights=G.ravel(), minlength=N * R).reshape(N, R)
        if CK is not None:
            dKh += CK @ aKh
            _acc(dak, h, CK.T @ kh)
        if rows_only:
            dq[bi, h, query_rows] = dQh[query_rows]
        else:
            dq[bi, h], dk[bi, h], dv[bi, h] = dQh, dKh, dVh
    return out


def _acc(grad, h, val):
    """Add ``val`` into the per-head or shared table gradient."""
    if grad.ndim == val.ndim:
        grad += val
    else:
        grad[h] += val
