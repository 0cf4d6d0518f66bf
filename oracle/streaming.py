"""Streaming float64 oracle: the same definitions as ``dense``, evaluated in
row strips and column chunks so that no N x N array is ever held.

Rows of attention are independent, so a strip of rows is computed exactly as
the dense definition would compute those rows.  Row sums over the key index
(the log-normaliser, O, alpha, E and the row-owned outputs) are taken chunk by
chunk over the keys and added up; this only re-associates float64 sums.
Because each row scalar needs a full row before the next one can be formed
(L before P, then alpha, then E), the row pass makes one sweep over the keys
per scalar, in the order the definitions need them:

1. row max of S (overflow guard for the log-sum-exp);
2. l_i = sum_j exp(S_ij - m_i) and the unnormalised forward output, giving
   L_i = m_i + log l_i and O = P V ([FlashBoB] section 3), then
   D_i = rowsum(dO * O)_i ([FA2-recompute]);
3. alpha_i = sum_j P_ij F_ij ([FlashBoB] appendix D, Step 2);
4. E_i = sum_j P_ij d~(P)_ij with
   d~(P) = C + F * (dP - D) - alpha * dP (appendix D, Steps 4-6);
5. the row-owned outputs gQ = tau (d~(S) K + dS U_K) and
   gdO = P U_V + (P * h) V (appendix D, Steps 3, 4, 7), and the first-backward
   dQ = tau dS K ([FlashBoB] section 3).

The column pass forms the column-owned outputs gK = tau (d~(S)^T Q + dS^T U_Q)
and gV = (P * h)^T dO, and the first-backward dK, dV, for any subset of key
columns, from the row scalars L, D, alpha, E of *all* rows.

Strips run on a thread pool (numpy releases the GIL inside BLAS and large
ufuncs); BLAS itself is pinned to one thread meanwhile.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

try:  # optional: pin BLAS threads while the strip pool runs
    from threadpoolctl import threadpool_limits
except Exception:  # pragma: no cover
    threadpool_limits = None


def _threads(n):
    if n is not None:
        return max(1, int(n))
    return max(1, os.cpu_count() or 1)


def _run_pool(fn, tasks, threads):
    threads = _threads(threads)
    if threads == 1 or len(tasks) <= 1:
        return [fn(t) for t in tasks]
    if threadpool_limits is not None:
        with threadpool_limits(limits=1, user_api="blas"):
            with ThreadPoolExecutor(threads) as ex:
                return list(ex.map(fn, tasks))
    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(fn, tasks))


def _chunks(n, size):
    return [(s, min(n, s + size)) for s in range(0, n, size)]


def _mask(rows, a, b, causal):
    """The causal part of B_mask ([FlashBoB] section 3) for query rows ``rows``
    and key columns a..b-1: -inf where key > query, else 0 (None if not causal)."""
    if not causal:
        return None
    return np.where(np.arange(a, b)[None, :] > np.asarray(rows)[:, None], -np.inf, 0.0)


def _row_strip(q, k, v, do, uq, uk, uv, tau, rows, col_chunk, outputs, causal=False):
    """All row quantities for the rows ``rows`` (an index array) of one head."""
    N = k.shape[0]
    Q, dO, UQ = q[rows], do[rows], uq[rows]
    R = Q.shape[0]
    chunks = _chunks(N, col_chunk)
    if causal:
        # A chunk whose keys all lie above every row of the strip is masked
        # throughout: P = 0 there, so it adds exact zeros to every sum.
        chunks = [(a, b) for a, b in chunks if a <= int(np.max(rows))]

    def scores(a, b):
        S = tau * (Q @ k[a:b].T)
        m = _mask(rows, a, b, causal)
        return S if m is None else S + m

    # sweep 1: row max
    m = np.full(R, -np.inf)
    for a, b in chunks:
        m = np.maximum(m, scores(a, b).max(axis=1))
    # sweep 2: log-normaliser and forward output
    l = np.zeros(R)
    On = np.zeros((R, v.shape[1]))
    for a, b in chunks:
        e = np.exp(scores(a, b) - m[:, None])
        l += e.sum(axis=1)
        On += e @ v[a:b]
    L = m + np.log(l)
    O = On / l[:, None]
    D = (dO * O).sum(axis=1)
    out = {"L": L, "O": O, "D": D}
    if outputs == "fwd":
        return out

    def blocks(a, b):
        P = np.exp(scores(a, b) - L[:, None])
        F = tau * (UQ @ k[a:b].T + Q @ uk[a:b].T)
        dP = dO @ v[a:b].T
        C = dO @ uv[a:b].T
        return P, F, dP, C

    # sweep 3: alpha
    alpha = np.zeros(R)
    for a, b in chunks:
        P = np.exp(scores(a, b) - L[:, None])
        F = tau * (UQ @ k[a:b].T + Q @ uk[a:b].T)
        alpha += (P * F).sum(axis=1)
    # sweep 4: E
    E = np.zeros(R)
    for a, b in chunks:
        P, F, dP, C = blocks(a, b)
        dt_P = C + F * (dP - D[:, None]) - alpha[:, None] * dP
        E += (P * dt_P).sum(axis=1)
    out.update(alpha=alpha, E=E)
    if outputs == "state":
        return out
    # sweep 5: row-owned outputs
    d = q.shape[1]
    gQ = np.zeros((R, d))
    gdO = np.zeros((R, d))
    dQ = np.zeros((R, d))
    for a, b in chunks:
        P, F, dP, C = blocks(a, b)
        dt_P = C + F * (dP - D[:, None]) - alpha[:, None] * dP
        dt_S = P * (dt_P - E[:, None])
        dS = P * (dP - D[:, None])
        h = F - alpha[:, None]
        gQ += tau * (dt_S @ k[a:b] + dS @ uk[a:b])
        gdO += P @ uv[a:b] + (P * h) @ v[a:b]
        dQ += tau * (dS @ k[a:b])
    out.update(gQ=gQ, gdO=gdO, dQ=dQ)
    return out


def _default_strip(N, d):
    return 64 if N <= 65536 else 128


def row_pass(q, k, v, do, uq, uk, uv, tau, rows=None, outputs="all",
             strip=None, col_chunk=2048, threads=None, causal=False):
    """Row quantities of one head for the rows ``rows`` (default: all).

    ``outputs``: "fwd" -> L, O, D; "state" -> also alpha, E;
    "all" -> also gQ, gdO, dQ.  Arrays are indexed like ``rows``.
    """
    N = q.shape[0]
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    strip = strip or _default_strip(N, q.shape[1])
    tasks = [rows[s:s + strip] for s in range(0, len(rows), strip)]
    parts = _run_pool(
        lambda r: _row_strip(q, k, v, do, uq, uk, uv, tau, r, col_chunk, outputs, causal),
        tasks, threads)
    return {key: np.concatenate([p[key] for p in parts], axis=0) for key in parts[0]}


def row_state(q, k, v, do, uq, uk, uv, tau, **kw):
    """L, O, D, alpha, E for every row of one head."""
    return row_pass(q, k, v, do, uq, uk, uv, tau, outputs="state", **kw)


def _col_strip(q, k, v, do, uq, uk, uv, tau, L, D, alpha, E, cols, row_chunk, causal=False):
    N, d = q.shape
    Kc, Vc, UKc, UVc = k[cols], v[cols], uk[cols], uv[cols]
    Cn = Kc.shape[0]
    gK = np.zeros((Cn, d))
    gV = np.zeros((Cn, d))
    dK = np.zeros((Cn, d))
    dV = np.zeros((Cn, d))
    first_col = int(np.min(cols))
    for a, b in _chunks(N, row_chunk):
        if causal and b - 1 < first_col:
            continue  # every row of the chunk precedes every column: P = 0
        Qi, dOi, UQi = q[a:b], do[a:b], uq[a:b]
        La, Da, Aa, Ea = L[a:b, None], D[a:b, None], alpha[a:b, None], E[a:b, None]
        S = tau * (Qi @ Kc.T)
        if causal:
            S = S + np.where(np.asarray(cols)[None, :] > np.arange(a, b)[:, None], -np.inf, 0.0)
        P = np.exp(S - La)
        F = tau * (UQi @ Kc.T + Qi @ UKc.T)
        dP = dOi @ Vc.T
        C = dOi @ UVc.T
        dt_P = C + F * (dP - Da) - Aa * dP
        dt_S = P * (dt_P - Ea)
        dS = P * (dP - Da)
        h = F - Aa
        gK += tau * (dt_S.T @ Qi + dS.T @ UQi)
        gV += (P * h).T @ dOi
        dK += tau * (dS.T @ Qi)
        dV += P.T @ dOi
    return {"gK": gK, "gV": gV, "dK": dK, "dV": dV}


def col_pass(q, k, v, do, uq, uk, uv, tau, state, cols=None, strip=64,
             row_chunk=2048, threads=None, causal=False):
    """Column-owned outputs gK, gV (and dK, dV) of one head for the key
    columns ``cols`` (default: all), given the row state of every row."""
    N = k.shape[0]
    cols = np.arange(N) if cols is None else np.asarray(cols, dtype=np.int64)
    tasks = [cols[s:s + strip] for s in range(0, len(cols), strip)]
    L, D, alpha, E = state["L"], state["D"], state["alpha"], state["E"]
    parts = _run_pool(
        lambda c: _col_strip(q, k, v, do, uq, uk, uv, tau, L, D, alpha, E, c, row_chunk, causal),
        tasks, threads)
    return {key: np.concatenate([p[key] for p in parts], axis=0) for key in parts[0]}


def bob_streaming(q, k, v, do, uq, uk, uv, tau, threads=None, strip=None,
                  col_chunk=2048, causal=False):
    """Full BoB over tensors of shape (B, H, N, d), float64.

    Returns a dict of (B, H, N, d) arrays gQ, gK, gV, gdO, dQ, dK, dV, O and
    (B, H, N) arrays L, D, alpha, E.
    """
    B, H, N, d = q.shape
    res = {}
    for b in range(B):
        for hh in range(H):
            args = [t[b, hh] for t in (q, k, v, do, uq, uk, uv)]
            r = row_pass(*args, tau, outputs="all", strip=strip,
                         col_chunk=col_chunk, threads=threads, causal=causal)
            c = col_pass(*args, tau, r, threads=threads, row_chunk=col_chunk,
                         causal=causal)
            r.update(c)
            for key, val in r.items():
                if key not in res:
                    res[key] = np.zeros((B, H) + val.shape)
                res[key][b, hh] = val
    return res
