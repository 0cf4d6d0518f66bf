"""Grouped-query and multi-query attention (GQA / MQA) for the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: [FlashBoB] "FlashBoB: I/O-Efficient Exact Backward-over-Backward for
Softmax Attention", section 4.3 (the paragraph after Algorithm 1): with
H_Q > H_KV query heads sharing key/value heads, each query head in pass 1
reads its group's shared (K, V, U_K, U_V) head, and pass 2 sums d~(K), d~(V)
over the row blocks and the H_Q / H_KV query heads of the group.

Reading (the pages do not say which query heads form a group): query head h
uses key/value head h // G with G = H_Q / H_KV, i.e. consecutive query heads
share a head (the layout that repeating each K/V head G times produces).

Why the outputs decompose: dK and dV of a shared head are sums over its
group's query heads, so <dK, U_K> + <dV, U_V> splits into one term per query
head and Phi = sum_h Phi_h, where Phi_h is the multi-head functional of
[FlashBoB] section 4.1 for query head h on its group's head.  Every row
quantity of query head h (O, L, D, alpha, E, dQ, gQ, gdO) is therefore the
multi-head one on (q_h, k_g, v_g, do_h, u_Q,h, u_K,g, u_V,g); the key-side
outputs (dK, dV, gK, gV) of head g are the sums of the multi-head ones over
h in the group.  The functions below compute exactly that, with the
multi-head definitions of ``dense`` and ``streaming``.
"""
from __future__ import annotations

import numpy as np

from .dense import bob_dense
from .streaming import col_pass, row_pass

ROW_KEYS = ("O", "L", "D", "alpha", "E", "dQ", "gQ", "gdO")
COL_KEYS = ("dK", "dV", "gK", "gV")


def group_size(Hq, Hkv):
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"H_Q = {Hq} is not a multiple of H_KV = {Hkv}")
    return Hq // Hkv


def bob_dense_gqa(q, k, v, do, uq, uk, uv, tau, causal=False):
    """q, do, uq: (H_Q, N, d); k, v, uk, uv: (H_KV, N, d); float64.

    Returns row quantities with a leading H_Q axis and key-side quantities
    with a leading H_KV axis."""
    Hq, Hkv = q.shape[0], k.shape[0]
    G = group_size(Hq, Hkv)
    out = {}
    for h in range(Hq):
        g = h // G
        r = bob_dense(q[h], k[g], v[g], do[h], uq[h], uk[g], uv[g], tau, causal)
        for key in ROW_KEYS:
            out.setdefault(key, np.zeros((Hq,) + r[key].shape))[h] = r[key]
        for key in COL_KEYS:
            out.setdefault(key, np.zeros((Hkv,) + r[key].shape))[g] += r[key]
    return out


def col_pass_group(q, k, v, do, uq, uk, uv, tau, states, cols=None, causal=False, **kw):
    """Key-side outputs of one shared head for the columns ``cols``: the sum
    over the group's query heads.  q, do, uq, states: one entry per query
    head of the group; k, v, uk, uv: (N, d) of the shared head."""
    total = None
    for qh, doh, uqh, st in zip(q, do, uq, states):
        c = col_pass(qh, k, v, doh, uqh, uk, uv, tau, st, cols=cols, causal=causal, **kw)
        if total is None:
            total = {key: val.copy() for key, val in c.items()}
        else:
            for key in total:
                total[key] += c[key]
    return total


def bob_streaming_gqa(q, k, v, do, uq, uk, uv, tau, threads=None, strip=None, col_chunk=2048, causal=False):
    """Full BoB for q, do, uq of shape (B, H_Q, N, d) and k, v, uk, uv of
    shape (B, H_KV, N, d), float64, strip by strip (no N x N array)."""
    B, Hq = q.shape[:2]
    Hkv = k.shape[1]
    G = group_size(Hq, Hkv)
    res = {}
    for b in range(B):
        for g in range(Hkv):
            heads = range(g * G, (g + 1) * G)
            states = []
            for h in heads:
                r = row_pass(q[b, h], k[b, g], v[b, g], do[b, h], uq[b, h], uk[b, g], uv[b, g], tau,
                             outputs="all", strip=strip, col_chunk=col_chunk, threads=threads, causal=causal)
                states.append(r)
                for key, val in r.items():
                    res.setdefault(key, np.zeros((B, Hq) + val.shape))[b, h] = val
            c = col_pass_group([q[b, h] for h in heads], k[b, g], v[b, g], [do[b, h] for h in heads],
                               [uq[b, h] for h in heads], uk[b, g], uv[b, g], tau, states,
                               causal=causal, threads=threads, row_chunk=col_chunk)
            for key, val in c.items():
                res.setdefault(key, np.zeros((B, Hkv) + val.shape))[b, g] = val
    return res
