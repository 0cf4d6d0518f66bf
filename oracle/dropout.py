"""Dense float64 oracle of attention with dropout: forward, first backward and
backward-over-backward (BoB).  TEST INFRASTRUCTURE ONLY (see the package
docstring).

Sources:

* [FlashBoB] "FlashBoB: I/O-Efficient Exact Backward-over-Backward for Softmax
  Attention", appendix G, "Analytical dropout extension": with the forward's
  scaled keep mask g, alpha_i = sum_j P_ij F_ij, C = g * (dO U_V^T),
  d~P_ij = C_ij + F_ij (A_ij - D_i) - alpha_i A_ij, E_i = sum_j P_ij d~P_ij,
  d~S_ij = P_ij (d~P_ij - E_i), h_ij = F_ij - alpha_i, where A = g * (dO V^T)
  is the first backward's dP.  The page prints these identities only; the
  remaining outputs follow from the same reverse-mode steps (appendix D) with
  the forward O = (P * g) V: d~(Q) = tau (d~S K + dS U_K), d~(K) =
  tau (d~S^T Q + dS^T U_Q) with dS = P * (A - D), d~(V) = (P g h)^T dO and
  d~(dO) = (P g) U_V + (P g h) V.  The pins in tests/test_oracle_dropout.py
  check all of them against central differences of the dropout backward.
* The mask g is the library's: Philox4x64-10 (Salmon, Moraes, Dror, Shaw,
  "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011), implemented here
  from that definition (pinned against numpy's Philox bit generator).
  Element (i, j) of head bh takes byte j % 8 of output word i % 4 of the
  block for counter (i // 4, j // 8, bh, 0) and key (seed, 0); with
  t = round(256 p) it is kept iff the byte is >= t and then scaled by
  256 / (256 - t).
"""
from __future__ import annotations

import numpy as np

from .dense import causal_mask

_M0, _M1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157  # Philox4x64 multipliers
_W0, _W1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B  # Weyl key increments
_LO = np.uint64(0xFFFFFFFF)


def _mulhilo(a, m):
    """High and low 64-bit words of the 128-bit product a * m (uint64 arrays),
    from four 32 x 32 -> 64-bit partial products."""
    m = np.uint64(m)
    a_lo, a_hi = a & _LO, a >> np.uint64(32)
    m_lo, m_hi = m & _LO, m >> np.uint64(32)
    ll, lh, hl, hh = a_lo * m_lo, a_lo * m_hi, a_hi * m_lo, a_hi * m_hi
    mid = (ll >> np.uint64(32)) + (lh & _LO) + (hl & _LO)
    lo = (ll & _LO) | ((mid & _LO) << np.uint64(32))
    hi = hh + (lh >> np.uint64(32)) + (hl >> np.uint64(32)) + (mid >> np.uint64(32))
    return hi, lo


def philox4x64_10(c0, c1, c2, c3, k0, k1):
    """Philox4x64-10 block function on uint64 arrays (broadcast): ten rounds,
    each replacing (c0, c1, c2, c3) by (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2),
    hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)), with the key advanced by (W0, W1) between
    rounds.  Returns the four output words."""
    with np.errstate(over="ignore"):
        c = [np.asarray(x, dtype=np.uint64) for x in (c0, c1, c2, c3)]
        k0, k1 = np.uint64(k0), np.uint64(k1)
        for r in range(10):
            if r:
                k0 = np.uint64((int(k0) + _W0) % 2 ** 64)
                k1 = np.uint64((int(k1) + _W1) % 2 ** 64)
            hi0, lo0 = _mulhilo(c[0], _M0)
            hi1, lo1 = _mulhilo(c[2], _M1)
            c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return c


def threshold(p):
    """t = round(256 p) and the keep scale 256 / (256 - t)."""
    t = int(np.floor(p * 256.0 + 0.5))
    if not 0 <= t <= 255:
        raise ValueError("dropout rate must round to a threshold in 0..255")
    return t, 256.0 / (256 - t)


def keep_bytes(bh, N, seed):
    """The generator byte of every element (i, j) of head bh, an N x N uint8
    array."""
    i = np.arange(N, dtype=np.uint64)[:, None]
    j = np.arange(N, dtype=np.uint64)[None, :]
    w = philox4x64_10(i >> np.uint64(2), j >> np.uint64(3), np.uint64(bh), np.uint64(0), np.uint64(seed), 0)
    word = np.select([(i & np.uint64(3)) == np.uint64(k) for k in range(4)], w)
    return ((word >> (np.uint64(8) * (j & np.uint64(7)))) & np.uint64(0xFF)).astype(np.uint8)


def dropout_mask(bh, N, p, seed):
    """The scaled keep mask g of head bh (N x N float64): 256 / (256 - t) where
    the element's byte is >= t, else 0; all ones when t = 0."""
    t, scale = threshold(p)
    if t == 0:
        return np.ones((N, N))
    return np.where(keep_bytes(bh, N, seed) >= t, scale, 0.0)


def forward_dropout(q, k, v, tau, g, causal=False):
    """S = tau Q K^T (+ causal mask), P = softmax(S), L = logsumexp(S) over P
    (no mask), O = (P * g) V."""
    S = tau * (q @ k.T)
    if causal:
        S = S + causal_mask(S.shape[0])
    m = S.max(axis=1, keepdims=True)
    L = (m + np.log(np.exp(S - m).sum(axis=1, keepdims=True)))[:, 0]
    P = np.exp(S - L[:, None])
    O = (P * g) @ v
    return {"S": S, "P": P, "O": O, "L": L}


def backward_dropout(q, k, v, do, tau, g, causal=False):
    """First backward with the forward's mask: dV = (P g)^T dO,
    A = g * (dO V^T) (the dP of the masked forward), D_i = sum_j P_ij A_ij
    (= rowsum(dO * O), both returned), dS = P * (A - D), dQ = tau dS K,
    dK = tau dS^T Q."""
    f = forward_dropout(q, k, v, tau, g, causal)
    P, O = f["P"], f["O"]
    A = g * (do @ v.T)
    dV = (P * g).T @ do
    D = (do * O).sum(axis=1)
    D_from_P = (P * A).sum(axis=1)
    dS = P * (A - D[:, None])
    return {**f, "A": A, "dS": dS, "D": D, "D_from_P": D_from_P,
            "dQ": tau * (dS @ k), "dK": tau * (dS.T @ q), "dV": dV}


def phi_dropout(q, k, v, do, uq, uk, uv, tau, g, causal=False):
    """Phi = <dQ, U_Q> + <dK, U_K> + <dV, U_V> of the dropout backward."""
    b = backward_dropout(q, k, v, do, tau, g, causal)
    return float((b["dQ"] * uq).sum() + (b["dK"] * uk).sum() + (b["dV"] * uv).sum())


def bob_dropout(q, k, v, do, uq, uk, uv, tau, g, causal=False):
    """BoB of the dropout backward by the identities of the analytical dropout
    extension (module docstring): F, alpha, C, d~P, E, d~S, h as printed, and
    the four outputs from them.  Returns the outputs, the row scalars alpha and
    E, and the forward/backward state."""
    b = backward_dropout(q, k, v, do, tau, g, causal)
    P, A, dS, D = b["P"], b["A"], b["dS"], b["D"]
    F = tau * (uq @ k.T + q @ uk.T)
    alpha = (P * F).sum(axis=1)
    C = g * (do @ uv.T)
    dt_P = C + F * (A - D[:, None]) - alpha[:, None] * A
    E = (P * dt_P).sum(axis=1)
    dt_S = P * (dt_P - E[:, None])
    h = F - alpha[:, None]
    Pg = P * g
    gQ = tau * (dt_S @ k + dS @ uk)
    gK = tau * (dt_S.T @ q + dS.T @ uq)
    gV = (Pg * h).T @ do
    gdO = Pg @ uv + (Pg * h) @ v
    return {**b, "F": F, "C": C, "alpha": alpha, "E": E, "dt_P": dt_P, "dt_S": dt_S,
            "gQ": gQ, "gK": gK, "gV": gV, "gdO": gdO}


def bob_dropout_heads(q, k, v, do, uq, uk, uv, tau, p, seed, causal=False):
    """All heads of [B, H, N, d] inputs (k, v, uk, uv with H_kv heads dividing
    H): each query head bh = b H + h takes its own mask and the key/value head
    h // (H / H_kv); the key-side outputs sum over each group's query heads
    ([FlashBoB] section 4.3, paragraph after Algorithm 1).  Returns dense
    outputs O, L, D, alpha, E, gQ, gdO ([B, H, ...]) and gK, gV, dK, dV
    ([B, H_kv, ...]) and dQ."""
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    out = {n: np.zeros((B, H, N, d)) for n in ("O", "gQ", "gdO", "dQ")}
    out.update({n: np.zeros((B, Hkv, N, d)) for n in ("gK", "gV", "dK", "dV")})
    out.update({n: np.zeros((B, H, N)) for n in ("L", "D", "alpha", "E")})
    for b in range(B):
        for h in range(H):
            hk = h // G
            g = dropout_mask(b * H + h, N, p, seed)
            r = bob_dropout(q[b, h], k[b, hk], v[b, hk], do[b, h], uq[b, h], uk[b, hk], uv[b, hk], tau, g, causal)
            for n in ("O", "gQ", "gdO", "dQ"):
                out[n][b, h] = r[n]
            for n in ("L", "D", "alpha", "E"):
                out[n][b, h] = r[n]
            for n in ("gK", "gV", "dK", "dV"):
                out[n][b, hk] += r[n]
    return out
