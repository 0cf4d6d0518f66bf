"""Dense float64 oracle: every N x N matrix is materialised (use for N <= ~1024).

All functions take one attention head: 2-D arrays of shape (N, d) (``q``,
``k``, ``v``, ``do`` and the cotangents ``uq``, ``uk``, ``uv``), the softmax
scale ``tau`` and ``causal``.  With ``causal`` the additive mask term B_mask of
[FlashBoB] section 3 is -inf where key j > query i and 0 elsewhere, so the
softmax runs over the valid columns j <= i only; P is exactly 0 on the
masked entries, which is all the later formulas need (every N x N quantity
enters the outputs multiplied by P).
"""
from __future__ import annotations

import numpy as np


def causal_mask(N):
    """B_mask of [FlashBoB] section 3 for causal attention: -inf above the
    diagonal (key j > query i), 0 elsewhere."""
    m = np.zeros((N, N))
    m[np.triu_indices(N, 1)] = -np.inf
    return m


def forward_dense(q, k, v, tau, causal=False):
    """Forward pass and saved log-normaliser.

    [FlashBoB] section 3: S = tau Q K^T, P = softmax(S) row-wise, O = P V, and
    the saved row statistic L_i = log sum_j exp(S_ij) (natural log), from
    which P_ij = exp(S_ij - L_i).  The max is subtracted before exponentiating
    only to avoid overflow; it cancels exactly in L.
    """
    S = tau * (q @ k.T)
    if causal:
        S = S + causal_mask(S.shape[0])
    m = S.max(axis=1, keepdims=True)
    L = (m + np.log(np.exp(S - m).sum(axis=1, keepdims=True)))[:, 0]
    P = np.exp(S - L[:, None])
    O = P @ v
    return {"S": S, "P": P, "O": O, "L": L}


def backward_dense(q, k, v, do, tau, causal=False):
    """First backward of attention at output cotangent dO.

    [FlashBoB] section 3: dP = dO V^T, dV = P^T dO, dS_ij = P_ij (dP_ij - D_i),
    dQ = tau dS K, dK = tau dS^T Q, with D_i = sum_j P_ij dP_ij, which
    [FA2-recompute] shows equals rowsum(dO * O).  Both forms of D are
    returned so the identity can be checked.
    """
    f = forward_dense(q, k, v, tau, causal)
    P, O = f["P"], f["O"]
    dP = do @ v.T
    dV = P.T @ do
    D = (do * O).sum(axis=1)
    D_from_P = (P * dP).sum(axis=1)
    dS = P * (dP - D[:, None])
    dQ = tau * (dS @ k)
    dK = tau * (dS.T @ q)
    return {**f, "dP": dP, "dS": dS, "D": D, "D_from_P": D_from_P,
            "dQ": dQ, "dK": dK, "dV": dV}


def phi_dense(q, k, v, do, uq, uk, uv, tau, causal=False):
    """The BoB functional of [FlashBoB] section 4.1:
    Phi = <dQ, U_Q> + <dK, U_K> + <dV, U_V> (Frobenius inner products)."""
    b = backward_dense(q, k, v, do, tau, causal)
    return float((b["dQ"] * uq).sum() + (b["dK"] * uk).sum() + (b["dV"] * uv).sum())


def bob_dense(q, k, v, do, uq, uk, uv, tau, causal=False):
    """Backward-over-backward by the reverse-mode steps of [FlashBoB] appendix D.

    The cotangents on the first-backward outputs are U_Q, U_K, U_V (appendix D,
    notation).  Step by step:

    * Step 1: F = d~(dS) = tau (U_Q K^T + Q U_K^T).
    * Step 2: d~(dP) = P * (F - alpha), with the row scalar
      alpha_i = sum_j P_ij F_ij (D depends on dP through D = sum_j P dP).
    * Step 3: d~(V) = d~(dP)^T dO; the dP child contributes d~(dP) V to d~(dO).
    * Step 4: C = dO U_V^T is d~(P) from the dV child; the dV child
      contributes P U_V to d~(dO).
    * Step 5: the dS child adds F * (dP - D) - alpha * dP to d~(P).
    * Step 6: softmax Jacobian: E_i = sum_j P_ij d~(P)_ij and
      d~(S) = P * (d~(P) - E).
    * Step 7: d~(Q) = tau (d~(S) K + dS U_K), d~(K) = tau (d~(S)^T Q + dS^T U_Q).

    These are the final assembled identities of appendix D (also the
    displayed outputs of section 4.2, with h = F - alpha).  Returns the four
    outputs gQ = d~(Q), gK = d~(K), gV = d~(V), gdO = d~(dO), the row scalars
    alpha and E, and the forward/backward state.
    """
    b = backward_dense(q, k, v, do, tau, causal)
    P, dP, dS, D = b["P"], b["dP"], b["dS"], b["D"]
    # Step 1
    F = tau * (uq @ k.T + q @ uk.T)
    # Step 2
    alpha = (P * F).sum(axis=1)
    h = F - alpha[:, None]
    dt_dP = P * h
    # Step 3
    gV = dt_dP.T @ do
    gdO = dt_dP @ v
    # Step 4
    C = do @ uv.T
    gdO = gdO + P @ uv
    # Step 5
    dt_P = C + F * (dP - D[:, None]) - alpha[:, None] * dP
    # Step 6
    E = (P * dt_P).sum(axis=1)
    dt_S = P * (dt_P - E[:, None])
    # Step 7
    gQ = tau * (dt_S @ k + dS @ uk)
    gK = tau * (dt_S.T @ q + dS.T @ uq)
    return {**b, "F": F, "C": C, "alpha": alpha, "E": E, "dt_P": dt_P,
            "dt_S": dt_S, "gQ": gQ, "gK": gK, "gV": gV, "gdO": gdO}
