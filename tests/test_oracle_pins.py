"""Pins of the float64 oracle against things other than itself.

Each test ties an oracle function to a fact fixed by the pages or by
mathematics: library routines (torch softmax / logsumexp / autograd in
float64 on the CPU), central finite differences, closed forms of special
cases, exact invariants.  Together they are chosen so that a dropped term, a
wrong sign or index, or a transposed operand anywhere in the oracle fails at
least one of them.
"""
import numpy as np
import pytest
import torch

from oracle import backward_dense, bob_dense, bob_streaming, forward_dense, phi_dense
from oracle.streaming import col_pass, row_pass

OUT_KEYS = ("gQ", "gK", "gV", "gdO")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def head(N, d, seed, qk=1.0, cot=1.0):
    r = np.random.default_rng(seed)
    t = [r.standard_normal((N, d)) for _ in range(7)]
    t[0] *= qk
    t[1] *= qk
    for i in (4, 5, 6):
        t[i] *= cot
    return t  # q, k, v, do, uq, uk, uv


def torch_bob(q, k, v, do, uq, uk, uv, tau):
    """Independent reference: float64 autograd double backward of the plain
    (materialising) attention, on the CPU."""
    Q, K, V, dO = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, do))
    UQ, UK, UV = (torch.tensor(x, dtype=torch.float64) for x in (uq, uk, uv))
    P = torch.softmax(tau * Q @ K.T, dim=-1)
    O = P @ V
    dQ, dK, dV = torch.autograd.grad(O, (Q, K, V), dO, create_graph=True)
    phi = (dQ * UQ).sum() + (dK * UK).sum() + (dV * UV).sum()
    g = torch.autograd.grad(phi, (Q, K, V, dO))
    return {"gQ": g[0].numpy(), "gK": g[1].numpy(), "gV": g[2].numpy(), "gdO": g[3].numpy(),
            "dQ": dQ.detach().numpy(), "dK": dK.detach().numpy(), "dV": dV.detach().numpy(),
            "O": O.detach().numpy(), "phi": float(phi.detach())}


def relerr(a, b):
    """max |a - b| / max |b|; an all-zero reference is compared in absolute terms."""
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-2))


# ---------------------------------------------------------------- forward


@pytest.mark.parametrize("N,d", [(1, 8), (13, 8), (100, 64), (257, 32)])
def test_forward_matches_torch_softmax_and_logsumexp(N, d):
    q, k, v = head(N, d, 11)[:3]
    tau = 1 / np.sqrt(d)
    f = forward_dense(q, k, v, tau)
    S = torch.tensor(q) @ torch.tensor(k).T * tau
    P = torch.softmax(S, dim=-1)
    assert relerr(f["P"], P.numpy()) < 1e-13
    assert relerr(f["O"], (P @ torch.tensor(v)).numpy()) < 1e-13
    assert np.max(np.abs(f["L"] - torch.logsumexp(S, dim=-1).numpy())) < 1e-12


# ---------------------------------------------------------------- first backward


def test_first_backward_central_fd_13x8():
    """The 13 x 8 problem of the FA2-recompute answer: central differences of
    <O, dO> against dQ, dK, dV (the page reports agreement to 1.7e-9)."""
    N, d = 13, 8
    q, k, v, do = head(N, d, 5)[:4]
    tau = 1 / np.sqrt(d)
    b = backward_dense(q, k, v, do, tau)

    def f(qq, kk, vv):
        return float((forward_dense(qq, kk, vv, tau)["O"] * do).sum())

    eps = 1e-6
    for name, idx, g in (("q", 0, b["dQ"]), ("k", 1, b["dK"]), ("v", 2, b["dV"])):
        base = [q.copy(), k.copy(), v.copy()]
        fd = np.zeros_like(g)
        for i in range(N):
            for a in range(d):
                p = [x.copy() for x in base]
                m = [x.copy() for x in base]
                p[idx][i, a] += eps
                m[idx][i, a] -= eps
                fd[i, a] = (f(*p) - f(*m)) / (2 * eps)
        assert np.max(np.abs(fd - g)) < 1e-8, name


def test_d_identity():
    """D_i = sum_j P_ij dP_ij equals rowsum(dO * O) (FA2-recompute; page
    reports 7e-16 on its example)."""
    for N, d, seed in ((13, 8, 1), (200, 64, 2), (512, 128, 3)):
        b = backward_dense(*head(N, d, seed)[:4], 1 / np.sqrt(d))
        assert np.max(np.abs(b["D"] - b["D_from_P"])) < 1e-12


def test_first_backward_matches_torch_autograd():
    N, d = 77, 16
    q, k, v, do = head(N, d, 9)[:4]
    tau = 1 / np.sqrt(d)
    t = torch_bob(q, k, v, do, *head(N, d, 10)[4:], tau)
    b = backward_dense(q, k, v, do, tau)
    for key in ("dQ", "dK", "dV"):
        assert relerr(b[key], t[key]) < 1e-12, key


# ---------------------------------------------------------------- BoB


def test_bob_central_fd_of_phi_13x8():
    """Every entry of gQ, gK, gV, gdO against a central difference of
    Phi = <dQ,U_Q> + <dK,U_K> + <dV,U_V> (FlashBoB section 4.1)."""
    N, d = 13, 8
    t = head(N, d, 21)
    tau = 1 / np.sqrt(d)
    out = bob_dense(*t, tau)
    eps = 1e-6
    for idx, key in enumerate(("gQ", "gK", "gV", "gdO")):
        fd = np.zeros((N, d))
        for i in range(N):
            for a in range(d):
                p = [x.copy() for x in t]
                m = [x.copy() for x in t]
                p[idx][i, a] += eps
                m[idx][i, a] -= eps
                fd[i, a] = (phi_dense(*p, tau) - phi_dense(*m, tau)) / (2 * eps)
        assert np.max(np.abs(fd - out[key])) < 2e-8 * max(1.0, np.max(np.abs(fd))), key


def test_bob_directional_fd_tiny_shape():
    """Random-direction central differences at the tiny workload's shape
    (N=128, d=64): <grad Phi, z> against (Phi(x+eps z) - Phi(x-eps z)) / 2 eps."""
    N, d = 128, 64
    t = head(N, d, 0)
    tau = 1 / np.sqrt(d)
    out = bob_dense(*t, tau)
    eps = 1e-5
    for idx, key in enumerate(("gQ", "gK", "gV", "gdO")):
        for s in range(8):
            z = rnd((N, d), 1000 + 10 * idx + s)
            p = [x.copy() for x in t]
            m = [x.copy() for x in t]
            p[idx] += eps * z
            m[idx] -= eps * z
            fd = (phi_dense(*p, tau) - phi_dense(*m, tau)) / (2 * eps)
            an = float((out[key] * z).sum())
            assert abs(fd - an) < 1e-6 * max(1.0, abs(an)), (key, s, fd, an)


@pytest.mark.parametrize("N,d,qk", [(1, 8, 1.0), (37, 8, 1.0), (128, 64, 1.0), (200, 64, 2.0),
                                    (64, 128, 1.0)])
def test_bob_dense_matches_torch_double_backward(N, d, qk):
    t = head(N, d, 31 + N, qk=qk)
    tau = 1 / np.sqrt(d)
    ref = torch_bob(*t, tau)
    out = bob_dense(*t, tau)
    for key in OUT_KEYS:
        assert relerr(out[key], ref[key]) < 1e-11, key
    assert abs(phi_dense(*t, tau) - ref["phi"]) < 1e-10 * max(1, abs(ref["phi"]))


def test_bob_linear_in_cotangents():
    N, d = 50, 16
    t = head(N, d, 41)
    u2 = head(N, d, 42)[4:]
    tau = 1 / np.sqrt(d)
    a, b = 0.7, -1.3
    o1 = bob_dense(*t, tau)
    o2 = bob_dense(*t[:4], *u2, tau)
    mix = [a * x + b * y for x, y in zip(t[4:], u2)]
    o3 = bob_dense(*t[:4], *mix, tau)
    for key in OUT_KEYS + ("alpha", "E"):
        assert relerr(o3[key], a * o1[key] + b * o2[key]) < 1e-12, key


def test_lower_bound_instance_reduces_to_forward():
    """V = dO = U_Q = U_K = 0, U_V = W gives gdO = softmax(tau Q K^T) W and
    gQ = gK = gV = 0 (the reduction of FlashBoB section 4.4)."""
    N, d = 96, 32
    q, k, _, _, _, _, w = head(N, d, 51)
    z = np.zeros((N, d))
    tau = 1 / np.sqrt(d)
    out = bob_dense(q, k, z, z, z, z, w, tau)
    P = torch.softmax(torch.tensor(q) @ torch.tensor(k).T * tau, dim=-1).numpy()
    assert relerr(out["gdO"], P @ w) < 1e-13
    for key in ("gQ", "gK", "gV"):
        assert np.max(np.abs(out[key])) == 0.0, key
    r = row_pass(q, k, z, z, z, z, w, tau, strip=7, col_chunk=13)
    assert relerr(r["gdO"], P @ w) < 1e-13


def test_zero_uq_uk_reduces_to_first_backward_with_v_replaced():
    """U_Q = U_K = 0: F = 0, so gQ, gK are the first backward with V := U_V,
    gdO is the forward output with V := U_V, and gV = 0 (torch reference)."""
    N, d = 70, 16
    q, k, v, do, _, _, uv = head(N, d, 61)
    z = np.zeros((N, d))
    tau = 1 / np.sqrt(d)
    out = bob_dense(q, k, v, do, z, z, uv, tau)
    t = torch_bob(q, k, uv, do, z, z, z, tau)
    assert relerr(out["gQ"], t["dQ"]) < 1e-12
    assert relerr(out["gK"], t["dK"]) < 1e-12
    assert relerr(out["gdO"], t["O"]) < 1e-13
    assert np.max(np.abs(out["gV"])) < 1e-15


def test_single_key_closed_form():
    """N = 1: P = 1, dS = 0, so Phi = <dO, U_V>: gdO = U_V and gQ = gK = gV = 0."""
    q, k, v, do, uq, uk, uv = head(1, 8, 71)
    out = bob_dense(q, k, v, do, uq, uk, uv, 0.3)
    assert np.allclose(out["gdO"], uv, rtol=0, atol=1e-15)
    for key in ("gQ", "gK", "gV"):
        assert np.max(np.abs(out[key])) < 1e-15


def test_euler_homogeneity():
    """Phi is linear in dO, so <gdO, dO> = Phi; Phi is affine in V with
    dQ, dK linear in V and dV free of V, so <gV, V> = <dQ,U_Q> + <dK,U_K>."""
    N, d = 90, 32
    t = head(N, d, 81)
    tau = 1 / np.sqrt(d)
    out = bob_dense(*t, tau)
    b = backward_dense(*t[:4], tau)
    phi = phi_dense(*t, tau)
    assert abs((out["gdO"] * t[3]).sum() - phi) < 1e-11 * max(1, abs(phi))
    rhs = (b["dQ"] * t[4]).sum() + (b["dK"] * t[5]).sum()
    assert abs((out["gV"] * t[2]).sum() - rhs) < 1e-11 * max(1, abs(rhs))


def test_shift_invariance_column_sums():
    """Adding the same vector to every key row leaves softmax unchanged, so
    sum_j gK_j = 0; rows of d~(S) sum to zero; and sum_j gV_j = 0 because
    sum_j P_ij (F_ij - alpha_i) = 0."""
    N, d = 120, 64
    t = head(N, d, 91)
    out = bob_dense(*t, 1 / np.sqrt(d))
    scale = np.max(np.abs(out["gK"]))
    assert np.max(np.abs(out["gK"].sum(axis=0))) < 1e-12 * N * scale
    assert np.max(np.abs(out["dt_S"].sum(axis=1))) < 1e-13
    assert np.max(np.abs(out["gV"].sum(axis=0))) < 1e-12 * N * np.max(np.abs(out["gV"]))


def test_alpha_and_r_second_forms():
    """alpha_i = tau (u_Q,i . B_i + q_i . (P U_K)_i) with B = P K, and
    R = (P * dP) K = dQ / tau + D * B: independent routes to the row scalars."""
    N, d = 64, 16
    t = head(N, d, 101)
    q, k, v, do, uq, uk, uv = t
    tau = 1 / np.sqrt(d)
    out = bob_dense(*t, tau)
    P = out["P"]
    Bm = P @ k
    alt = tau * ((uq * Bm).sum(1) + (q * (P @ uk)).sum(1))
    assert relerr(out["alpha"], alt) < 1e-12
    R = (P * out["dP"]) @ k
    assert relerr(R, out["dQ"] / tau + out["D"][:, None] * Bm) < 1e-12


# ---------------------------------------------------------------- streaming oracle


@pytest.mark.parametrize("strip,chunk", [(1, 5), (7, 64), (64, 33), (None, 4096)])
def test_streaming_matches_dense(strip, chunk):
    N, d = 150, 32
    t = head(N, d, 111)
    tau = 1 / np.sqrt(d)
    ref = bob_dense(*t, tau)
    r = row_pass(*t, tau, strip=strip, col_chunk=chunk, threads=3)
    c = col_pass(*t, tau, r, strip=strip or 64, row_chunk=chunk, threads=2)
    for key in ("L", "O", "D", "alpha", "E", "gQ", "gdO", "dQ"):
        assert relerr(r[key], ref[key]) < 1e-12, key
    for key in ("gK", "gV", "dK", "dV"):
        assert relerr(c[key], ref[key]) < 1e-12, key


def test_streaming_sampled_rows_and_columns():
    N, d = 300, 16
    t = head(N, d, 121, qk=2.0)
    tau = 1 / np.sqrt(d)
    ref = bob_dense(*t, tau)
    rows = np.array([0, 5, 17, 299, 150])
    r = row_pass(*t, tau, rows=rows, strip=2, col_chunk=64)
    for key in ("gQ", "gdO", "alpha", "E"):
        assert relerr(r[key], ref[key][rows]) < 1e-12
    st = row_pass(*t, tau, outputs="state")
    cols = np.array([3, 0, 299, 128])
    c = col_pass(*t, tau, st, cols=cols, strip=3, row_chunk=100)
    for key in ("gK", "gV"):
        assert relerr(c[key], ref[key][cols]) < 1e-12


def test_bob_streaming_multihead_vs_torch():
    B, H, N, d = 2, 2, 65, 8
    rng = np.random.default_rng(131)
    t = [rng.standard_normal((B, H, N, d)) for _ in range(7)]
    tau = 0.3
    out = bob_streaming(*t, tau, threads=2, strip=16, col_chunk=20)
    for b in range(B):
        for h in range(H):
            ref = torch_bob(*[x[b, h] for x in t], tau)
            for key in OUT_KEYS + ("dQ", "dK", "dV", "O"):
                assert relerr(out[key][b, h], ref[key]) < 1e-12, (b, h, key)


# ---------------------------------------------------------------- causal mask


def torch_bob_causal(q, k, v, do, uq, uk, uv, tau):
    """Independent reference for causal attention: float64 autograd double
    backward with the mask applied by masked_fill before the softmax."""
    Q, K, V, dO = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, do))
    UQ, UK, UV = (torch.tensor(x, dtype=torch.float64) for x in (uq, uk, uv))
    N = Q.shape[0]
    keep = torch.ones(N, N, dtype=torch.bool).tril()
    S = (tau * Q @ K.T).masked_fill(~keep, float("-inf"))
    P = torch.softmax(S, dim=-1)
    O = P @ V
    dQ, dK, dV = torch.autograd.grad(O, (Q, K, V), dO, create_graph=True)
    phi = (dQ * UQ).sum() + (dK * UK).sum() + (dV * UV).sum()
    g = torch.autograd.grad(phi, (Q, K, V, dO))
    return {"gQ": g[0].numpy(), "gK": g[1].numpy(), "gV": g[2].numpy(), "gdO": g[3].numpy(),
            "dQ": dQ.detach().numpy(), "dK": dK.detach().numpy(), "dV": dV.detach().numpy(),
            "O": O.detach().numpy(), "L": torch.logsumexp(S, dim=-1).detach().numpy(),
            "phi": float(phi.detach())}


@pytest.mark.parametrize("N,d,qk", [(1, 8, 1.0), (13, 8, 1.0), (37, 16, 1.0), (130, 64, 2.0), (64, 128, 1.0)])
def test_causal_bob_dense_matches_torch_double_backward(N, d, qk):
    t = head(N, d, 501 + N, qk=qk)
    tau = 1 / np.sqrt(d)
    ref = torch_bob_causal(*t, tau)
    out = bob_dense(*t, tau, causal=True)
    for key in ("O", "L", "dQ", "dK", "dV", *OUT_KEYS):
        assert relerr(out[key], ref[key]) < 1e-11, key
    assert abs(phi_dense(*t, tau, causal=True) - ref["phi"]) < 1e-10 * max(1, abs(ref["phi"]))


def test_causal_bob_central_fd_of_phi_13x8():
    """Elementwise central differences of the causal Phi."""
    N, d = 13, 8
    t = head(N, d, 521)
    tau = 1 / np.sqrt(d)
    out = bob_dense(*t, tau, causal=True)
    eps = 1e-6
    for idx, key in enumerate(("gQ", "gK", "gV", "gdO")):
        fd = np.zeros((N, d))
        for i in range(N):
            for a in range(d):
                p = [x.copy() for x in t]
                m = [x.copy() for x in t]
                p[idx][i, a] += eps
                m[idx][i, a] -= eps
                fd[i, a] = (phi_dense(*p, tau, causal=True) - phi_dense(*m, tau, causal=True)) / (2 * eps)
        assert np.max(np.abs(fd - out[key])) < 2e-8 * max(1.0, np.max(np.abs(fd))), key


def test_causal_first_row_and_last_row_closed_forms():
    """Row 0 attends only to key 0 (P = 1, dS = 0), so gQ_0 = 0 and
    gdO_0 = u_V,0 + (F_00 - alpha_0) v_0 = u_V,0; the last row sees every key,
    so its forward output equals the non-causal one."""
    N, d = 40, 16
    t = head(N, d, 531)
    tau = 1 / np.sqrt(d)
    c = bob_dense(*t, tau, causal=True)
    n = bob_dense(*t, tau)
    assert np.max(np.abs(c["gQ"][0])) < 1e-13
    assert np.max(np.abs(c["gdO"][0] - t[6][0])) < 1e-13
    assert np.max(np.abs(c["O"][-1] - n["O"][-1])) < 1e-13
    assert abs(c["L"][-1] - n["L"][-1]) < 1e-13


def test_causal_lower_bound_instance():
    """V = dO = U_Q = U_K = 0, U_V = W gives gdO = softmax(tau Q K^T + B_mask) W."""
    N, d = 33, 8
    q, k, _, _, _, _, w = head(N, d, 541)
    z = np.zeros((N, d))
    tau = 1 / np.sqrt(d)
    out = bob_dense(q, k, z, z, z, z, w, tau, causal=True)
    S = torch.tensor(q) @ torch.tensor(k).T * tau
    S = S.masked_fill(~torch.ones(N, N, dtype=torch.bool).tril(), float("-inf"))
    ref = torch.softmax(S, dim=-1).numpy() @ w
    assert relerr(out["gdO"], ref) < 1e-13
    for key in ("gQ", "gK", "gV"):
        assert np.max(np.abs(out[key])) == 0.0, key


@pytest.mark.parametrize("strip,chunk", [(1, 5), (7, 64), (64, 33), (None, 4096)])
def test_causal_streaming_matches_dense(strip, chunk):
    N, d = 150, 16
    t = head(N, d, 551)
    tau = 1 / np.sqrt(d)
    ref = bob_dense(*t, tau, causal=True)
    r = row_pass(*t, tau, outputs="all", strip=strip, col_chunk=chunk, causal=True)
    c = col_pass(*t, tau, r, strip=strip or 64, row_chunk=chunk, causal=True)
    for key in ("L", "O", "D", "alpha", "E", "gQ", "gdO", "dQ"):
        assert relerr(r[key], ref[key]) < 1e-12, key
    for key in ("gK", "gV", "dK", "dV"):
        assert relerr(c[key], ref[key]) < 1e-12, key


def test_causal_shift_invariance_column_sums():
    """Adding one vector to every key shifts each valid row of scores by a
    constant, so Phi is unchanged and sum_j gK_j = 0 under the mask too."""
    N, d = 90, 16
    t = head(N, d, 561)
    out = bob_dense(*t, 1 / np.sqrt(d), causal=True)
    assert np.max(np.abs(out["gK"].sum(axis=0))) < 1e-11 * max(1.0, np.max(np.abs(out["gK"])))
