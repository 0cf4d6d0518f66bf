"""Pins of the dropout oracle (``oracle/dropout.py``) against things other than
itself: numpy's Philox4x64-10 bit generator (the mask's generator), the
binomial keep rate, torch float64 autograd double backward of attention with
a fixed mask, central finite differences of Phi, and the reduction to the
dropout-free oracle at p = 0."""
import numpy as np
import pytest
import torch

from oracle import (backward_dropout, bob_dense, bob_dropout, bob_dropout_heads, dropout_mask, keep_bytes,
                    philox4x64_10, phi_dropout, threshold)

OUT_KEYS = ("gQ", "gK", "gV", "gdO")


def head(N, d, seed):
    r = np.random.default_rng(seed)
    return [r.standard_normal((N, d)) for _ in range(7)]  # q, k, v, do, uq, uk, uv


def numpy_block(c, key):
    """numpy's Philox4x64-10 output block for 256-bit counter c (four words,
    least significant first): the generator increments its counter before
    each block, so it starts one below."""
    ctr = sum(int(w) << (64 * i) for i, w in enumerate(c)) - 1
    bg = np.random.Philox(counter=ctr, key=np.array(key, dtype=np.uint64))
    return [int(x) for x in bg.random_raw(4)]


def test_philox_block_matches_numpy():
    r = np.random.default_rng(5)
    for _ in range(40):
        c = [int(x) for x in r.integers(0, 2 ** 63, size=4, dtype=np.uint64)]
        c[0] |= 1
        key = [int(x) for x in r.integers(0, 2 ** 63, size=2, dtype=np.uint64)]
        got = philox4x64_10(*[np.uint64(x) for x in c], np.uint64(key[0]), np.uint64(key[1]))
        assert [int(x) for x in got] == numpy_block(c, key)
    # vectorised over counters
    c0 = np.arange(1, 9, dtype=np.uint64)
    got = philox4x64_10(c0, np.uint64(3), np.uint64(4), np.uint64(0), np.uint64(77), np.uint64(0))
    for n in range(8):
        assert [int(w[n]) for w in got] == numpy_block([n + 1, 3, 4, 0], [77, 0])


def test_keep_byte_layout():
    """Byte of element (i, j) = byte j % 8 of word i % 4 of the block for
    counter (i // 4, j // 8, bh, 0), key (seed, 0), checked against numpy's
    generator element by element."""
    N, bh, seed = 37, 5, 2024
    kb = keep_bytes(bh, N, seed)
    r = np.random.default_rng(1)
    for _ in range(60):
        i, j = (int(x) for x in r.integers(0, N, size=2))
        if i < 4 and j < 8:  # counter 0 cannot be reached from one below in numpy's generator
            continue
        block = numpy_block([i // 4, j // 8, bh, 0], [seed, 0])
        assert kb[i, j] == (block[i % 4] >> (8 * (j % 8))) & 0xFF, (i, j)


def test_threshold_and_keep_rate():
    assert threshold(0.0) == (0, 1.0)
    assert threshold(0.25) == (64, 256 / 192)
    assert threshold(0.1)[0] == 26  # round(25.6)
    with pytest.raises(ValueError):
        threshold(0.999)
    g = dropout_mask(3, 512, 0.25, 11)
    kept = g > 0
    assert set(np.unique(g)) == {0.0, 256 / 192}
    n = kept.size
    # binomial: keep probability 192/256, five standard deviations
    assert abs(kept.mean() - 0.75) < 5 * np.sqrt(0.75 * 0.25 / n)
    # E[g] = 1
    assert abs(g.mean() - 1.0) < 5 * np.sqrt(0.75 * 0.25 / n) * 256 / 192
    # heads and seeds draw different masks
    assert (dropout_mask(4, 64, 0.25, 11) != dropout_mask(3, 64, 0.25, 11)).any()
    assert (dropout_mask(3, 64, 0.25, 12) != dropout_mask(3, 64, 0.25, 11)).any()


def test_p_zero_reduces_to_the_dropout_free_oracle():
    t = head(40, 16, 3)
    tau = 0.25
    g = dropout_mask(0, 40, 0.0, 9)
    assert (g == 1).all()
    a, b = bob_dropout(*t, tau, g), bob_dense(*t, tau)
    for key in OUT_KEYS + ("alpha", "E", "O", "L", "D"):
        assert np.max(np.abs(a[key] - b[key])) < 1e-12 * max(1, np.max(np.abs(b[key]))), key


def torch_bob_dropout(q, k, v, do, uq, uk, uv, tau, g, causal):
    """float64 autograd double backward of O = (softmax(S) * g) V on the CPU."""
    Q, K, V, dO = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, do))
    UQ, UK, UV, Gm = (torch.tensor(x, dtype=torch.float64) for x in (uq, uk, uv, g))
    S = tau * Q @ K.T
    if causal:
        S = S.masked_fill(torch.triu(torch.ones_like(S, dtype=torch.bool), 1), float("-inf"))
    O = (torch.softmax(S, dim=-1) * Gm) @ V
    dQ, dK, dV = torch.autograd.grad(O, (Q, K, V), dO, create_graph=True)
    phi = (dQ * UQ).sum() + (dK * UK).sum() + (dV * UV).sum()
    gr = torch.autograd.grad(phi, (Q, K, V, dO))
    return {"gQ": gr[0].numpy(), "gK": gr[1].numpy(), "gV": gr[2].numpy(), "gdO": gr[3].numpy(),
            "dQ": dQ.detach().numpy(), "dK": dK.detach().numpy(), "dV": dV.detach().numpy(), "O": O.detach().numpy()}


@pytest.mark.parametrize("N,d,p,causal", [(1, 8, 0.5, False), (37, 8, 0.1, False), (64, 32, 0.3, True),
                                          (130, 64, 0.5, False), (96, 16, 0.9, True)])
def test_dropout_bob_matches_torch_double_backward(N, d, p, causal):
    t = head(N, d, 50 + N)
    tau = 1 / np.sqrt(d)
    g = dropout_mask(7, N, p, 123)
    ref = torch_bob_dropout(*t, tau, g, causal)
    out = bob_dropout(*t, tau, g, causal)
    for key in OUT_KEYS + ("dQ", "dK", "dV", "O"):
        scale = max(np.max(np.abs(ref[key])), 1e-2)
        assert np.max(np.abs(out[key] - ref[key])) < 1e-11 * scale, key
    assert np.max(np.abs(out["D"] - out["D_from_P"])) < 1e-12 * max(1, np.max(np.abs(out["D"])))


def test_dropout_bob_central_fd_of_phi():
    """Every entry of gQ, gK, gV, gdO against central differences of the
    dropout Phi (mask fixed)."""
    N, d = 12, 6
    t = head(N, d, 77)
    tau = 0.4
    g = dropout_mask(1, N, 0.3, 5)
    out = bob_dropout(*t, tau, g)
    eps = 1e-6
    for idx, key in enumerate(OUT_KEYS):
        fd = np.zeros((N, d))
        for i in range(N):
            for a in range(d):
                pp = [x.copy() for x in t]
                mm = [x.copy() for x in t]
                pp[idx][i, a] += eps
                mm[idx][i, a] -= eps
                fd[i, a] = (phi_dropout(*pp, tau, g) - phi_dropout(*mm, tau, g)) / (2 * eps)
        assert np.max(np.abs(fd - out[key])) < 2e-8 * max(1.0, np.max(np.abs(fd))), key


def test_dropout_first_backward_linear_in_do_and_bob_linear_in_cotangents():
    t = head(20, 8, 9)
    tau = 0.3
    g = dropout_mask(2, 20, 0.2, 4)
    b1 = backward_dropout(t[0], t[1], t[2], t[3], tau, g)
    b2 = backward_dropout(t[0], t[1], t[2], 2.5 * t[3], tau, g)
    for key in ("dQ", "dK", "dV"):
        assert np.allclose(b2[key], 2.5 * b1[key], rtol=1e-12, atol=1e-12)
    o1 = bob_dropout(*t, tau, g)
    o2 = bob_dropout(*t[:4], *(3.0 * x for x in t[4:]), tau, g)
    for key in OUT_KEYS:
        assert np.allclose(o2[key], 3.0 * o1[key], rtol=1e-11, atol=1e-11)


def test_heads_helper_sums_key_side_over_groups():
    r = np.random.default_rng(8)
    B, H, Hkv, N, d = 1, 4, 2, 24, 8
    qs = [r.standard_normal((B, H, N, d)) for _ in range(3)]
    ks = [r.standard_normal((B, Hkv, N, d)) for _ in range(4)]
    q, do, uq = qs
    k, v, uk, uv = ks
    out = bob_dropout_heads(q, k, v, do, uq, uk, uv, 0.3, 0.25, 99)
    gk = np.zeros((N, d))
    for h in (2, 3):
        g = dropout_mask(h, N, 0.25, 99)
        gk += bob_dropout(q[0, h], k[0, 1], v[0, 1], do[0, h], uq[0, h], uk[0, 1], uv[0, 1], 0.3, g)["gK"]
    assert np.allclose(out["gK"][0, 1], gk, rtol=1e-13, atol=1e-13)
