"""Pins of the grouped-query / multi-query oracle (oracle/gqa.py).

The independent reference is float64 autograd on the CPU through an explicit
repetition of each K/V head G times (torch.repeat_interleave), so the sums
over a group come from the chain rule of the repetition, not from the
oracle's own grouping code.
"""
import numpy as np
import pytest
import torch

from oracle import bob_dense, bob_dense_gqa, bob_streaming_gqa

KEYS_Q = ("O", "L", "dQ", "gQ", "gdO")
KEYS_KV = ("dK", "dV", "gK", "gV")


def heads(Hq, Hkv, N, d, seed):
    r = np.random.default_rng(seed)
    q, do, uq = (r.standard_normal((Hq, N, d)) for _ in range(3))
    k, v, uk, uv = (r.standard_normal((Hkv, N, d)) for _ in range(4))
    return q, k, v, do, uq, uk, uv


def torch_bob_gqa(q, k, v, do, uq, uk, uv, tau, causal):
    G = q.shape[0] // k.shape[0]
    Q, K, V, dO = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, do))
    UQ, UK, UV = (torch.tensor(x, dtype=torch.float64) for x in (uq, uk, uv))
    Ke, Ve = K.repeat_interleave(G, dim=0), V.repeat_interleave(G, dim=0)
    S = tau * Q @ Ke.transpose(1, 2)
    if causal:
        N = q.shape[1]
        S = S.masked_fill(~torch.ones(N, N, dtype=torch.bool).tril(), float("-inf"))
    P = torch.softmax(S, dim=-1)
    O = P @ Ve
    dQ, dK, dV = torch.autograd.grad(O, (Q, K, V), dO, create_graph=True)
    phi = (dQ * UQ).sum() + (dK * UK).sum() + (dV * UV).sum()
    g = torch.autograd.grad(phi, (Q, K, V, dO))
    return {"gQ": g[0].numpy(), "gK": g[1].numpy(), "gV": g[2].numpy(), "gdO": g[3].numpy(),
            "dQ": dQ.detach().numpy(), "dK": dK.detach().numpy(), "dV": dV.detach().numpy(),
            "O": O.detach().numpy(), "L": torch.logsumexp(S, dim=-1).detach().numpy()}


def relerr(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-2))


@pytest.mark.parametrize("Hq,Hkv,N,d,causal", [(4, 1, 23, 8, False), (4, 2, 23, 8, True), (6, 3, 17, 16, False),
                                                (8, 1, 40, 8, True)])
def test_gqa_dense_matches_torch_repeat_interleave(Hq, Hkv, N, d, causal):
    t = heads(Hq, Hkv, N, d, 900 + Hq + Hkv + N)
    tau = 1 / np.sqrt(d)
    ref = torch_bob_gqa(*t, tau, causal)
    out = bob_dense_gqa(*t, tau, causal)
    for key in KEYS_Q + KEYS_KV:
        assert out[key].shape == ref[key].shape, key
        assert relerr(out[key], ref[key]) < 1e-11, key


def test_gqa_with_one_query_head_per_group_is_multi_head():
    t = heads(3, 3, 19, 8, 911)
    out = bob_dense_gqa(*t, 0.4)
    for h in range(3):
        ref = bob_dense(*(x[h] for x in t), 0.4)
        for key in KEYS_Q + KEYS_KV:
            assert np.array_equal(out[key][h], ref[key]), key


def test_gqa_rejects_non_multiple_head_counts():
    t = heads(3, 2, 5, 8, 912)
    with pytest.raises(ValueError):
        bob_dense_gqa(*t, 0.4)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_streaming_matches_dense(causal):
    B, Hq, Hkv, N, d = 2, 4, 2, 37, 8
    r = np.random.default_rng(913)
    q, do, uq = (r.standard_normal((B, Hq, N, d)) for _ in range(3))
    k, v, uk, uv = (r.standard_normal((B, Hkv, N, d)) for _ in range(4))
    out = bob_streaming_gqa(q, k, v, do, uq, uk, uv, 0.35, threads=2, strip=8, col_chunk=10, causal=causal)
    for b in range(B):
        ref = bob_dense_gqa(q[b], k[b], v[b], do[b], uq[b], uk[b], uv[b], 0.35, causal)
        for key in KEYS_Q + KEYS_KV + ("D", "alpha", "E"):
            assert relerr(out[key][b], ref[key]) < 1e-12, (b, key)
