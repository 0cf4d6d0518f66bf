"""Host logic of sdpa_bob (exact_second_order_fa_amd/autograd.py) on the CPU.

The library calls are replaced by plain torch stand-ins (monkeypatched), so
only the wiring of the two autograd nodes is under test: which call receives
which tensors, that the gradients of (dQ, dK, dV) arrive as the cotangents
(U_Q, U_K, U_V), that nothing flows into O or L, dtype handling, and that a
third derivative is refused.  The numerics are checked on the GPU against
the oracle in tests/test_gpu_autograd.py.
"""
import pytest
import torch

import exact_second_order_fa_amd.autograd as ag

calls = []
drops = []  # (call, dropout, seed)


def fa_fwd(q, k, v, scale=None, causal=False, dropout=0.0, seed=0):
    calls.append(("fwd", q.dtype, causal))
    drops.append(("fwd", dropout, seed))
    return (q.float() * 2 + k.float() * 3 + v.float() * 5), q.float().sum(-1)


def fa_bwd(q, k, v, o, lse, do, scale=None, causal=False, dropout=0.0, seed=0):
    calls.append(("bwd", do.dtype, causal))
    drops.append(("bwd", dropout, seed))
    return do.float() * 7, do.float() * 11, do.float() * 13, None


def fa_bob(q, k, v, o, lse, do, uq, uk, uv, scale=None, causal=False, dropout=0.0, seed=0):
    calls.append(("bob", uq.dtype, uk.dtype, causal))
    drops.append(("bob", dropout, seed))
    return uq.float() * 17, uk.float() * 19, uv.float() * 23, uq.float() * 29 + uv.float() * 31, None


@pytest.fixture(autouse=True)
def standins(monkeypatch):
    monkeypatch.setattr(ag, "fa_fwd", fa_fwd)
    monkeypatch.setattr(ag, "fa_bwd", fa_bwd)
    monkeypatch.setattr(ag, "fa_bob", fa_bob)
    calls.clear()
    drops.clear()


def leaves(dtype=torch.float32, Hkv=2):
    g = torch.Generator().manual_seed(0)
    q = torch.randn(1, 2, 3, 4, generator=g).to(dtype).requires_grad_(True)
    k = torch.randn(1, Hkv, 3, 4, generator=g).to(dtype).requires_grad_(True)
    v = torch.randn(1, Hkv, 3, 4, generator=g).to(dtype).requires_grad_(True)
    return q, k, v


def test_first_and_second_order_wiring():
    q, k, v = leaves()
    W = torch.full((1, 2, 3, 4), 0.5)
    z = [torch.full_like(t, 1.0, dtype=torch.float32) for t in (q, k, v)]
    o = ag.sdpa_bob(q, k, v, causal=True)
    g = torch.autograd.grad((o * W).sum(), (q, k, v), create_graph=True)
    # first backward at dO = W
    assert torch.equal(g[0], W * 7) and torch.equal(g[1], W * 11) and torch.equal(g[2], W * 13)
    h = torch.autograd.grad(sum((gi * zi).sum() for gi, zi in zip(g, z)), (q, k, v))
    # second order: fa_bob with (U_Q, U_K, U_V) = z; dO = W is constant here, so gdO goes nowhere
    assert torch.equal(h[0], z[0] * 17) and torch.equal(h[1], z[1] * 19) and torch.equal(h[2], z[2] * 23)
    assert [c[0] for c in calls] == ["fwd", "bwd", "bob"] and all(c[-1] is True for c in calls)


def test_gdo_flows_into_the_loss_path():
    """L = |O|^2 / 2: dO = O depends on the inputs, so the BoB's gdO comes
    back through the first backward (a second fa_bwd call)."""
    q, k, v = leaves()
    o = ag.sdpa_bob(q, k, v)
    g = torch.autograd.grad(0.5 * (o * o).sum(), (q, k, v), create_graph=True)
    z = [torch.ones_like(t) for t in g]
    torch.autograd.grad(sum((gi * zi).sum() for gi, zi in zip(g, z)), (q, k, v))
    assert [c[0] for c in calls] == ["fwd", "bwd", "bob", "bwd"]


def test_bf16_inputs_get_do_and_cotangents_in_bf16():
    q, k, v = leaves(torch.bfloat16)
    o = ag.sdpa_bob(q, k, v)
    assert o.dtype == torch.float32
    g = torch.autograd.grad(o.sum(), (q, k, v), create_graph=True)
    assert all(x.dtype == torch.bfloat16 for x in g)  # autograd casts to the inputs' dtype
    h = torch.autograd.grad(sum(x.float().sum() for x in g), (q, k, v))
    assert calls[1] == ("bwd", torch.bfloat16, False)
    assert calls[2][:3] == ("bob", torch.bfloat16, torch.bfloat16)
    assert all(x.dtype == torch.bfloat16 for x in h)


def test_third_derivative_is_refused():
    q, k, v = leaves()
    o = ag.sdpa_bob(q, k, v)
    g = torch.autograd.grad(o.sum(), (q, k, v), create_graph=True)
    h = torch.autograd.grad(sum(x.sum() for x in g), (q, k, v), create_graph=True)
    with pytest.raises(RuntimeError, match="beyond the second"):
        torch.autograd.grad(sum(x.sum() for x in h), (q, k, v))


def test_rejects_non_contiguous_head_dim():
    q, k, v = leaves()
    with pytest.raises(ValueError):
        ag.sdpa_bob(q.transpose(2, 3), k, v)


def test_dropout_rate_and_seed_reach_every_call():
    """One mask for the forward, the first backward and the BoB: all three
    calls get the same (rate, seed)."""
    q, k, v = leaves()
    o = ag.sdpa_bob(q, k, v, dropout_p=0.25, seed=2 ** 40 + 3)
    g = torch.autograd.grad(0.5 * (o * o).sum(), (q, k, v), create_graph=True)
    torch.autograd.grad(sum(x.sum() for x in g), (q, k, v))
    assert [d[0] for d in drops] == ["fwd", "bwd", "bob", "bwd"]
    assert all(d[1:] == (0.25, 2 ** 40 + 3) for d in drops)
