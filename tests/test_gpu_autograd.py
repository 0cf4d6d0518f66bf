"""sdpa_bob (exact_second_order_fa_amd/autograd.py): softmax attention
differentiated twice through the library, against the float64 oracle.

Hessian-vector products through one attention layer, H z = d/dx <dL/dx, z>
for x = (Q, K, V):

* linear loss L = <O, W>: the first gradient is the first backward at dO = W,
  so H z is exactly the backward-over-backward with (U_Q, U_K, U_V) = z
  ([FlashBoB] section 4.1): oracle ``bob_dense`` at dO = W;
* quadratic loss L = |O|^2 / 2: dO = O depends on x, so H z adds the first
  backward applied to the BoB's gdO: oracle ``bob_dense`` at dO = O plus
  ``backward_dense`` at dO = gdO.

bf16 inputs use W and z that are exactly representable in bf16 (the library
takes dO and the cotangents in the input dtype), so both sides see the same
values.  Tolerances as everywhere: 2e-2 (bf16), 1e-4 (fp32), max-abs-error
over max-abs-reference per tensor.
"""
import numpy as np
import pytest

from fa_inputs import make_inputs
from oracle import backward_dense, bob_dense, bob_dense_gqa, bob_dropout, dropout_mask, forward_dense
from tests.gpu_helpers import host, rel, say

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "fp32": 1e-4}


def tensors(raw, dtype, names, grad):
    import torch

    out = []
    for n in names:
        x = raw[n]
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16) if dtype == "bf16" \
            else torch.from_numpy(np.ascontiguousarray(x))
        t = t.cuda()
        if grad:
            t.requires_grad_(True)
        out.append(t)
    return out


def hvp(q, k, v, loss, z, causal, dropout_p=0.0, seed=0):
    import torch

    from exact_second_order_fa_amd.autograd import sdpa_bob

    o = sdpa_bob(q, k, v, causal=causal, dropout_p=dropout_p, seed=seed)
    g = torch.autograd.grad(loss(o), (q, k, v), create_graph=True)
    s = sum((gi.float() * zi).sum() for gi, zi in zip(g, z))
    h = torch.autograd.grad(s, (q, k, v))
    torch.cuda.synchronize()
    return o, g, h


@pytest.mark.parametrize("dtype,causal", [("fp32", False), ("fp32", True), ("bf16", False), ("bf16", True)])
def test_hvp_linear_loss(dtype, causal):
    B, H, N, d = 1, 2, 100, 64
    say(f"hvp linear loss {dtype} causal={causal}")
    raw, f64 = make_inputs(B, H, N, d, 1100 + causal, dtype)
    q, k, v = tensors(raw, dtype, ("q", "k", "v"), True)
    W, zq, zk, zv = (t.float() for t in tensors(raw, dtype, ("do", "uq", "uk", "uv"), False))
    o, g, h = hvp(q, k, v, lambda o: (o * W).sum(), (zq, zk, zv), causal)
    tau = 1 / np.sqrt(d)
    for b in range(B):
        for hh in range(H):
            ref = bob_dense(*(f64[n][b, hh] for n in ("q", "k", "v", "do", "uq", "uk", "uv")), tau, causal=causal)
            errs = {"O": rel(host(o[b, hh]), ref["O"])}
            for i, key in enumerate(("dQ", "dK", "dV")):
                errs[key] = rel(host(g[i][b, hh]), ref[key])
            for i, key in enumerate(("gQ", "gK", "gV")):
                errs["H z " + key[1]] = rel(host(h[i][b, hh]), ref[key])
            say("  " + " ".join(f"{k_}={v_:.1e}" for k_, v_ in errs.items()))
            assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("dtype,causal", [("fp32", False), ("bf16", True)])
def test_hvp_linear_loss_with_dropout(dtype, causal):
    """With dropout the HVP of L = <O, W> is the BoB of the dropout backward
    (oracle ``bob_dropout`` with the same Philox mask)."""
    B, H, N, d, p, seed = 1, 2, 100, 64, 0.2, 4242
    say(f"hvp linear loss with dropout {dtype} causal={causal}")
    raw, f64 = make_inputs(B, H, N, d, 1130 + causal, dtype)
    q, k, v = tensors(raw, dtype, ("q", "k", "v"), True)
    W, zq, zk, zv = (t.float() for t in tensors(raw, dtype, ("do", "uq", "uk", "uv"), False))
    o, g, h = hvp(q, k, v, lambda o: (o * W).sum(), (zq, zk, zv), causal, dropout_p=p, seed=seed)
    tau = 1 / np.sqrt(d)
    for hh in range(H):
        gm = dropout_mask(hh, N, p, seed)
        ref = bob_dropout(*(f64[n][0, hh] for n in ("q", "k", "v", "do", "uq", "uk", "uv")), tau, gm, causal=causal)
        errs = {"O": rel(host(o[0, hh]), ref["O"])}
        for i, key in enumerate(("dQ", "dK", "dV")):
            errs[key] = rel(host(g[i][0, hh]), ref[key])
        for i, key in enumerate(("gQ", "gK", "gV")):
            errs["H z " + key[1]] = rel(host(h[i][0, hh]), ref[key])
        say("  " + " ".join(f"{k_}={v_:.1e}" for k_, v_ in errs.items()))
        assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("causal", [False, True])
def test_hvp_quadratic_loss_fp32(causal):
    B, H, N, d = 1, 2, 90, 64
    say(f"hvp quadratic loss fp32 causal={causal}")
    raw, f64 = make_inputs(B, H, N, d, 1110 + causal, "fp32")
    q, k, v = tensors(raw, "fp32", ("q", "k", "v"), True)
    zq, zk, zv = tensors(raw, "fp32", ("uq", "uk", "uv"), False)
    _, _, h = hvp(q, k, v, lambda o: 0.5 * (o * o).sum(), (zq, zk, zv), causal)
    tau = 1 / np.sqrt(d)
    for hh in range(H):
        x = {n: f64[n][0, hh] for n in ("q", "k", "v", "uq", "uk", "uv")}
        O = forward_dense(x["q"], x["k"], x["v"], tau, causal)["O"]
        r = bob_dense(x["q"], x["k"], x["v"], O, x["uq"], x["uk"], x["uv"], tau, causal=causal)
        b2 = backward_dense(x["q"], x["k"], x["v"], r["gdO"], tau, causal)
        for i, (gk_, dk_) in enumerate((("gQ", "dQ"), ("gK", "dK"), ("gV", "dV"))):
            e = rel(host(h[i][0, hh]), r[gk_] + b2[dk_])
            say(f"  head {hh} H z {gk_[1]} {e:.1e}")
            assert e <= TOL["fp32"], (hh, gk_)


def test_hvp_grouped_query_bf16():
    B, H, Hkv, N, d = 1, 4, 1, 120, 64
    say("hvp linear loss, multi-query bf16")
    raw, f64 = make_inputs(B, H, N, d, 1120, "bf16", H_kv=Hkv)
    q, k, v = tensors(raw, "bf16", ("q", "k", "v"), True)
    W, zq, zk, zv = (t.float() for t in tensors(raw, "bf16", ("do", "uq", "uk", "uv"), False))
    _, _, h = hvp(q, k, v, lambda o: (o * W).sum(), (zq, zk, zv), False)
    ref = bob_dense_gqa(*(f64[n][0] for n in ("q", "k", "v", "do", "uq", "uk", "uv")), 1 / np.sqrt(d))
    assert tuple(h[1].shape) == (B, Hkv, N, d)
    for i, key in enumerate(("gQ", "gK", "gV")):
        e = rel(host(h[i][0]), ref[key])
        say(f"  H z {key[1]} {e:.1e}")
        assert e <= TOL["bf16"], key


def test_third_derivative_is_refused():
    import torch

    from exact_second_order_fa_amd.autograd import sdpa_bob

    raw, _ = make_inputs(1, 1, 40, 64, 1130, "fp32")
    q, k, v = tensors(raw, "fp32", ("q", "k", "v"), True)
    o = sdpa_bob(q, k, v)
    g = torch.autograd.grad(o.sum(), (q, k, v), create_graph=True)
    h = torch.autograd.grad(sum(x.sum() for x in g), (q, k, v), create_graph=True)
    with pytest.raises(RuntimeError):
        torch.autograd.grad(sum(x.sum() for x in h), (q, k, v))
