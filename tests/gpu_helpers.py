"""Shared helpers of the GPU parity tests (device tensors from the seeded
inputs, one call of every entry point, error metrics)."""
from __future__ import annotations

import os
import sys

import numpy as np

NAMES = ("q", "k", "v", "do", "uq", "uk", "uv")


def say(msg):
    """Print and flush, so a run that dies still names the case it was on."""
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_threads():
    return max(1, min(16, os.cpu_count() or 1))


def to_device(raw, dtype, layout="bhnd"):
    """Device tensors [B, H, N, d] from the generator's arrays.  layout
    "bnhd" stores them as [B, N, H, d] and returns permuted (strided) views."""
    import torch

    out = {}
    for k, v in raw.items():
        if dtype == "bf16":
            t = torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(v))
        if layout == "bnhd":
            t = t.permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3)
        else:
            t = t.cuda()
        out[k] = t
    return out


def run_path(t, scale=None, with_bwd=True, layout="bhnd", causal=False, schedule=None):
    """fa_fwd, fa_bwd (optional) and fa_bob on device tensors; returns torch
    tensors on the GPU."""
    import torch

    import exact_second_order_fa_amd as fa

    def empty_like_out(x):
        if layout == "bnhd":
            B, H, N, d = x.shape
            return torch.empty((B, N, H, d), dtype=torch.float32, device=x.device).permute(0, 2, 1, 3)
        return torch.empty(x.shape, dtype=torch.float32, device=x.device)

    o, lse = fa.fa_fwd(t["q"], t["k"], t["v"], scale=scale, o=empty_like_out(t["q"]), causal=causal)
    res = {"O": o, "L": lse}
    if with_bwd:
        dq, dk, dv, _ = fa.fa_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], scale=scale,
                                  dq=empty_like_out(t["q"]), dk=empty_like_out(t["k"]),
                                  dv=empty_like_out(t["k"]), causal=causal)
        res.update(dQ=dq, dK=dk, dV=dv)
    outs = [empty_like_out(t[n]) for n in ("q", "k", "k", "q")]  # gQ, gK, gV, gdO
    gq, gk, gv, gdo, ws = fa.fa_bob(t["q"], t["k"], t["v"], o, lse, t["do"], t["uq"], t["uk"], t["uv"],
                                    scale=scale, gq=outs[0], gk=outs[1], gv=outs[2], gdo=outs[3],
                                    causal=causal, schedule=schedule)
    B, H, N, _ = t["q"].shape
    D, alpha, E = fa.split_workspace(ws, B, H, N)
    res.update(gQ=gq, gK=gk, gV=gv, gdO=gdo, D=D, alpha=alpha, E=E)
    torch.cuda.synchronize()
    return res


def run_dropout(t, p, seed, causal):
    """fa_fwd, fa_bwd and fa_bob with dropout rate p and generator key seed."""
    import torch

    import exact_second_order_fa_amd as fa

    kw = dict(causal=causal, dropout=p, seed=seed)
    o, lse = fa.fa_fwd(t["q"], t["k"], t["v"], **kw)
    dq, dk, dv, _ = fa.fa_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], **kw)
    gq, gk, gv, gdo, ws = fa.fa_bob(t["q"], t["k"], t["v"], o, lse, t["do"], t["uq"], t["uk"], t["uv"], **kw)
    B, H, N, _ = t["q"].shape
    D, alpha, E = fa.split_workspace(ws, B, H, N)
    torch.cuda.synchronize()
    return dict(O=o, L=lse, dQ=dq, dK=dk, dV=dv, D=D, alpha=alpha, E=E, gQ=gq, gK=gk, gV=gv, gdO=gdo)


def rel(got, ref):
    """max |got - ref| / max |ref| (all-zero references compare absolutely)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def host(x):
    return x.detach().double().cpu().numpy()
