"""Host-side argument checks of the Python binding (no GPU needed): the saved
forward state, caller-supplied outputs and workspaces are validated before
anything reaches the library, and a dropout rate that rounds to no dropout
says so.  The same checks on GPU tensors, through the public calls, are in
tests/test_gpu_parity.py::test_binding_rejects_bad_arguments_before_launch."""
import warnings

import pytest
import torch

import exact_second_order_fa_amd as fa


def q_like(B=1, H=2, N=8, d=64, dtype=torch.bfloat16):
    return torch.zeros(B, H, N, d, dtype=dtype)


def test_saved_state_checks():
    q = q_like()
    o = torch.zeros(q.shape, dtype=torch.float32)
    lse = torch.zeros(1, 2, 8, dtype=torch.float32)
    fa._check_saved_state(q, o, lse)
    bad = [
        (o.to(torch.bfloat16), lse),                  # O read as fp32 by the kernels
        (o[:, :1], lse),                              # wrong shape
        (o, lse.double()),                            # wrong dtype
        (o, lse[:, :, :4]),                           # wrong length
        (o, torch.zeros(1, 8, 2).permute(0, 2, 1)),   # not contiguous
        (o, torch.zeros(1, 2, 8, 1)),                 # extra dim
    ]
    for oo, ll in bad:
        with pytest.raises(ValueError):
            fa._check_saved_state(q, oo, ll)


def test_output_checks():
    q = q_like()
    out, new = fa._f32_like(q, None, "gq")
    assert new and out.dtype == torch.float32 and out.shape == q.shape
    same, new = fa._f32_like(q, out, "gq")
    assert same is out and not new
    for bad in (out.to(torch.bfloat16), out[:, :, :4], torch.zeros(1, 2, 8, 32)):
        with pytest.raises(ValueError):
            fa._f32_like(q, bad, "gq")


def test_workspace_checks():
    dev = torch.device("cpu")
    ws, new = fa._workspace(64, dev, None)
    assert new and ws.numel() * ws.element_size() >= 64
    ok, new = fa._workspace(64, dev, torch.zeros(16))
    assert not new
    with pytest.raises(ValueError):
        fa._workspace(64, dev, torch.zeros(15))                   # too small
    with pytest.raises(ValueError):
        fa._workspace(64, dev, torch.zeros(32, 2).t())            # not contiguous
    with pytest.raises(ValueError):
        fa._workspace(64, torch.device("meta"), torch.zeros(16))  # another device


def test_dropout_rate_rounding_warns():
    with pytest.warns(UserWarning, match="rounds to threshold 0"):
        fa.problem(1, 1, 8, 64, dropout=0.001)
    with warnings.catch_warnings():
        warnings.simplefilter("error")
        fa.problem(1, 1, 8, 64, dropout=0.0)
        fa.problem(1, 1, 8, 64, dropout=1.0 / 256)
