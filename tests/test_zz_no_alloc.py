"""fa_bob_noalloc (the allocation-free variant of fa_bob, for callers that
cannot allocate device memory) through the C ABI: two calls in a row, the
second on a smaller problem, each compared with fa_bob on the same inputs.
Both entry points run the same kernels, so the outputs must agree bit for
bit (which is within the 2e-2 bar of every bf16 GPU result); the calls must
not allocate device memory."""
import numpy as np
import pytest

from fa_inputs import make_inputs
from tests.gpu_helpers import NAMES, host, rel, say, to_device

pytestmark = pytest.mark.gpu


def _case(B, H, Hkv, N, d, seed, causal, dropout=0.0):
    import torch

    import exact_second_order_fa_amd as fa

    say(f"no-alloc case B={B} H={H} H_kv={Hkv} N={N} d={d} causal={causal} dropout={dropout} seed={seed}")
    raw, _ = make_inputs(B, H, N, d, seed, "bf16", H_kv=Hkv)
    t = to_device(raw, "bf16")
    q, k, v, do, uq, uk, uv = (t[n] for n in NAMES)
    kw = dict(causal=causal, dropout=dropout, seed=seed)
    o, lse = fa.fa_fwd(q, k, v, **kw)
    ref = fa.fa_bob(q, k, v, o, lse, do, uq, uk, uv, **kw)[:4]
    outs = [torch.full(x.shape, float("nan"), dtype=torch.float32, device="cuda") for x in (q, k, k, q)]
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    got = fa.fa_bob_noalloc(q, k, v, o, lse, do, uq, uk, uv, *outs, **kw)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == base
    assert free0 - torch.cuda.mem_get_info()[0] <= 0
    for name, a, b in zip(("gQ", "gK", "gV", "gdO"), got, ref):
        e = rel(host(a), host(b))
        say(f"  {name} vs fa_bob: {e:.1e}, bitwise equal {bool(torch.equal(a, b))}")
        assert e <= 2e-2 and torch.equal(a, b), name


def test_noalloc_matches_fa_bob_twice_second_smaller():
    _case(2, 4, 2, 2000, 64, 41, False)  # row pass and column pass both split
    _case(1, 2, 2, 700, 128, 42, True)


def test_noalloc_with_dropout_twice_second_smaller():
    _case(1, 16, 16, 4000, 64, 43, False, 0.2)  # the two-wave dropout column pass
    _case(1, 2, 2, 700, 128, 44, True, 0.1)


def test_noalloc_refuses_a_problem_beyond_its_scratch():
    import torch

    import exact_second_order_fa_amd as fa

    B, H, N, d = 1, 16, 262144, 64
    x = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.fa_bob_noalloc(x, x, x, o, lse, x, x, x, x, o, o, o, o)
    assert e.value.status == 6
