"""Parity of the HIP path (through the C ABI) with the float64 CPU oracle.

Tolerance (per output tensor, whole tensor): max |gpu - oracle| / max |oracle|
<= 2e-2 for bf16 inputs and <= 1e-4 for fp32 inputs.  The same bar is applied
to the forward (O, L), the first backward (dQ, dK, dV) and the row scalars
(D, alpha, E) the BoB path writes to its workspace.

Small cases (several tiles and a ragged tail, ragged and degenerate N,
strided layouts, non power-of-two scales) compare every element with the
dense oracle.  The full-size workloads are in test_gpu_workloads.py.
"""
import numpy as np
import pytest

from fa_inputs import bf16_bits_to_f32, f32_to_bf16_bits, make_inputs
from oracle import bob_dense, bob_dense_gqa
from tests.gpu_helpers import NAMES, host, rel, run_path, say, to_device

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "fp32": 1e-4}
ALL = ("O", "L", "dQ", "dK", "dV", "D", "alpha", "E", "gQ", "gK", "gV", "gdO")


def oracle_heads(f64, scale, causal=False):
    B, H = f64["q"].shape[:2]
    out = {}
    for b in range(B):
        for h in range(H):
            r = bob_dense(*(f64[n][b, h] for n in NAMES), scale, causal=causal)
            for key in ALL:
                out.setdefault(key, np.zeros((B, H) + r[key].shape))[b, h] = r[key]
    return out


def check_case(B, H, N, d, dtype, seed, scale=None, qk=1.0, cot=1.0, layout="bhnd", causal=False, schedule=None,
               shape_inputs=None):
    say(f"case B={B} H={H} N={N} d={d} {dtype} seed={seed} scale={scale} layout={layout} causal={causal} "
        f"schedule={schedule}")
    raw, f64 = make_inputs(B, H, N, d, seed, dtype, cot_std=cot, qk_gain=qk)
    if shape_inputs is not None:
        shape_inputs(raw, f64)
    tau = scale if scale is not None else 1.0 / np.sqrt(d)
    got = run_path(to_device(raw, dtype, layout), scale=scale, layout=layout, causal=causal, schedule=schedule)
    ref = oracle_heads(f64, tau, causal)
    errs = {k: rel(host(got[k]), ref[k]) for k in ALL}
    say("  " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL[dtype]}
    assert not bad, bad
    return got


def test_tiny_fp32_workload():
    """B=1, H=1, N=128, d=64, fp32 inputs, seed 0, tolerance 1e-4."""
    check_case(1, 1, 128, 64, "fp32", 0)


@pytest.mark.parametrize("B,H,N,d", [
    (1, 2, 100, 64),   # one ragged tile
    (1, 1, 37, 64),    # ragged, smaller than a sub-tile
    (2, 3, 130, 64),   # several heads, ragged resident block
    (1, 1, 640, 64),   # ten streamed tiles
    (1, 2, 300, 128),  # d = 128 (tau not a power of two)
    (1, 1, 257, 128),
])
def test_bf16_shapes(B, H, N, d):
    check_case(B, H, N, d, "bf16", 100 + N + d)


def test_single_key_degenerate():
    """N = 1: P = 1 and dS = 0 exactly, so dQ, dK, gQ, gK are exactly 0 in the
    oracle and a relative error is undefined for them.  They are held to the
    bf16 bar relative to the size of the terms that cancel in them
    (tau |do| |u_V| |k|-sized products); every other output uses the usual
    relative bar."""
    for d in (64, 128):
        raw, f64 = make_inputs(1, 2, 1, d, 401 + d, "bf16")
        tau = 1.0 / np.sqrt(d)
        got = run_path(to_device(raw, "bf16"))
        ref = oracle_heads(f64, tau)
        m = {n: np.max(np.abs(f64[n])) for n in NAMES}
        terms = tau * (m["do"] * (m["uv"] + m["v"]) + m["uq"] * m["k"] + m["q"] * m["uk"]) * max(
            m["k"], m["uk"], m["q"], m["uq"])
        for key in ALL:
            if np.max(np.abs(ref[key])) == 0.0:
                assert np.max(np.abs(host(got[key]))) <= 2e-2 * terms, key
            else:
                assert rel(host(got[key]), ref[key]) <= 2e-2, key


@pytest.mark.parametrize("B,H,N", [(1, 1, 257), (2, 1, 70)])
def test_fp32_shapes(B, H, N):
    check_case(B, H, N, 64, "fp32", 200 + N)


def test_custom_scale_bf16():
    """A scale that is not a power of two at d = 64 (rho != 1 path); at
    N = 700 the row pass also splits each block's keys into two ranges (and
    the column pass each head's rows), at d = 64 and d = 128."""
    check_case(1, 2, 200, 64, "bf16", 301, scale=0.1)
    check_case(1, 2, 700, 64, "bf16", 310, scale=0.1)
    check_case(1, 2, 700, 128, "bf16", 311, scale=0.1)


def test_custom_scale_fp32():
    check_case(1, 1, 150, 64, "fp32", 302, scale=0.3)


def test_peaked_rows():
    """Q, K scaled by 2 (peaked softmax rows) and small cotangents."""
    check_case(1, 2, 512, 64, "bf16", 303, qk=2.0, cot=0.1)
    check_case(1, 1, 256, 128, "bf16", 304, qk=2.0, cot=0.1)


def _rising_keys(raw, f64):
    """Key norms growing tenfold along the sequence, so that the row maxima
    keep rising (the reference maximum of the forward moves about twice per
    row besides the first tile), and key 900 of every head set along q_950
    with norm 64: row 950's score on it is about 40 above every other one
    (natural log), far beyond the 2^16 factor the forward accepts against an
    earlier maximum, so its reference maximum has to jump.  Values are
    rounded to bf16 for both sides."""
    k = f64["k"].copy()
    n = k.shape[2]
    k *= (1.0 + 9.0 * np.arange(n) / n)[None, None, :, None]
    q950 = f64["q"][:, :, 950]
    k[:, :, 900] = 64.0 * q950 / np.linalg.norm(q950, axis=-1, keepdims=True)
    bits = f32_to_bf16_bits(k.astype(np.float32))
    raw["k"] = bits
    f64["k"] = bf16_bits_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("causal", [False, True])
def test_rising_scores_move_the_reference_maximum(causal):
    """Rising scores and one late outlier (see _rising_keys), N = 1000 (eight
    key tiles with a ragged one), d = 64: every output against the oracle."""
    check_case(1, 2, 1000, 64, "bf16", 309, causal=causal, shape_inputs=_rising_keys)


def test_strided_layout():
    """Inputs and outputs stored [B, N, H, d] (non-contiguous head stride); at
    N = 700 the row pass's key split and the column pass's row split write
    their results through the same strides."""
    check_case(2, 3, 150, 64, "bf16", 305, layout="bnhd")
    check_case(1, 2, 90, 128, "bf16", 306, layout="bnhd")
    check_case(1, 2, 700, 64, "bf16", 312, layout="bnhd")
    check_case(1, 2, 700, 128, "bf16", 313, layout="bnhd")


def test_deterministic():
    """No atomics: two runs are bitwise identical."""
    raw, _ = make_inputs(1, 2, 333, 64, 307, "bf16")
    t = to_device(raw, "bf16")
    a = run_path(t)
    b = run_path(t)
    for key in ("O", "L", "dQ", "dK", "dV", "gQ", "gK", "gV", "gdO", "alpha", "E"):
        assert bool((a[key] == b[key]).all()), key


# ---------------------------------------------------------------- causal attention


@pytest.mark.parametrize("B,H,N,d", [
    (1, 2, 100, 64),   # ragged, one tile
    (1, 1, 37, 64),
    (2, 1, 300, 64),   # diagonal tiles inside several row blocks
    (1, 1, 640, 64),   # full tiles below the diagonal
    (1, 2, 300, 128),
    (1, 1, 513, 128),
])
def test_causal_bf16_shapes(B, H, N, d):
    check_case(B, H, N, d, "bf16", 700 + N + d, causal=True)


def test_causal_fp32():
    check_case(1, 1, 200, 64, "fp32", 710, causal=True)


def test_causal_strided_and_scaled():
    check_case(1, 2, 260, 64, "bf16", 711, layout="bnhd", causal=True)
    check_case(1, 1, 150, 64, "bf16", 712, scale=0.1, causal=True)


def test_causal_deterministic():
    raw, _ = make_inputs(1, 2, 333, 64, 713, "bf16")
    t = to_device(raw, "bf16")
    a = run_path(t, causal=True)
    b = run_path(t, causal=True)
    for key in ("O", "L", "dQ", "dK", "dV", "gQ", "gK", "gV", "gdO", "alpha", "E"):
        assert bool((a[key] == b[key]).all()), key


# ---------------------------------------------------------------- grouped-query / multi-query attention

KV_KEYS = ("dK", "dV", "gK", "gV")


def check_case_gqa(B, H, Hkv, N, d, dtype, seed, causal=False, layout="bhnd", scale=None, schedule=None):
    """K, V, U_K, U_V with Hkv heads shared by groups of H / Hkv query heads,
    against the grouped-query oracle (key-side outputs summed over each group)."""
    say(f"case GQA B={B} H={H} Hkv={Hkv} N={N} d={d} {dtype} seed={seed} causal={causal} layout={layout}")
    raw, f64 = make_inputs(B, H, N, d, seed, dtype, H_kv=Hkv)
    tau = scale if scale is not None else 1.0 / np.sqrt(d)
    got = run_path(to_device(raw, dtype, layout), scale=scale, layout=layout, causal=causal, schedule=schedule)
    ref = {}
    for b in range(B):
        r = bob_dense_gqa(*(f64[n][b] for n in NAMES), tau, causal)
        for key in ALL:
            ref.setdefault(key, np.zeros((B,) + r[key].shape))[b] = r[key]
    for key in KV_KEYS:
        assert tuple(got[key].shape) == (B, Hkv, N, d), key
    errs = {k: rel(host(got[k]), ref[k]) for k in ALL}
    say("  " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL[dtype]}
    assert not bad, bad
    return got


@pytest.mark.parametrize("B,H,Hkv,N,d,causal", [
    (1, 4, 1, 100, 64, False),   # MQA, ragged single tile
    (2, 6, 2, 130, 64, True),    # GQA, causal, ragged resident block
    (1, 2, 1, 640, 64, False),   # ten streamed tiles per query head, crossing a head boundary
    (1, 8, 2, 300, 128, False),  # d = 128
    (1, 4, 2, 257, 128, True),
    (1, 3, 3, 70, 64, False),    # H_kv = H (multi-head through the grouped path)
    (1, 8, 1, 600, 128, False),  # MQA, d = 128, column pass split over heads and two row ranges
])
def test_gqa_bf16_shapes(B, H, Hkv, N, d, causal):
    check_case_gqa(B, H, Hkv, N, d, "bf16", 800 + H + Hkv + N + d, causal=causal)


def test_gqa_fp32():
    check_case_gqa(1, 4, 1, 128, 64, "fp32", 820)
    check_case_gqa(1, 2, 1, 90, 64, "fp32", 821, causal=True)


def test_gqa_strided_and_scaled():
    check_case_gqa(1, 4, 2, 150, 64, "bf16", 822, layout="bnhd")
    check_case_gqa(1, 4, 1, 200, 64, "bf16", 823, scale=0.1, causal=True)


def test_gqa_deterministic():
    raw, _ = make_inputs(1, 4, 333, 64, 824, "bf16", H_kv=1)
    t = to_device(raw, "bf16")
    a = run_path(t)
    b = run_path(t)
    for key in ("dK", "dV", "gK", "gV", "gQ", "gdO"):
        assert bool((a[key] == b[key]).all()), key



# ---------------------------------------------------------------- schedule ablation ([FlashBoB] appendix G.1)

THREE, ONE_WAVE = 2, 1


@pytest.mark.parametrize("B,H,N,d,causal", [
    (1, 2, 100, 64, False),   # ragged single tile
    (2, 3, 130, 64, True),
    (1, 1, 640, 64, False),
    (1, 2, 300, 128, False),
    (1, 1, 513, 128, True),
])
def test_three_pass_schedule(B, H, N, d, causal):
    check_case(B, H, N, d, "bf16", 1200 + N + d, causal=causal, schedule=THREE)


def test_three_pass_schedule_strided_scaled_peaked():
    check_case(1, 2, 150, 64, "bf16", 1210, layout="bnhd", schedule=THREE)
    check_case(1, 2, 200, 64, "bf16", 1211, scale=0.1, schedule=THREE)
    check_case(1, 2, 512, 64, "bf16", 1212, qk=2.0, cot=0.1, schedule=THREE)


def test_three_pass_schedule_grouped_query():
    check_case_gqa(1, 4, 1, 150, 64, "bf16", 1220, schedule=THREE)
    check_case_gqa(1, 4, 2, 200, 128, "bf16", 1221, causal=True, schedule=THREE)


@pytest.mark.parametrize("B,H,N,causal", [(1, 2, 100, False), (2, 3, 300, True)])
def test_two_pass_one_wave_schedule(B, H, N, causal):
    check_case(B, H, N, 64, "bf16", 1230 + N, causal=causal, schedule=ONE_WAVE)


def test_three_pass_phases_in_order_equal_the_whole():
    import torch

    import exact_second_order_fa_amd as fa

    raw, _ = make_inputs(1, 2, 333, 64, 1240, "bf16")
    t = to_device(raw, "bf16")
    o, lse = fa.fa_fwd(t["q"], t["k"], t["v"])
    args = (t["q"], t["k"], t["v"], o, lse, t["do"], t["uq"], t["uk"], t["uv"])
    whole = fa.fa_bob(*args, schedule=THREE)
    outs = [torch.empty_like(x) for x in whole[:4]]
    ws = torch.empty_like(whole[4])
    for ph in range(4):
        fa.fa_bob(*args, gq=outs[0], gk=outs[1], gv=outs[2], gdo=outs[3], ws=ws, schedule=THREE, phase=ph)
    torch.cuda.synchronize()
    # the outputs and the workspace's D, alpha, E (its ABI part)
    for a_, b_ in zip(whole[:4] + (whole[4][:3 * 2 * 333],), outs + [ws[:3 * 2 * 333]]):
        assert bool((a_ == b_).all())


def test_binding_rejects_bad_arguments_before_launch():
    """Wrongly typed, shaped or placed saved state, outputs and workspaces
    raise ValueError in the binding, before the library is called; the
    outputs given to the rejected calls are left untouched."""
    import torch

    import exact_second_order_fa_amd as fa

    raw, _ = make_inputs(1, 2, 96, 64, 5, "bf16")
    t = to_device(raw, "bf16")
    q, k, v, do, uq, uk, uv = (t[n] for n in NAMES)
    o, lse = fa.fa_fwd(q, k, v)
    sentinel = torch.full(q.shape, 7.0, device="cuda")
    good = dict(gq=sentinel)
    bad_calls = {
        "bf16 O": lambda: fa.fa_bob(q, k, v, o.to(torch.bfloat16), lse, do, uq, uk, uv, **good),
        "O of another shape": lambda: fa.fa_bob(q, k, v, o[:, :1], lse, do, uq, uk, uv, **good),
        "float64 L": lambda: fa.fa_bob(q, k, v, o, lse.double(), do, uq, uk, uv, **good),
        "L of another length": lambda: fa.fa_bwd(q, k, v, o, lse[:, :, :50], do),
        "strided L": lambda: fa.fa_bwd(q, k, v, o, torch.empty(1, 96, 2, device="cuda").permute(0, 2, 1), do),
        "host L": lambda: fa.fa_bob(q, k, v, o, lse.cpu(), do, uq, uk, uv, **good),
        "host O": lambda: fa.fa_bwd(q, k, v, o.cpu(), lse, do),
        "host output": lambda: fa.fa_bob(q, k, v, o, lse, do, uq, uk, uv, gk=torch.empty(k.shape)),
        "bf16 output": lambda: fa.fa_bwd(q, k, v, o, lse, do, dq=torch.empty(q.shape, dtype=torch.bfloat16,
                                                                               device="cuda")),
        "host workspace": lambda: fa.fa_bob(q, k, v, o, lse, do, uq, uk, uv, ws=torch.empty(1 << 20), **good),
        "small workspace": lambda: fa.fa_bob(q, k, v, o, lse, do, uq, uk, uv,
                                             ws=torch.empty(4, device="cuda"), **good),
        "host fa_fwd lse": lambda: fa.fa_fwd(q, k, v, lse=torch.empty(1, 2, 96)),
    }
    for what, call in bad_calls.items():
        with pytest.raises(ValueError):
            call()
        torch.cuda.synchronize()
        say(f"  rejected: {what}")
    assert bool((sentinel == 7.0).all())


@pytest.mark.parametrize("d,causal,layout,rising", [
    (64, False, "bhnd", False), (64, True, "bhnd", False), (128, False, "bhnd", False), (128, True, "bhnd", False),
    (64, False, "bnhd", False), (128, True, "bnhd", False), (64, False, "bhnd", True), (128, True, "bhnd", True)])
def test_three_wave_forward_ragged(d, causal, layout, rising):
    """fa_fwd on a grid of 1536 row workgroups (48 heads x 32 row blocks) runs
    three waves per SIMD (64-key tiles at d = 64, 32-key tiles at d = 128);
    N = 4000 leaves a ragged last tile; "bnhd" passes strided head views;
    rising: key norms growing along the sequence and one late outlier (see
    _rising_keys), so the lazy reference maximum moves.  O and L of every head
    against the dense oracle."""
    import exact_second_order_fa_amd as fa
    from oracle import forward_dense

    B, H, N, seed = 1, 48, 4000, 610 + int(causal) + d + 2 * int(rising)
    say(f"three-wave forward: B={B} H={H} N={N} d={d} causal={causal} layout={layout} rising={rising} seed={seed}")
    raw, f64 = make_inputs(B, H, N, d, seed, "bf16")
    if rising:
        _rising_keys(raw, f64)
    t = to_device(raw, "bf16", layout)
    o, lse = fa.fa_fwd(t["q"], t["k"], t["v"], causal=causal)
    o, lse = host(o), host(lse)
    ref_o, ref_l = np.zeros((B, H, N, d)), np.zeros((B, H, N))
    for h in range(H):
        r = forward_dense(f64["q"][0, h], f64["k"][0, h], f64["v"][0, h], 1.0 / np.sqrt(d), causal=causal)
        ref_o[0, h], ref_l[0, h] = r["O"], r["L"]
    errs = {"O": rel(o, ref_o), "L": rel(lse, ref_l)}
    say("  " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    assert all(v <= TOL["bf16"] for v in errs.values()), errs
