"""Parity of the dropout path (fa_fwd, fa_bwd, fa_bob with a dropout rate and
seed, through the C ABI) with the float64 dropout oracle, which draws the same
Philox4x64-10 mask from its own implementation.  Every output is compared
element by element, with the bars of the dropout-free tests (bf16 2e-2, fp32
1e-4 relative to the oracle's maximum)."""
import numpy as np
import pytest

from fa_inputs import make_inputs
from oracle import bob_dropout, bob_dropout_heads, dropout_mask
from tests.gpu_helpers import host, rel, run_dropout, say, to_device

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "fp32": 1e-4}
ALL = ("O", "L", "dQ", "dK", "dV", "D", "alpha", "E", "gQ", "gK", "gV", "gdO")


@pytest.mark.parametrize("B,H,Hkv,N,d,dtype,p,causal", [
    (1, 2, 2, 100, 64, "fp32", 0.1, False),   # ragged tile
    (1, 1, 1, 128, 64, "fp32", 0.5, True),
    (1, 2, 2, 130, 64, "bf16", 0.25, False),  # ragged resident block
    (1, 2, 2, 300, 64, "bf16", 0.3, False),   # several key tiles and resident blocks
    (1, 1, 1, 290, 128, "bf16", 0.3, True),
    (2, 2, 2, 97, 64, "bf16", 0.5, True),
    (1, 4, 2, 64, 64, "bf16", 0.1, False),    # grouped-query heads
    (1, 2, 2, 75, 128, "bf16", 0.2, False),   # d = 128
    (1, 1, 1, 33, 128, "bf16", 0.9, True),
    (1, 2, 2, 2048, 64, "bf16", 0.2, True),     # many key tiles and mask granules
    (1, 2, 1, 1100, 128, "bf16", 0.15, False),  # grouped-query, d = 128, ragged, many tiles
])
def test_dropout_parity(B, H, Hkv, N, d, dtype, p, causal):
    seed = 1000 + N + d
    say(f"dropout case B={B} H={H} H_kv={Hkv} N={N} d={d} {dtype} p={p} causal={causal} seed={seed}")
    raw, f64 = make_inputs(B, H, N, d, seed, dtype, H_kv=Hkv)
    got = run_dropout(to_device(raw, dtype), p, seed, causal)
    ref = bob_dropout_heads(*(f64[n] for n in ("q", "k", "v", "do", "uq", "uk", "uv")), 1.0 / np.sqrt(d), p, seed,
                            causal)
    errs = {k: rel(host(got[k]), ref[k]) for k in ALL}
    say("  " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL[dtype]}
    assert not bad, bad


def _dropout_edge_heads(H, Hkv, p, seed, causal, what):
    """Every head of B = 1, N = 4000 (32 ragged 128-row blocks), d = 64 runs on
    the GPU; the first and the last key/value head, with all their query
    heads, are compared element by element with the dropout oracle (its mask
    draw is what bounds the count)."""
    B, N, d = 1, 4000, 64
    say(f"dropout {what}: B={B} H={H} H_kv={Hkv} N={N} d={d} p={p} causal={causal} seed={seed}")
    raw, f64 = make_inputs(B, H, N, d, seed, "bf16", H_kv=Hkv)
    got = {k: host(v) for k, v in run_dropout(to_device(raw, "bf16"), p, seed, causal).items()}
    G = H // Hkv
    for hk in (0, Hkv - 1):
        col = {}
        for h in range(hk * G, (hk + 1) * G):
            r = bob_dropout(f64["q"][0, h], f64["k"][0, hk], f64["v"][0, hk], f64["do"][0, h], f64["uq"][0, h],
                            f64["uk"][0, hk], f64["uv"][0, hk], 1.0 / np.sqrt(d), dropout_mask(h, N, p, seed),
                            causal)
            errs = {k: rel(got[k][0, h], r[k]) for k in ("O", "L", "D", "alpha", "E", "gQ", "gdO", "dQ")}
            say(f"  head {h}: " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
            assert all(v <= TOL["bf16"] for v in errs.values()), errs
            for k in ("gK", "gV", "dK", "dV"):
                col[k] = col.get(k, 0.0) + r[k]
        errs = {k: rel(got[k][0, hk], col[k]) for k in col}
        say(f"  key/value head {hk}: " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
        assert all(v <= TOL["bf16"] for v in errs.values()), errs


@pytest.mark.parametrize("H,Hkv", [(16, 16), (32, 16)])
def test_dropout_two_wave_column_pass(H, Hkv):
    """d = 64 grids of a whole multiple of 512 column workgroups run the
    dropout column pass at two waves per SIMD (64-row tiles): 16 key/value
    heads, with one and with two query heads per key/value head."""
    _dropout_edge_heads(H, Hkv, 0.2, 4242 + H, False, "two-wave column pass")


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_three_wave_forward(causal):
    """d = 64 grids of at least 1536 row workgroups (48 heads here) run the
    dropout forward at three waves per SIMD with 64-key tiles."""
    _dropout_edge_heads(48, 48, 0.15, 4300 + int(causal), causal, "three-wave forward")


def test_dropout_rate_rounding_to_zero_is_the_dropout_free_path():
    """A rate below 1/512 rounds to threshold 0: no element is dropped and the
    library takes its dropout-free kernels (bit-identical outputs)."""
    raw, _ = make_inputs(1, 2, 96, 64, 77, "bf16")
    t = to_device(raw, "bf16")
    a = run_dropout(t, 0.0, 5, False)
    b = run_dropout(t, 0.001, 5, False)
    for k in ALL:
        assert np.array_equal(host(a[k]), host(b[k])), k


def test_dropout_seed_determinism():
    """The same (p, seed) reproduces every output bit for bit; another seed
    draws another mask."""
    raw, _ = make_inputs(1, 1, 64, 64, 78, "fp32")
    t = to_device(raw, "fp32")
    a = run_dropout(t, 0.3, 11, False)
    b = run_dropout(t, 0.3, 11, False)
    c = run_dropout(t, 0.3, 12, False)
    for k in ALL:
        assert np.array_equal(host(a[k]), host(b[k])), k
    assert not np.array_equal(host(a["O"]), host(c["O"]))
