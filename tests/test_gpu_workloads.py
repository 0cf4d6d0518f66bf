"""Parity at the benchmarked workloads' full sizes, in the launch configuration
the benchmark times (the same entry points, contiguous [B, H, N, d] tensors).

The bar is the one for every GPU result: per output tensor,
max |gpu - oracle| / max |oracle| <= 2e-2 for bf16 inputs, 1e-4 for fp32.
Each test below asserts it over the heads it covers (at least as strict as
the whole-tensor measure) and the last test of a workload prints the
whole-tensor measure.

* tiny (fp32) and mid: every element, dense / streaming oracle.
* hd128, long, gpt2c_4k, gpt2c_16k, c128_16k and the multi-query mqa_2k,
  mqa_8k, mqa_32k, mqa128_8k: every
  element of every output (O, L, D, alpha, E, dQ, dK, dV, gQ, gK, gV, gdO),
  against the streaming float64 oracle run in-test head by head, split over
  several tests so that each finishes in well under a minute of host time.
* max (N = 262,144; a full oracle run is about 2.7e14 float64 flops):
  L, D, alpha, E of every row and the per-128-row / per-128-column block sums
  of every output against values stored by tests/golden/make_golden.py
  (which calls only the oracle), whole 128-column blocks against stored
  values, and whole 128-row blocks against the oracle run in-test; plus the
  memory check (the call allocates nothing, no N x N buffer exists).
* The benchmark's dropout leg (mid, p = 0.1, seed 1234): every element of all
  16 heads against the dense dropout oracle.
"""
import gc
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

from fa_inputs import WORKLOADS, workload_inputs
from oracle import bob_dense, bob_dropout, bob_streaming, col_pass_group, dropout_mask, row_pass
from tests.gpu_helpers import NAMES, host, oracle_threads, rel, run_dropout, run_path, say, to_device

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL = {"bf16": 2e-2, "fp32": 1e-4}
ROW_KEYS = ("O", "L", "D", "alpha", "E", "dQ", "gQ", "gdO")
COL_KEYS = ("dK", "dV", "gK", "gV")
ALL_KEYS = ROW_KEYS + COL_KEYS


def test_tiny_workload_full():
    w = WORKLOADS["tiny"]
    say("workload tiny")
    raw, f64 = workload_inputs(w)
    got = run_path(to_device(raw, w.dtype))
    ref = bob_dense(*(f64[n][0, 0] for n in NAMES), w.scale)
    for key in ALL_KEYS:
        e = rel(host(got[key])[0, 0], ref[key])
        say(f"  {key} {e:.2e}")
        assert e <= TOL["fp32"], key


def test_mid_workload_full():
    w = WORKLOADS["mid"]
    say("workload mid: GPU path")
    raw, f64 = workload_inputs(w)
    got = run_path(to_device(raw, w.dtype))
    say("workload mid: streaming oracle")
    ref = bob_streaming(*(f64[n] for n in NAMES), w.scale, threads=oracle_threads())
    for key in ALL_KEYS:
        e = rel(host(got[key]), ref[key])
        say(f"  {key} {e:.2e}")
        assert e <= TOL["bf16"], key


# ------------------------------------------------- two-wave column pass
# d = 64 grids of a whole multiple of 512 column workgroups run the column
# pass at two waves per SIMD (64-row tiles).  The workloads reach it only at
# N a multiple of 128 with one query head per key/value head; these cases,
# 2 x 8 x 32 = 512 column blocks each, add a ragged last tile (N = 4000,
# also causal) and two query heads per key/value head (its head loop).
# Every element of every output against the streaming oracle.


def _two_wave_case(H, Hkv, N, causal, seed, schedule=None):
    from fa_inputs import make_inputs
    from oracle import bob_streaming_gqa

    say(f"two-wave column pass: B=2 H={H} H_kv={Hkv} N={N} d=64 causal={causal} seed={seed} schedule={schedule}")
    raw, f64 = make_inputs(2, H, N, 64, seed, "bf16", H_kv=Hkv)
    got = run_path(to_device(raw, "bf16"), causal=causal, schedule=schedule)
    args = (*(f64[n] for n in NAMES), 1.0 / 8.0)
    if Hkv == H:
        ref = bob_streaming(*args, threads=oracle_threads(), causal=causal)
    else:
        ref = bob_streaming_gqa(*args, threads=oracle_threads(), causal=causal)
    for key in ALL_KEYS:
        e = rel(host(got[key]), ref[key])
        say(f"  {key} {e:.2e}")
        assert e <= TOL["bf16"], key


@pytest.mark.parametrize("causal", [False, True])
def test_two_wave_column_pass_ragged(causal):
    _two_wave_case(8, 8, 4000, causal, 511 + int(causal))


def test_two_wave_column_pass_grouped_heads():
    _two_wave_case(16, 8, 4096, False, 513)


def test_two_wave_column_pass_after_the_three_pass_row_sweeps():
    """The three-pass schedule (alpha sweep, row pass with alpha known) hands
    its chain inits to the same two-wave column pass."""
    _two_wave_case(8, 8, 4000, False, 514, schedule=2)


# --------------------------------------------------------------- whole tensors

_RUN = {}


def gpu_run(name, dropout=0.0, seed=0):
    """The GPU path (fa_fwd, fa_bwd, fa_bob) on a workload, run once and kept
    as host float32 arrays together with the oracle's inputs, the row states
    the oracle has computed so far and running whole-tensor error totals.
    Only one workload is kept at a time."""
    import torch

    tag = (name, dropout, seed)
    if tag in _RUN:
        return _RUN[tag]
    _RUN.clear()
    gc.collect()
    w = WORKLOADS[name]
    say(f"workload {name}{f' dropout {dropout} seed {seed}' if dropout else ''}: inputs and GPU path")
    raw, f64 = workload_inputs(w)
    t = to_device(raw, w.dtype)
    del raw
    if dropout:
        got = run_dropout(t, dropout, seed, w.causal)
    else:
        got = run_path(t, causal=w.causal)
    out = {k: v.detach().float().cpu().numpy() for k, v in got.items()}
    del got, t
    torch.cuda.empty_cache()
    r = {"w": w, "f64": f64, "got": out, "states": {}, "err": {}, "heads": set(), "kv_heads": set()}
    _RUN[tag] = r
    return r


def _compare(r, key, got, ref, part):
    """max |got - ref| and max |ref| of one part, folded into the workload's
    running totals; returns the part's relative error."""
    got = np.asarray(got, dtype=np.float64)
    e = float(np.max(np.abs(got - ref)))
    m = float(np.max(np.abs(ref)))
    tot = r["err"].setdefault(key, [0.0, 0.0])
    tot[0], tot[1] = max(tot[0], e), max(tot[1], m)
    part.setdefault(key, [0.0, 0.0])
    part[key][0], part[key][1] = max(part[key][0], e), max(part[key][1], m)
    return e / max(m, 1e-30)


def _assert_part(r, part, what):
    tol = TOL[r["w"].dtype]
    errs = {k: v[0] / max(v[1], 1e-30) for k, v in part.items()}
    say(f"  {what}: " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, (what, bad)


def check_rows(name, heads):
    """Every row-owned output of the query heads ``heads`` ((b, h) pairs)
    against the oracle's row pass; the row states are kept for the column
    side."""
    r = gpu_run(name)
    w, f64 = r["w"], r["f64"]
    G = w.H // w.Hkv
    part = {}
    for b, h in heads:
        hk = h // G
        st = row_pass(f64["q"][b, h], f64["k"][b, hk], f64["v"][b, hk], f64["do"][b, h], f64["uq"][b, h],
                      f64["uk"][b, hk], f64["uv"][b, hk], w.scale, outputs="all", threads=oracle_threads(),
                      causal=w.causal)
        for key in ROW_KEYS:
            _compare(r, key, r["got"][key][b, h], st[key], part)
        r["states"][(b, h)] = {k: st[k] for k in ("L", "D", "alpha", "E")}
        r["heads"].add((b, h))
    _assert_part(r, part, f"{name} rows of heads {heads[0]}..{heads[-1]}")


def check_cols(name, kv_heads):
    """Every column-owned output of the key/value heads ``kv_heads`` against
    the oracle's column pass (summed over each group's query heads), from the
    row states of those query heads."""
    r = gpu_run(name)
    w, f64 = r["w"], r["f64"]
    G = w.H // w.Hkv
    part = {}
    for b, hk in kv_heads:
        qh = list(range(hk * G, (hk + 1) * G))
        for h in qh:
            if (b, h) not in r["states"]:
                check_rows(name, [(b, h)])
        kside = [f64[n][b, hk] for n in ("k", "v")]
        c = col_pass_group([f64["q"][b, h] for h in qh], *kside, [f64["do"][b, h] for h in qh],
                           [f64["uq"][b, h] for h in qh], f64["uk"][b, hk], f64["uv"][b, hk], w.scale,
                           [r["states"][(b, h)] for h in qh], causal=w.causal, threads=oracle_threads())
        for key in COL_KEYS:
            _compare(r, key, r["got"][key][b, hk], c[key], part)
        for h in qh:
            del r["states"][(b, h)]
        r["kv_heads"].add((b, hk))
    _assert_part(r, part, f"{name} columns of key/value heads {kv_heads[0]}..{kv_heads[-1]}")


def report_whole(name, dropout=0.0, seed=0):
    """The whole-tensor measure of every output, once every head was checked."""
    r = gpu_run(name, dropout, seed)
    w = r["w"]
    assert len(r["heads"]) == w.B * w.H and len(r["kv_heads"]) == w.B * w.Hkv, "not every head was compared"
    _assert_part(r, r["err"], f"{name} whole tensors ({w.B}x{w.H} heads, N={w.N}, d={w.d})")


def _heads(w, per, kv=False):
    H = w.Hkv if kv else w.H
    hs = [(b, h) for b in range(w.B) for h in range(H)]
    return [hs[i:i + per] for i in range(0, len(hs), per)]


# (workload, query heads per test); multi-head workloads check the column side
# of a head right after its rows.
WHOLE = {"hd128": 4, "long": 1, "gpt2c_4k": 48, "gpt2c_16k": 12, "c128_16k": 12}
WHOLE_CASES = [(name, i) for name, per in WHOLE.items() for i in range(len(_heads(WORKLOADS[name], per)))]


@pytest.mark.parametrize("name,part", WHOLE_CASES, ids=[f"{n}-{i}" for n, i in WHOLE_CASES])
def test_workload_whole_tensors(name, part):
    w = WORKLOADS[name]
    chunks = _heads(w, WHOLE[name])
    heads = chunks[part]
    check_rows(name, heads)
    check_cols(name, heads)
    if part == len(chunks) - 1:
        report_whole(name)


# Multi-query workloads (8 query heads share one key/value head): the rows of
# the query heads, then the shared head's columns summed over the group.
# Below 256 key blocks the column kernels split each key block's query heads
# over several workgroups: mqa_8k and mqa128_8k into 4; mqa_32k does not
# split; mqa_2k and mqa128_2k into 8 (one head each) and, in the BoB column
# pass, each head's rows into two ranges (16 partial sums per key block).
MQA = {"mqa_32k": 4, "mqa128_8k": 8, "mqa_8k": 8, "mqa_2k": 8, "mqa128_2k": 8}
MQA_CASES = [(name, i) for name, per in MQA.items() for i in range(WORKLOADS[name].H // per + 1)]


@pytest.mark.parametrize("name,part", MQA_CASES, ids=[f"{n}-{i}" for n, i in MQA_CASES])
def test_mqa_workload_whole_tensors(name, part):
    w = WORKLOADS[name]
    chunks = _heads(w, MQA[name])
    if part < len(chunks):
        check_rows(name, chunks[part])
    else:
        check_cols(name, [(b, hk) for b in range(w.B) for hk in range(w.Hkv)])
        report_whole(name)


# ------------------------------------------------------------ N = 262,144

def _block_sums(x, blk):
    n = x.shape[0]
    nb = (n + blk - 1) // blk
    x = np.asarray(x, dtype=np.float64)
    if nb * blk != n:
        x = np.concatenate([x, np.zeros((nb * blk - n,) + x.shape[1:])], axis=0)
    return x.reshape(nb, blk, *x.shape[1:]).sum(axis=1)


def test_max_workload_blocks_and_sums():
    r = gpu_run("max")
    w, f64, got = r["w"], r["f64"], r["got"]
    g = np.load(os.path.join(GOLDEN, "max_blocks.npz"), allow_pickle=False)
    blk, blocks = int(g["blk"]), [int(b) for b in g["blocks"]]
    tol = TOL[w.dtype]
    errs = {}
    for key in ("L", "D", "alpha", "E"):
        errs[f"{key} every row"] = rel(got[key][0, 0], g[key])
    for key in ("O", "dQ", "gQ", "gdO"):
        errs[f"{key} row-block sums"] = rel(_block_sums(got[key][0, 0], blk), g[f"rowsum_{key}"])
    for key in COL_KEYS:
        errs[f"{key} column-block sums"] = rel(_block_sums(got[key][0, 0], blk), g[f"colsum_{key}"])
        errs[f"{key} {len(blocks)} whole column blocks"] = rel(
            np.stack([got[key][0, 0][b * blk:(b + 1) * blk] for b in blocks]), g[f"cols_{key}"])
    rows = np.concatenate([np.arange(b * blk, min((b + 1) * blk, w.N)) for b in blocks])
    say(f"  oracle: {len(blocks)} whole row blocks of max")
    ref = row_pass(*(f64[n][0, 0] for n in NAMES), w.scale, rows=rows, outputs="all", strip=16,
                   threads=oracle_threads(), causal=w.causal)
    for key in ROW_KEYS:
        errs[f"{key} {len(blocks)} whole row blocks"] = rel(got[key][0, 0][rows], ref[key])
    for k, v in errs.items():
        say(f"  max {k}: {v:.2e}")
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad


def test_max_workload_memory():
    import torch

    import exact_second_order_fa_amd as fa

    _RUN.clear()
    gc.collect()
    torch.cuda.empty_cache()
    w = WORKLOADS["max"]
    g = torch.Generator(device="cuda").manual_seed(4)
    shape = (w.B, w.H, w.N, w.d)
    t = {n: torch.randn(shape, device="cuda", generator=g).to(torch.bfloat16) for n in NAMES}
    o, lse = fa.fa_fwd(t["q"], t["k"], t["v"])
    outs = [torch.empty(shape, dtype=torch.float32, device="cuda") for _ in range(4)]
    ws = torch.empty(fa.bob_workspace_bytes(*shape) // 4, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    fa.fa_bob(t["q"], t["k"], t["v"], o, lse, t["do"], t["uq"], t["uk"], t["uv"],
              gq=outs[0], gk=outs[1], gv=outs[2], gdo=outs[3], ws=ws)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    peak = torch.cuda.max_memory_allocated()
    say(f"  memory: device free delta {free0 - free1} B, torch peak {peak / 2**20:.0f} MiB, "
        f"resident {base / 2**20:.0f} MiB")
    assert free0 - free1 <= 4 << 20          # the library allocates nothing
    assert peak == base                      # no allocation during the call
    assert peak < 2 << 30                    # an N x N bf16 buffer would be 128 GiB


# --------------------------------------------------- the dropout leg at mid

DROP_P, DROP_SEED, DROP_PER = 0.1, 1234, 8


def _dropout_head(args):
    f64, w, b, h = args
    from threadpoolctl import threadpool_limits

    with threadpool_limits(limits=1, user_api="blas"):
        gmask = dropout_mask(b * w.H + h, w.N, DROP_P, DROP_SEED)
        return bob_dropout(*(f64[n][b, h] for n in NAMES), w.scale, gmask, w.causal)


@pytest.mark.parametrize("part", range(2))
def test_mid_dropout_leg_whole_tensors(part):
    """Every element of every output of the benchmark's dropout leg (mid,
    p = 0.1, seed 1234) against the dense dropout oracle, 8 heads per test."""
    r = gpu_run("mid", DROP_P, DROP_SEED)
    w, f64 = r["w"], r["f64"]
    heads = _heads(w, DROP_PER)[part]
    say(f"  dropout oracle: heads {heads[0]}..{heads[-1]}")
    with ThreadPoolExecutor(min(len(heads), oracle_threads())) as ex:
        refs = list(ex.map(_dropout_head, [(f64, w, b, h) for b, h in heads]))
    part_err = {}
    for (b, h), ref in zip(heads, refs):
        for key in ALL_KEYS:
            _compare(r, key, r["got"][key][b, h], ref[key], part_err)
        r["heads"].add((b, h))
        r["kv_heads"].add((b, h))
    _assert_part(r, part_err, f"mid dropout heads {heads[0]}..{heads[-1]}")
    if part == 1:
        report_whole("mid", DROP_P, DROP_SEED)
