"""Write the stored oracle values for the full-size parity tests.

The column-owned BoB outputs gK, gV of one key column need the row scalars
L, D, alpha, E of every query row, i.e. a full O(N^2 d) sweep per head, which
is too slow to repeat inside a GPU test at N = 16K .. 262K.  This script runs
that sweep once with the float64 oracle (``oracle/``) on the seeded inputs of
each workload (``fa_inputs``) and stores gK, gV for a seeded sample of key
columns, plus the row scalars of a seeded sample of rows.  It calls nothing
but ``oracle`` and ``fa_inputs``.

Usage:  python tests/golden/make_golden.py [hd128] [long] [max] [gpt2c_16k] [mqa_32k] [--threads N]
"""
from __future__ import annotations

import argparse
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from fa_inputs import WORKLOADS, workload_inputs  # noqa: E402
from oracle import col_pass, col_pass_group, row_state  # noqa: E402

# (workload, heads (b, h) to sample, key columns per head).  For grouped-query
# workloads h is a key/value head; its columns sum over the group's query heads.
PLAN = {
    "hd128": ([(0, 0), (0, 15)], 24),
    "long": ([(0, 1), (0, 3)], 24),
    "max": ([(0, 0)], 32),
    "gpt2c_16k": ([(0, 0), (3, 11)], 24),
    "mqa_32k": ([(0, 0)], 24),
}


def sample_cols(N, n, seed):
    rng = np.random.default_rng(seed)
    cols = set(rng.choice(N, size=n - 2, replace=False).tolist())
    cols.update({0, N - 1})
    return np.array(sorted(cols), dtype=np.int64)


def make(name, threads):
    w = WORKLOADS[name]
    heads, ncol = PLAN[name]
    t0 = time.time()
    _, f64 = workload_inputs(w)
    out = {"heads": [], "cols": [], "gK": [], "gV": [], "dK": [], "dV": [], "state_rows": [],
           "L": [], "D": [], "alpha": [], "E": []}
    G = w.H // w.Hkv
    for (b, h) in heads:
        kside = {n: f64[n][b, h] for n in ("k", "v", "uk", "uv")}
        qheads = range(h * G, (h + 1) * G) if G > 1 else [h]
        states = {}
        for hq in qheads:
            args = [f64["q"][b, hq], kside["k"], kside["v"], f64["do"][b, hq], f64["uq"][b, hq], kside["uk"],
                    kside["uv"]]
            states[hq] = row_state(*args, w.scale, threads=threads, causal=w.causal)
            print(f"{name}: row state of ({b},{hq}) at {time.time() - t0:.0f}s", flush=True)
        cols = sample_cols(w.N, ncol, 1000 * w.seed + 17 * b + h)
        if G > 1:
            c = col_pass_group([f64["q"][b, hq] for hq in qheads], kside["k"], kside["v"],
                               [f64["do"][b, hq] for hq in qheads], [f64["uq"][b, hq] for hq in qheads],
                               kside["uk"], kside["uv"], w.scale, [states[hq] for hq in qheads], cols=cols,
                               causal=w.causal, strip=8, threads=threads)
        else:
            args = [f64[n][b, h] for n in ("q", "k", "v", "do", "uq", "uk", "uv")]
            c = col_pass(*args, w.scale, states[h], cols=cols, strip=8, threads=threads, causal=w.causal)
        for j, col in enumerate(cols):
            out["heads"].append((b, h))
            out["cols"].append(col)
            out["gK"].append(c["gK"][j])
            out["gV"].append(c["gV"][j])
            out["dK"].append(c["dK"][j])
            out["dV"].append(c["dV"][j])
        for hq in qheads:
            srows = sample_cols(w.N, ncol, 2000 * w.seed + 17 * b + hq)
            for r in srows:
                out["state_rows"].append((b, hq, r))
                for key in ("L", "D", "alpha", "E"):
                    out[key].append(states[hq][key][r])
        print(f"{name}: head ({b},{h}) done at {time.time() - t0:.0f}s", flush=True)
    path = os.path.join(HERE, f"{name}_cols.npz")
    np.savez(path, **{k: np.asarray(v) for k, v in out.items()})
    print(f"wrote {path} in {time.time() - t0:.0f}s", flush=True)


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("names", nargs="*", default=list(PLAN))
    ap.add_argument("--threads", type=int, default=None)
    a = ap.parse_args()
    for n in a.names:
        make(n, a.threads)
