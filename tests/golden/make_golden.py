"""Write the stored oracle values for the N = 262,144 parity test.

Every other workload is compared with the float64 oracle run inside the test,
over whole tensors.  At N = 262,144 a full oracle run (row and column sweeps,
about 62 N^2 d float64 flops) takes too long for a test, so this script runs
it once with the oracle (``oracle/``) on the seeded inputs (``fa_inputs``) and
stores, in float32:

* the row scalars L, D, alpha, E of every row;
* per block of 128 rows, the sums over the block's rows of the row-owned
  outputs O, dQ, gQ, gdO; per block of 128 key columns, the sums of the
  column-owned outputs dK, dV, gK, gV (a whole-tensor check: a wrong value
  anywhere moves its block's sum);
* whole 128-column blocks of dK, dV, gK, gV for the blocks listed in BLOCKS
  (the test computes the same row blocks itself, a row at a time being
  cheap).

It calls nothing but ``oracle`` and ``fa_inputs``.

Usage:  python tests/golden/make_golden.py [--threads N]
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
from oracle import col_pass, row_pass  # noqa: E402

NAME = "max"
BLK = 128
# 128-row / 128-column blocks compared element by element: the first and last
# two and interior blocks spread over the whole sequence (every 1/8 of it, so
# each group of workgroups the launch places on one XCD has some).
BLOCKS = (0, 1, 255, 256, 511, 700, 1023, 1024, 1300, 1535, 1600, 1792, 1999, 2046, 2047)
PATH = os.path.join(HERE, f"{NAME}_blocks.npz")


def block_sums(x, blk=BLK):
    n = x.shape[0]
    nb = (n + blk - 1) // blk
    pad = nb * blk - n
    if pad:
        x = np.concatenate([x, np.zeros((pad,) + x.shape[1:])], axis=0)
    return x.reshape(nb, blk, *x.shape[1:]).sum(axis=1)


def make(threads):
    w = WORKLOADS[NAME]
    assert (w.B, w.H) == (1, 1)
    t0 = time.time()
    _, f64 = workload_inputs(w)
    args = [f64[n][0, 0] for n in ("q", "k", "v", "do", "uq", "uk", "uv")]
    r = row_pass(*args, w.scale, outputs="all", threads=threads, causal=w.causal)
    print(f"{NAME}: row pass at {time.time() - t0:.0f}s", flush=True)
    c = col_pass(*args, w.scale, r, threads=threads, causal=w.causal)
    print(f"{NAME}: column pass at {time.time() - t0:.0f}s", flush=True)
    out = {"blocks": np.asarray(BLOCKS, dtype=np.int64), "blk": np.int64(BLK)}
    for key in ("L", "D", "alpha", "E"):
        out[key] = r[key].astype(np.float32)
    for key in ("O", "dQ", "gQ", "gdO"):
        out[f"rowsum_{key}"] = block_sums(r[key]).astype(np.float32)
    for key in ("dK", "dV", "gK", "gV"):
        out[f"colsum_{key}"] = block_sums(c[key]).astype(np.float32)
        out[f"cols_{key}"] = np.stack([c[key][b * BLK:(b + 1) * BLK] for b in BLOCKS]).astype(np.float32)
    np.savez(PATH, **out)
    print(f"wrote {PATH} in {time.time() - t0:.0f}s", flush=True)


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--threads", type=int, default=None)
    make(ap.parse_args().threads)
