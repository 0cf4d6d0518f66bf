"""Seeded input generator (see the package docstring for the recipe)."""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# Draw order of the seven tensors.  U_Q, U_K, U_V are the upstream cotangents
# on dQ, dK, dV (called gdQ, gdK, gdV in the workload descriptions).
NAMES = ("q", "k", "v", "do", "uq", "uk", "uv")


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "bf16" or "fp32": the element type the kernels receive
    seed: int
    cot_std: float = 1.0  # standard deviation of U_Q, U_K, U_V
    qk_gain: float = 1.0  # extra factor on Q and K rows (peaked softmax rows)
    causal: bool = False
    H_kv: int = 0  # key/value heads (0: same as H); grouped-query / multi-query below H
    note: str = field(default="", compare=False)

    @property
    def Hkv(self) -> int:
        return self.H_kv or self.H

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    @property
    def bob_flops(self) -> float:
        """Algorithmic flops of one BoB call: 19 N x N x d contractions per head.

        Row pass: S, F (two products), dP, C, then four accumulations that
        contract over the key index with two products each for gdO and the
        Omega term plus one each for R and B (11 in all).  Column pass: S, F
        (two), dP, C, then gK (two) and gV (one), 8 in all.  Each contraction
        is 2 N^2 d flops, so 38 B H N^2 d for non-causal attention; causal
        attention keeps half of the score entries and counts half of that.
        """
        f = 38.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f
    # With grouped-query attention the count is per query head: every query
    # head's rows meet every key of its group's head in both passes.


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 128, 64, "fp32", 0,
                     note="fp32 inputs; parity against the float64 oracle"),
    "mid": Workload("mid", 2, 8, 4096, 64, "bf16", 1),
    "hd128": Workload("hd128", 1, 16, 16384, 128, "bf16", 2, cot_std=0.1),
    "long": Workload("long", 1, 4, 65536, 64, "bf16", 3, qk_gain=2.0),
    "max": Workload("max", 1, 1, 262144, 64, "bf16", 4),
    # The isolated-layer shape of the FlashBoB benchmarks (batch 4, 12 heads,
    # causal); the pages state no input distribution, N(0,1) is used.
    "gpt2c_4k": Workload("gpt2c_4k", 4, 12, 4096, 64, "bf16", 5, causal=True),
    "gpt2c_16k": Workload("gpt2c_16k", 4, 12, 16384, 64, "bf16", 6, causal=True),
    "c128_16k": Workload("c128_16k", 4, 12, 16384, 128, "bf16", 7, causal=True),
    # The pages' multi-query benchmark shape (H_Q / H_KV = 8 / 1, batch 1,
    # N from 2K to 128K); no mask or input distribution is stated for it.
    "mqa_32k": Workload("mqa_32k", 1, 8, 32768, 64, "bf16", 8, H_kv=1),
}
# The rest of that multi-query range, at both head dims: N = 2K, 8K, 32K, 128K.
_MQA_SEED = 9
for _d in (64, 128):
    for _n in (2048, 8192, 32768, 131072):
        _name = f"mqa{'' if _d == 64 else '128'}_{_n // 1024}k"
        if _name not in WORKLOADS:
            WORKLOADS[_name] = Workload(_name, 1, 8, _n, _d, "bf16", _MQA_SEED, H_kv=1)
            _MQA_SEED += 1
# The schedule ablation's longer lengths (the pages' three-pass vs two-pass
# table runs the causal isolated-layer shape, batch 4 and 12 heads, from 1K to
# 262K).
WORKLOADS["gpt2c_64k"] = Workload("gpt2c_64k", 4, 12, 65536, 64, "bf16", 16, causal=True)
WORKLOADS["gpt2c_256k"] = Workload("gpt2c_256k", 4, 12, 262144, 64, "bf16", 17, causal=True)
MQA_SWEEP = tuple(sorted((n for n in WORKLOADS if n.startswith("mqa")), key=lambda n: (WORKLOADS[n].d, WORKLOADS[n].N)))


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def make_inputs(B: int, H: int, N: int, d: int, seed: int, dtype: str = "bf16",
                cot_std: float = 1.0, qk_gain: float = 1.0, with_f64: bool = True, H_kv: int = 0):
    """Draw the seven inputs, in the order of NAMES: q, do, uq with shape
    (B, H, N, d); k, v, uk, uv with shape (B, H_kv, N, d) (H_kv = 0: H).

    Returns ``(raw, f64)``: ``raw`` maps each name to the array the device
    receives (uint16 bf16 bits, or float32), ``f64`` maps each name to the
    same values as float64 for the oracle (``None`` values when
    ``with_f64`` is false).
    """
    if dtype not in ("bf16", "fp32"):
        raise ValueError(f"unknown dtype {dtype!r}")
    rng = np.random.default_rng(seed)
    Hk = H_kv or H
    if H % Hk:
        raise ValueError(f"H_kv = {Hk} does not divide H = {H}")
    raw, f64 = {}, {}
    for name in NAMES:
        heads = Hk if name in ("k", "v", "uk", "uv") else H
        x = rng.standard_normal(size=(B, heads, N, d), dtype=np.float32)
        if name in ("uq", "uk", "uv") and cot_std != 1.0:
            x = (x * np.float32(cot_std)).astype(np.float32)
        if name in ("q", "k") and qk_gain != 1.0:
            x = (x * np.float32(qk_gain)).astype(np.float32)
        if dtype == "bf16":
            bits = f32_to_bf16_bits(x)
            raw[name] = bits
            f64[name] = bf16_bits_to_f32(bits).astype(np.float64) if with_f64 else None
        else:
            raw[name] = x
            f64[name] = x.astype(np.float64) if with_f64 else None
    return raw, f64


def workload_inputs(w: Workload, N: int | None = None, with_f64: bool = True):
    """Inputs of a named workload (optionally with a different length N)."""
    return make_inputs(w.B, w.H, w.N if N is None else N, w.d, w.seed, w.dtype,
                       w.cot_std, w.qk_gain, with_f64, w.H_kv)
