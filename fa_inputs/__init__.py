"""Seeded synthetic inputs for attention backward-over-backward.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It holds no arithmetic of the method itself: it draws the seven
input tensors (Q, K, V, dO and the cotangents U_Q, U_K, U_V that sit on the
first-backward outputs dQ, dK, dV), applies the per-workload scalings and
rounds them to bfloat16 when the workload asks for bf16 inputs.

Recipe (the same on every machine, since numpy's PCG64 stream is portable):

* ``numpy.random.default_rng(seed)``;
* ``standard_normal(size=(B, H, N, d), dtype=float32)`` drawn seven times in
  the order Q, K, V, dO, U_Q, U_K, U_V (with grouped-query / multi-query
  attention K, V, U_K, U_V are drawn with H_kv heads instead of H);
* workload scalings (cotangent standard deviation, a Q/K gain that peaks the
  softmax rows);
* for bf16 workloads, round-to-nearest-even to bfloat16.  The GPU receives
  those 16-bit patterns; the oracle receives the same values widened exactly
  to float64.
"""
from .gen import (  # noqa: F401
    NAMES,
    Workload,
    MQA_SWEEP,
    WORKLOADS,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_inputs,
    workload,
    workload_inputs,
)
