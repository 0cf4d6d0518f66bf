"""CPU float64 oracle for softmax attention forward, first backward and
backward-over-backward (BoB).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only the test-suite, the smoke check in ``__graft_entry__`` and the CPU
baseline leg of ``bench.py`` call it.  It shares no code with the HIP
library (``exact_second_order_fa_amd``) and imports nothing from it.

Sources (cited by page title and section throughout):

* [FlashBoB] "FlashBoB: I/O-Efficient Exact Backward-over-Backward for Softmax
  Attention" (Givans, Crawshaw, Liu): section 3 (forward, log-normaliser,
  first backward), section 4.1 (the BoB functional Phi), section 4.2 (the
  closed-form outputs), appendix D (notation, reverse-mode Steps 1-7 and the
  final assembled identities).
  Section 4.3 (the paragraph after Algorithm 1) for grouped-query and
  multi-query attention (``gqa``).
* [FA2-recompute] the interview answer "Why does FlashAttention-2's backward
  pass recompute attention, and what exactly does the forward pass save for
  it?": the saved state (O and one fp32 log-sum-exp per row) and the identity
  D = rowsum(dO * O).

Every function below computes a plain definition from those passages in
float64.  ``dense`` materialises every N x N matrix (small N); ``streaming``
computes the same quantities strip by strip so that long sequences fit in
memory.  Parity pins for every function live in ``tests/test_oracle_*.py``;
none is "parity unpinned".
"""
from .dense import backward_dense, bob_dense, forward_dense, phi_dense  # noqa: F401
from .gqa import bob_dense_gqa, bob_streaming_gqa, col_pass_group  # noqa: F401
from .streaming import (  # noqa: F401
    bob_streaming,
    col_pass,
    row_pass,
    row_state,
)
from .dropout import (  # noqa: F401
    backward_dropout,
    bob_dropout,
    bob_dropout_heads,
    dropout_mask,
    forward_dropout,
    keep_bytes,
    philox4x64_10,
    phi_dropout,
    threshold,
)
