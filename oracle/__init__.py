"""CPU float64 oracle for exact blockwise causal attention with masked sequence packing.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's CPU
baseline leg may import this package.  The HIP library never calls it and shares no code
with it; the two meet only in the seeded input generators of `lwm_inputs`.

What it computes is the plain definition of the attention the LWM pages describe: exact,
full (not windowed, not sparse) softmax attention ("RingAttention 为什么必要 / why
RingAttention is necessary" in the LWM deep dive), causal because the model predicts the
next token of one unified sequence ("核心问题 / core problem" and "模型结构 / model
structure"), and confined to each packed sample by the attention mask of "Masked sequence
packing".  Blockwise and ring evaluation reorder the same sums, so the oracle forms the full
masked score matrix (or whole rows of it) and applies softmax directly.

Modules:
  attention  -- vectorised NumPy float64 definitions (forward, backward, partial state,
                merge, finalize, sampled rows)
  brute      -- pure-Python loops over tiny inputs, used to pin `attention`
  table      -- exact SKIP / PARTIAL / FULL classification of (query block, key block) pairs
  rope       -- rotary position embedding with a large base theta, and attention on rotated
                queries and keys
  packed_loss -- next-token cross-entropy reweighted so every packed sample weighs the same
"""
from . import attention, brute, packed_loss, rope, table  # noqa: F401
from .attention import (  # noqa: F401
    visibility, forward, backward, forward_head, backward_head, partial_state, merge_states,
    finalize_state, forward_rows, dq_rows, EMPTY_M,
)
