"""CPU oracle for one SparseX prefill layer -- TEST INFRASTRUCTURE ONLY.

This package is the slow, obviously-correct reference that the GPU path is
checked against.  It is imported only by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``.
The product path (``segment_level_kv_amd``) never imports, links or calls it,
and the oracle imports nothing from the product: the two share no code.

Everything is plain NumPy in float64.  Storage rounding to the kernel's
storage type (bf16 or fp32) is emulated at exactly the points where the GPU
path stores a tensor (the cached/realigned K and V, the Q buffer, recomputed
K/V and the layer output), so that the two agree up to accumulation order.

Source of every definition: "SparseX: Efficient Segment-Level KV Cache
Sharing for Interleaved LLM Serving" (arXiv 2606.01751), cited per function
by section and display equation.

Parity status per function (see each docstring):
  round_bf16, rope_rotate, realign_segment, plan_request, project_rows,
  causal_attention, attention_mass_scores, select_topk, sparse_layer,
  full_layer -- pinned by tests/test_oracle_pins.py and
  tests/test_oracle_layer.py against closed forms, invariants, library
  routines and brute force.
"""

from .sparsex import (  # noqa: F401
    round_bf16,
    round_store,
    rope_inv_freq,
    rope_rotate,
    realign_segment,
    plan_request,
    project_rows,
    causal_attention,
    attention_mass_scores,
    select_topk,
    sparse_layer,
    full_layer,
)
