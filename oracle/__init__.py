"""Plain, slow, fp64 CPU oracle for exact ring (blockwise) attention.

TEST INFRASTRUCTURE ONLY.  This package is the checker, not the product: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product path (the HIP library and its Python
binding) never imports, calls or links anything here, and this package imports
nothing from the product path.  The two share no arithmetic; only the seeded
input generator (which holds none of the method's arithmetic) feeds both.

What it computes, and from which passage:

* ``attention_rows`` / ``ring_attention``: softmax(Q K^T / sqrt(d)) V, the
  attention definition in "Ring Attention: Train 1M Tokens on 8GB GPUs in 2026",
  section "Why Standard Attention Explodes Past 100K Tokens" (the display
  equation), evaluated over the union of the KV blocks a device receives in the
  ring ("Ring Attention: Partition Sequence Length, Not Batch", same page).  The
  result must equal full attention exactly up to rounding ("Ring Attention with
  Blockwise Transformers for Near-Infinite Context", Abstract: no
  approximation).  Causal masking and the log-sum-exp are not defined on the
  pages; their readings are stated on each function.
* ``partial_state``: the (running max, running sum, unnormalised output)
  triple the "Gotchas and Failure Modes" section of "Ring Attention: Train 1M
  Tokens on 8GB GPUs in 2026" names as
  the state carried across chunks, written as its closed form over the blocks
  processed so far (not as an iteration), following the online-normaliser idea
  of Milakov & Gimelshein cited in the arXiv record's reference list.

* ``ring_attention_bwd`` / ``delta`` (``backward.py``): the exact gradients of
  that output with respect to Q, K and V for an upstream dO (the pages train
  through the ring but never write the backward pass; the reading is stated
  in that module); ``key_rows_bwd`` gives the same dK and dV for chosen keys
  only, over all query rows, so that long sequences can be checked key by
  key.
* ``blockwise_ffn`` / ``gelu_tanh`` (``ffn.py``): the position-wise
  feedforward computed over row blocks ("Ring Attention with Blockwise
  Transformers for Near-Infinite Context", Abstract: blockwise computation of
  self-attention and feedforward); its readings are stated in that module.

Every function is pinned by tests in ``tests/test_oracle_pins.py`` against
brute force in 50-digit arithmetic, closed forms, invariants and a library
routine.  No function here is "parity unpinned".
"""

from .attention import (  # noqa: F401
    attention_rows,
    default_scale,
    partial_state,
    ring_attention,
    visible,
)
from .backward import delta, key_rows_bwd, ring_attention_bwd  # noqa: F401
from .ffn import blockwise_ffn, gelu_tanh  # noqa: F401
