"""fp64 reference for the blockwise feedforward of one device's chunk (TEST
INFRASTRUCTURE ONLY; see the package docstring).

"Ring Attention with Blockwise Transformers for Near-Infinite Context"
(Abstract) computes both self-attention and the feedforward blockwise; it
does not write the feedforward out.  Readings used:

* The feedforward is the position-wise two-layer network of a Transformer
  block, y = act(x W1^T + b1) W2^T + b2, with W1 [F, d], W2 [d, F] (rows are
  output features) and a hidden width F = 4 d.
* act is GELU in its tanh form, 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715
  x^3))) (Hendrycks and Gimpel, "Gaussian Error Linear Units"), the
  activation of GPT-style language models such as the 1.3B model of "Ring
  Attention: Train 1M Tokens on 8GB GPUs in 2026", section "Memory
  Breakdown: 512K Tokens on 4x RTX 3090" (hidden dim 2048).
* Blockwise: the chunk's rows are processed in blocks, so the hidden
  activation exists for one block of rows at a time.  The network is
  position-wise, so the blockwise result is the whole-chunk result exactly;
  the oracle still evaluates block by block so that property is tested.
"""

from __future__ import annotations

import numpy as np


def gelu_tanh(x):
    """GELU, tanh form (Hendrycks and Gimpel), elementwise in fp64."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))


def blockwise_ffn(x, w1, b1, w2, b2, block_rows: int | None = None):
    """y [N, d] = gelu(x W1^T + b1) W2^T + b2 over row blocks of block_rows
    (all rows at once when None).  x [N, d], w1 [F, d], b1 [F], w2 [d, F],
    b2 [d]; every input is widened to fp64 (bf16 values are exact)."""
    x = np.asarray(x, dtype=np.float64)
    w1 = np.asarray(w1, dtype=np.float64)
    b1 = np.asarray(b1, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    b2 = np.asarray(b2, dtype=np.float64)
    n = x.shape[0]
    step = n if not block_rows else int(block_rows)
    y = np.full((n, w2.shape[0]), np.nan)  # a row no block writes stays NaN
    for r0 in range(0, n, max(step, 1)):
        h = gelu_tanh(x[r0:r0 + step] @ w1.T + b1)
        y[r0:r0 + step] = h @ w2.T + b2
    return y
