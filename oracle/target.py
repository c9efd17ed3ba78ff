"""Oracle: row-normalised distillation target and its MSE against gate scores.  TEST INFRASTRUCTURE ONLY.

Source passages:
* Rebuttal "SeerAttention: Learning Intrinsic Sparse Attention in Your LLMs",
  "Question 2: (Row-Normalization of Max-Pooled Attention Map)": the max-pooled
  attention map is normalised per row so that, like the gate's softmax output,
  every row sums to 1; that normalised map is the ground truth the gate learns.
* Same rebuttal, "Question 2 (Currently use MSE loss, how about e2e LM loss?)":
  the gate is trained with an MSE loss against that ground truth.
* Reproducibility summary of "SeerAttention: Self-distilled Attention Gating for
  Efficient Long-context Prefilling", Pseudocode row, Figure 8: the map itself
  (A, one max probability per 64x64 causal tile).

Readings (also in the design notes):
* Row i of a map has causal entries j <= i; the normalisation divides them by
  their sum and leaves the entries j > i at 0.
* The MSE runs over the causal entries only (the gate's softmax has no mass on
  j > i either): loss = sum over every (b, h, i, j <= i) of (g - t)^2 divided by
  the number of such entries.  Per-row sums of squared errors are returned too.
* A row whose causal entries sum to 0 (impossible for a map of probabilities,
  whose diagonal entry is positive) normalises to all zeros.
"""

from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def pooled_target_ref(amap: np.ndarray, gate: Optional[np.ndarray] = None
                      ) -> Tuple[np.ndarray, Optional[np.ndarray], Optional[float]]:
    """amap [B,H,nQB,nQB] -> (target, row_sse [B,H,nQB] or None, loss or None), float64."""
    a = np.asarray(amap, dtype=np.float64)
    b, h, nqb, nkb = a.shape
    causal = np.tril(np.ones((nqb, nkb), dtype=bool))
    a = np.where(causal, a, 0.0)
    sums = a.sum(axis=-1, keepdims=True)
    target = np.divide(a, sums, out=np.zeros_like(a), where=sums != 0.0)
    if gate is None:
        return target, None, None
    g = np.where(causal, np.asarray(gate, dtype=np.float64), 0.0)
    sq = np.where(causal, (g - target) ** 2, 0.0)
    row_sse = sq.sum(axis=-1)
    count = b * h * int(causal.sum())
    loss = float(row_sse.sum() / count) if count else 0.0
    return target, row_sse, loss
