"""Oracle: dense causal attention plus the 2D max-pooled attention map.  TEST INFRASTRUCTURE ONLY.

Source passages:
* Reproducibility summary of "SeerAttention: Self-distilled Attention Gating for
  Efficient Long-context Prefilling", Pseudocode row, Figure 8: a flash
  attention pass that stores the block row maxima r_ij, then, once the final
  m_i and l_i are known, rescales them as exp(r_ij - m_i) / l_i and takes the
  column max, returning O and A.  Same page, Open Datasets row: the kernel
  outputs the 2D max-pooled attention map as ground truth.
* Model card "SeerAttention-Llama-3.1-8B-AttnGates", method summary: the gates
  learn the 2D max-pooled attention patterns of the frozen model.

exp(r_ij[r] - m_r) / l_r is the largest softmax probability of row r inside KV
block j, and the column max over the rows of query block i makes A_ij the
largest probability of the whole 64x64 tile.  That plain definition is what this
oracle writes out: full causal softmax rows, then a max over every tile.

Readings (also in the design notes):
* A_ij covers j <= i; tiles above the diagonal are 0.
* The map is the raw max probability; the row normalisation of the rebuttal's
  "Question 2: (Row-Normalization of Max-Pooled Attention Map)" is a separate
  later step and is not applied here.
* For a short last block (T not a multiple of 64) only existing rows and keys
  take part in the max.
"""

from __future__ import annotations

import math
from typing import Dict, Iterable, Optional, Tuple

import numpy as np

from .attention import BLOCK, _f64, block_probs


def pooled_map_blocks_ref(q, k, v, sm_scale: Optional[float],
                          blocks: Iterable[Tuple[int, int, int]]
                          ) -> Dict[Tuple[int, int, int], Tuple[np.ndarray, np.ndarray]]:
    """{(b, h, i): (O_i [rows, D], A_i [nQB])} for selected query blocks."""
    bsz, hq, seq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    nqb = (seq + BLOCK - 1) // BLOCK
    scale = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    out = {}
    for (b, h, i) in blocks:
        b, h, i = int(b), int(h), int(i)
        g = h // group
        r0, r1 = BLOCK * i, min(BLOCK * i + BLOCK, seq)
        rows = np.arange(r0, r1)
        keys = np.arange(0, r1)
        p = block_probs(_f64(q[b, h, r0:r1]), _f64(k[b, g, :r1]), rows, keys, scale)
        o = p @ _f64(v[b, g, :r1])
        a = np.zeros((nqb,))
        for j in range(i + 1):
            a[j] = p[:, BLOCK * j: min(BLOCK * j + BLOCK, r1)].max()
        out[(b, h, i)] = (o, a)
    return out


def pooled_map_ref(q, k, v, sm_scale: Optional[float] = None):
    """O [B,Hq,T,D] and A [B,Hq,nQB,nQB] (float64) of the dense causal pass."""
    bsz, hq, seq, d = q.shape
    nqb = (seq + BLOCK - 1) // BLOCK
    blocks = [(b, h, i) for b in range(bsz) for h in range(hq) for i in range(nqb)]
    res = pooled_map_blocks_ref(q, k, v, sm_scale, blocks)
    o = np.zeros((bsz, hq, seq, d))
    a = np.zeros((bsz, hq, nqb, nqb))
    for (b, h, i), (oi, ai) in res.items():
        o[b, h, BLOCK * i: BLOCK * i + oi.shape[0]] = oi
        a[b, h, i] = ai
    return o, a
