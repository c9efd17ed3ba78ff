"""Oracle: AttnGate soft block scores (pooling, linear, block RoPE, causal softmax).  TEST INFRASTRUCTURE ONLY.

Source passages:
* Rebuttal "SeerAttention: Learning Intrinsic Sparse Attention in Your LLMs",
  "Weakness 3 (The meaning of "max and min pooling on K matrix" is not clear)":
  pooling runs along the sequence, [Batch, Head, Seq, Dim] -> [Batch, Head,
  Seq / Block, Dim]; with two poolings of K (max and min) the results are
  concatenated along the hidden dimension before the linear layer, giving Dim * 2.
* Same rebuttal, "Question 1 (Theoretical or Intuitive Explanation for Pooling
  Selection)": Q is average-pooled, K max- and min-pooled.
* Same rebuttal, "Q1 More about in AttnGate's RoPE" and "Question 1 (Why RoPE in
  AttnGate?)": the gate pools the Q and K from before the model's RoPE and applies
  its own block-level RoPE after the linear layer.
* Same rebuttal, "Weakness 4 (Rounding Issue when Seq not evenly divided by B)":
  a sequence that is not a multiple of the block is padded as torch pooling does
  with ceil_mode (the last window covers the remaining tokens only).
* Same rebuttal, "Question 2: (Row-Normalization of Max-Pooled Attention Map)":
  the gate's output is a softmax (each row sums to 1).
* Model card "SeerAttention-Llama-3.1-8B-AttnGates", method summary: threshold or
  TopK on these soft scores gives the block mask (seer_build_mask).

Readings where the pages are silent (also in the design notes):
* The linear layers are per head and have no bias: Q~ = avgpool(Q) Wq[h] with Wq[h]
  of shape [D, Dg]; K~ = [maxpool(K) | minpool(K)] Wk[g] with Wk[g] of shape
  [2D, Dg], g the KV head; Dg is a parameter.  Query head h uses KV head h // G.
* Block RoPE is the rotate-half rotary embedding over Dg with frequencies
  base^(-2t/Dg), t = 0 .. Dg/2 - 1, at the block index (i for Q~_i, j for K~_j).
* Scores: s_ij = scale <rope(Q~_i, i), rope(K~_j, j)> for j <= i, softmax over
  j <= i; entries j > i are 0.  scale defaults to 1/sqrt(Dg), base to 10000.

Decode (abstract of "SeerAttention-R: Sparse Attention Adaptation for Long
Reasoning": the gate drops query pooling for decoding and keeps 64- or 128-token
blocks).  Readings where that page is silent: the K side is the prefill gate's
(block max | min pooling of the cached K, a short last block pooling the tokens
it has, the same linear layer and block RoPE at the block index); the new token's
q goes through the same Q linear layer with no pooling and is rotated at its own
block index nb - 1 (nb = ceil(kv_len / block)), which is where the prefill gate
rotates the query block holding that token; the softmax runs over the blocks
j < nb.  Scores are per query head.
"""

from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

from .attention import BLOCK, _f64


def pool_qk(q, k, block: int = BLOCK) -> Tuple[np.ndarray, np.ndarray]:
    """avg-pooled Q [B,Hq,nB,D] and [max | min]-pooled K [B,Hkv,nB,2D], float64."""
    q = _f64(q)
    k = _f64(k)
    seq = q.shape[2]
    nb = (seq + block - 1) // block
    qp = np.stack([q[:, :, block * i: min(block * i + block, seq)].mean(axis=2)
                   for i in range(nb)], axis=2)
    kmax = np.stack([k[:, :, block * i: min(block * i + block, seq)].max(axis=2)
                     for i in range(nb)], axis=2)
    kmin = np.stack([k[:, :, block * i: min(block * i + block, seq)].min(axis=2)
                     for i in range(nb)], axis=2)
    return qp, np.concatenate([kmax, kmin], axis=-1)


def block_rope(x: np.ndarray, base: float = 10000.0) -> np.ndarray:
    """Rotate-half RoPE of x [..., nB, Dg] at positions 0 .. nB-1 (the block index)."""
    nb, dg = x.shape[-2], x.shape[-1]
    half = dg // 2
    inv = base ** (-2.0 * np.arange(half) / dg)
    ang = np.arange(nb)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def gate_qk_ref(q, k, wq, wk, base: float = 10000.0, block: int = BLOCK
                ) -> Tuple[np.ndarray, np.ndarray]:
    """Q~ [B,Hq,nB,Dg] and K~ [B,Hkv,nB,Dg] after pooling, linear and block RoPE."""
    qp, kp = pool_qk(q, k, block)
    wq = np.asarray(wq, dtype=np.float64)
    wk = np.asarray(wk, dtype=np.float64)
    qt = block_rope(np.einsum("bhnd,hde->bhne", qp, wq), base)
    kt = block_rope(np.einsum("bgnd,gde->bgne", kp, wk), base)
    return qt, kt


def gate_scores_ref(q, k, wq, wk, scale: Optional[float] = None, base: float = 10000.0,
                    block: int = BLOCK) -> np.ndarray:
    """Soft block scores [B,Hq,nB,nB] float64 (rows sum to 1 over j <= i, 0 above)."""
    qt, kt = gate_qk_ref(q, k, wq, wk, base, block)
    grp = qt.shape[1] // kt.shape[1]
    dg = qt.shape[-1]
    sc = 1.0 / math.sqrt(dg) if scale is None else float(scale)
    kt = np.repeat(kt, grp, axis=1)
    s = sc * np.einsum("bhie,bhje->bhij", qt, kt)
    nb = s.shape[-1]
    causal = np.tril(np.ones((nb, nb), dtype=bool))
    s = np.where(causal, s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    e = np.where(causal, np.exp(s), 0.0)
    return e / e.sum(axis=-1, keepdims=True)


def rope_at(x: np.ndarray, pos, base: float = 10000.0) -> np.ndarray:
    """Rotate-half RoPE of x [..., Dg] at position(s) pos (broadcast over the leading dims)."""
    dg = x.shape[-1]
    half = dg // 2
    inv = base ** (-2.0 * np.arange(half) / dg)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def decode_gate_scores_ref(q, k_cache, kv_len, wq, wk, block: int = BLOCK,
                           scale: Optional[float] = None, base: float = 10000.0) -> np.ndarray:
    """Per-token gate scores [B,Hq,nKB] float64 (nKB = ceil(Tmax / block)) for the new
    token of each sequence: q [B,Hq,D] (no pooling), the cache K [B,Hkv,Tmax,D] of which
    the first kv_len[b] tokens exist.  Row (b, h) sums to 1 over j < nb and is 0 beyond
    (all 0 when kv_len[b] = 0)."""
    q = _f64(q)
    kc = _f64(k_cache)
    kv_len = np.asarray(kv_len)
    wq = np.asarray(wq, dtype=np.float64)
    wk = np.asarray(wk, dtype=np.float64)
    bsz, hq, _ = q.shape
    hkv, tmax = kc.shape[1], kc.shape[2]
    grp = hq // hkv
    nkb = (tmax + block - 1) // block
    dg = wq.shape[-1]
    sc = 1.0 / math.sqrt(dg) if scale is None else float(scale)
    out = np.zeros((bsz, hq, nkb))
    for b in range(bsz):
        n = int(kv_len[b])
        nb = (n + block - 1) // block
        if nb == 0:
            continue
        _, kp = pool_qk(kc[b:b + 1, :, :n], kc[b:b + 1, :, :n], block)  # K pooling only
        kt = block_rope(np.einsum("gnd,gde->gne", kp[0], wk), base)      # [Hkv, nb, Dg]
        for h in range(hq):
            qt = rope_at(q[b, h] @ wq[h], nb - 1, base)
            s = sc * (kt[h // grp] @ qt)
            e = np.exp(s - s.max())
            out[b, h, :nb] = e / e.sum()
    return out
