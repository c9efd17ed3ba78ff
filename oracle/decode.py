"""Oracle: block-sparse decode attention and its block selection.  TEST INFRASTRUCTURE ONLY.

Source passages:
* Abstract of "SeerAttention-R: Sparse Attention Adaptation for Long Reasoning":
  the method carries the learned block sparsity over to auto-regressive
  decoding (the gate drops query pooling, so it scores blocks for the single new
  token), runs with a token budget (4K tokens) and sparse-attention blocks of 64
  or 128 tokens, and measures a sparse decoding kernel at 90 % sparsity.
* Rebuttal "SeerAttention: Learning Intrinsic Sparse Attention in Your LLMs",
  "Weakness 5 (Pseudo code of Inference Kernel)": attention visits only the
  listed KV blocks (K and V of a step share the block index); as in the prefill
  oracle, the online recurrence is written out as an ordinary softmax over the
  allowed keys.
* Same rebuttal, "Weakness 2 (Memory complexity)": TopK per row, index lists.

Readings where the pages are silent (also in the design notes):
* One new token per sequence.  Its K and V are already in the cache, so with
  ``kv_len[b]`` cached tokens the query sits at position kv_len[b] - 1 and may
  see cache positions 0 .. kv_len[b] - 1 that fall in its listed blocks.
* The cache is [B, Hkv, Tmax, D]; positions >= kv_len[b] do not exist.  Blocks
  are ``block`` tokens (64 or 128); the last block of a sequence may be short.
* Lists have one row per list head: H = Hq (each query head its own list) or
  H = Hkv (the G query heads of a KV group share one list).  Query head h reads
  KV head h // G and list head h (H = Hq) or h // G (H = Hkv).
* List entries outside [0, nb) with nb = ceil(kv_len / block) are skipped; the
  list is read as a set; a row with no valid entry outputs zeros.
* Selection per (b, list head) over the candidate blocks 0 .. nb - 1: the block
  holding the query token (nb - 1) is always kept, block 0 too with
  ``keep_sink``; TopK keeps k = min(nb, max(|forced|, k_blocks)) blocks, with
  k_blocks the token budget divided by the block size; threshold keeps the
  forced blocks and every block whose fp32 score is >= fp32(threshold), cut to
  the best ``max_k`` by (score desc, index asc).  This is the prefill row rule
  of ``mask.select_row`` with row i = nb - 1 and a fixed count instead of a
  density.
"""

from __future__ import annotations

import math
from typing import List, Optional

import numpy as np

from .attention import _f64, allowed_blocks, block_probs
from .mask import MODE_THRESHOLD, MODE_TOPK, _rank


def decode_blocks(kv_len: int, block: int) -> int:
    """Number of (possibly short) blocks holding kv_len cached tokens."""
    return max(0, (int(kv_len) + block - 1) // block)


def select_decode_row(row_scores: np.ndarray, kv_len: int, block: int, mode: int,
                      threshold: float, k_blocks: int, keep_sink: bool,
                      max_k: int) -> List[int]:
    """Selected blocks of one decode row, ascending.  Only scores 0 .. nb-1 are read."""
    nb = decode_blocks(kv_len, block)
    if nb == 0:
        return []
    row = np.asarray(row_scores, dtype=np.float32)
    forced = sorted({nb - 1} | ({0} if keep_sink else set()))
    others = [j for j in range(nb) if j not in forced]
    if mode == MODE_TOPK:
        k = min(nb, max(len(forced), int(k_blocks)))
        if k > max_k:
            raise ValueError(f"decode row needs {k} entries but max_k is {max_k}")
        ranked = sorted(others, key=lambda j: _rank(row[j], j))
        chosen = forced + ranked[: k - len(forced)]
    elif mode == MODE_THRESHOLD:
        tau = np.float32(threshold)
        passing = [j for j in others if bool(row[j] >= tau)]
        room = max_k - len(forced)
        if room < 0:
            raise ValueError(f"max_k {max_k} cannot hold the forced blocks")
        if len(passing) > room:
            passing = sorted(passing, key=lambda j: _rank(row[j], j))[:room]
        chosen = forced + passing
    else:
        raise ValueError(f"unknown mode {mode}")
    return sorted(chosen)


def build_mask_decode_ref(scores: np.ndarray, kv_len, block: int, mode: int,
                          threshold: float, k_blocks: int, keep_sink: bool, max_k: int):
    """Decode lists: scores [B,H,nKB] fp32 -> idx [B,H,max_k] int32 (-1 padded), cnt [B,H]."""
    scores = np.asarray(scores, dtype=np.float32)
    kv_len = np.asarray(kv_len)
    bsz, heads, _ = scores.shape
    idx = np.full((bsz, heads, max_k), -1, dtype=np.int32)
    cnt = np.zeros((bsz, heads), dtype=np.int32)
    for b in range(bsz):
        for h in range(heads):
            sel = select_decode_row(scores[b, h], int(kv_len[b]), block, mode, threshold,
                                    k_blocks, keep_sink, max_k)
            idx[b, h, : len(sel)] = sel
            cnt[b, h] = len(sel)
    return idx, cnt


def sparse_decode_ref(q, k_cache, v_cache, kv_len, idx, cnt, sm_scale: Optional[float] = None,
                      block: int = 64) -> np.ndarray:
    """Decode output O [B,Hq,D] float64 for q [B,Hq,D] over a [B,Hkv,Tmax,D] cache."""
    q = _f64(q)
    kc = _f64(k_cache)
    vc = _f64(v_cache)
    kv_len = np.asarray(kv_len)
    idx = np.asarray(idx)
    cnt = np.asarray(cnt)
    bsz, hq, d = q.shape
    hkv = kc.shape[1]
    group = hq // hkv
    per_query_head = idx.shape[1] == hq
    scale = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    out = np.zeros((bsz, hq, d))
    for b in range(bsz):
        n = int(kv_len[b])
        nb = decode_blocks(n, block)
        for h in range(hq):
            g = h // group
            lh = h if per_query_head else g
            sel = allowed_blocks(idx[b, lh], cnt[b, lh], nb - 1)
            keys = [c for j in sel for c in range(block * j, min(block * j + block, n))]
            if not keys:
                continue
            keys = np.asarray(keys)
            p = block_probs(q[b, h][None, :], kc[b, g][keys], np.array([n - 1]), keys, scale)
            out[b, h] = (p @ vc[b, g][keys])[0]
    return out
