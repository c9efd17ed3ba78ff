"""Oracle: per-row block selection (threshold or TopK).  TEST INFRASTRUCTURE ONLY.

Source passages:
* Model card "SeerAttention-Llama-3.1-8B-AttnGates", method summary: the gates
  turn their soft block scores into a block-sparse binary mask by threshold or
  TopK.
* Rebuttal "SeerAttention: Learning Intrinsic Sparse Attention in Your LLMs",
  "Weakness 2 (Memory complexity)": TopK is taken per row (per query block), and
  the selection is stored as a [Seq/Block, TopK] index tensor per head.
* Same rebuttal, "Weakness 1 (How to choose sparsity?)": the TopK budget is a
  user-chosen knob.
* Reproducibility summary of "SeerAttention: Self-distilled Attention Gating for
  Efficient Long-context Prefilling", Experiment Setup row: thresholds 2e-3,
  5e-4 and 3e-2 are used.

Readings where the pages are silent (each also listed in the design notes):
* Candidates of query block i are the causal KV blocks 0..i.
* Forced blocks F_i = {i} (the diagonal, which guarantees every query row has a
  key) plus {0} when ``keep_sink`` is set.  Forced blocks always survive.
* TopK count k_i = min(i + 1, max(|F_i|, ceil(density * (i + 1)))), with the
  product and the ceiling evaluated in IEEE double precision.
* Ranking of the non-forced candidates: score descending, ties by lower block
  index; a NaN score ranks as -inf.
* Threshold: keep non-forced j with fp32(score) >= fp32(threshold) (NaN never
  passes).  If F_i plus the passing blocks exceed ``max_k``, the passing
  blocks are cut to the ``max_k - |F_i|`` best by the ranking above.
* The list of each row is written in ascending block order and padded with -1
  up to ``max_k``; ``cnt`` holds the list length.
* A row's "need" is the number of blocks the rule selects before any cut to
  ``max_k``: k_i under TopK, |F_i| plus every passing block under threshold.  A
  threshold row whose need exceeds ``max_k`` is the capacity overflow the
  library reports.

List validation (what the sparse calls require of a list, and what a cut
threshold row looks like) follows the same [Seq/Block, TopK] index layout of
"Weakness 2 (Memory complexity)": row r of a head may hold blocks 0..r; the
calls read a count clamped to [0, max_k], skip entries outside [0, r], and
accept any order, but a block listed twice would be accumulated twice.
"""

from __future__ import annotations

import math
from typing import Dict, Iterable, List, Tuple

import numpy as np

MODE_THRESHOLD = 0
MODE_TOPK = 1


def forced_blocks(i: int, keep_sink: bool) -> List[int]:
    """The blocks a row keeps whatever its scores: diagonal, plus block 0 on request."""
    f = {i}
    if keep_sink:
        f.add(0)
    return sorted(f)


def topk_count(i: int, density: float, keep_sink: bool) -> int:
    """Number of KV blocks query block i keeps under TopK at the given density."""
    f = len(forced_blocks(i, keep_sink))
    return min(i + 1, max(f, math.ceil(float(density) * float(i + 1))))


def _rank(score, j: int) -> Tuple[float, int]:
    s = float(score)
    if math.isnan(s):
        s = -math.inf
    return (-s, j)


def select_row(row_scores: np.ndarray, i: int, mode: int, threshold: float,
               density: float, keep_sink: bool, max_k: int) -> List[int]:
    """Selected KV blocks of query block i, ascending.

    ``row_scores`` is the fp32 score row; only entries 0..i are looked at.
    """
    row = np.asarray(row_scores, dtype=np.float32)
    forced = forced_blocks(i, keep_sink)
    others = [j for j in range(i + 1) if j not in forced]
    if mode == MODE_TOPK:
        k = topk_count(i, density, keep_sink)
        if k > max_k:
            raise ValueError(f"row {i} needs {k} entries but max_k is {max_k}")
        ranked = sorted(others, key=lambda j: _rank(row[j], j))
        chosen = forced + ranked[: k - len(forced)]
    elif mode == MODE_THRESHOLD:
        tau = np.float32(threshold)
        passing = [j for j in others if bool(row[j] >= tau)]
        room = max_k - len(forced)
        if room < 0:
            raise ValueError(f"max_k {max_k} cannot hold the forced blocks of row {i}")
        if len(passing) > room:
            passing = sorted(passing, key=lambda j: _rank(row[j], j))[:room]
        chosen = forced + passing
    else:
        raise ValueError(f"unknown mode {mode}")
    return sorted(chosen)


def row_need(row_scores: np.ndarray, i: int, mode: int, threshold: float, density: float,
             keep_sink: bool) -> int:
    """Blocks query block i selects before any cut to max_k."""
    row = np.asarray(row_scores, dtype=np.float32)
    forced = forced_blocks(i, keep_sink)
    if mode == MODE_TOPK:
        return topk_count(i, density, keep_sink)
    tau = np.float32(threshold)
    return len(forced) + sum(1 for j in range(i + 1) if j not in forced and bool(row[j] >= tau))


def build_mask_need_ref(scores: np.ndarray, mode: int, threshold: float, density: float,
                        keep_sink: bool, max_k: int):
    """build_mask_ref plus need [B,H,nQB] int32 (see row_need)."""
    idx, cnt = build_mask_ref(scores, mode, threshold, density, keep_sink, max_k)
    scores = np.asarray(scores, dtype=np.float32)
    bsz, heads, nqb, _ = scores.shape
    need = np.zeros((bsz, heads, nqb), dtype=np.int32)
    for b in range(bsz):
        for h in range(heads):
            for i in range(nqb):
                need[b, h, i] = row_need(scores[b, h, i], i, mode, threshold, density, keep_sink)
    return idx, cnt, need


LIST_BAD_COUNT = 1   # cnt < 0 or cnt > max_k
LIST_BAD_ENTRY = 2   # a counted entry outside [0, r]
LIST_REPEAT = 4      # a block counted twice in one row
LIST_UNSORTED = 8    # counted entries not strictly ascending
LIST_CAPACITY = 16   # need > max_k


def validate_row_ref(entries, count: int, r: int, max_k: int, need=None) -> int:
    """Flag bits of one list row r (entries: the row's max_k stored values)."""
    f = 0
    if count < 0 or count > max_k:
        f |= LIST_BAD_COUNT
    if need is not None and need > max_k:
        f |= LIST_CAPACITY
    n = min(max(count, 0), max_k)
    seen = set()
    for x in range(n):
        e = int(entries[x])
        if e < 0 or e > r:
            f |= LIST_BAD_ENTRY
        elif e in seen:
            f |= LIST_REPEAT
        else:
            seen.add(e)
        if x > 0 and e <= int(entries[x - 1]):
            f |= LIST_UNSORTED
    return f


def validate_lists_ref(idx: np.ndarray, cnt: np.ndarray, need, max_k: int):
    """Per-row flags [B,H,nB] and their OR over all rows."""
    idx = np.asarray(idx)
    cnt = np.asarray(cnt)
    bsz, heads, nb = cnt.shape
    flags = np.zeros((bsz, heads, nb), dtype=np.int32)
    for b in range(bsz):
        for h in range(heads):
            for r in range(nb):
                nd = None if need is None else int(np.asarray(need)[b, h, r])
                flags[b, h, r] = validate_row_ref(idx[b, h, r], int(cnt[b, h, r]), r, max_k, nd)
    return flags, int(np.bitwise_or.reduce(flags.reshape(-1))) if flags.size else 0


def build_mask_ref(scores: np.ndarray, mode: int, threshold: float, density: float,
                   keep_sink: bool, max_k: int):
    """Index lists for every row: idx [B,H,nQB,max_k] int32 (-1 padded), cnt [B,H,nQB]."""
    scores = np.asarray(scores, dtype=np.float32)
    bsz, heads, nqb, _ = scores.shape
    idx = np.full((bsz, heads, nqb, max_k), -1, dtype=np.int32)
    cnt = np.zeros((bsz, heads, nqb), dtype=np.int32)
    for b in range(bsz):
        for h in range(heads):
            for i in range(nqb):
                sel = select_row(scores[b, h, i], i, mode, threshold, density, keep_sink, max_k)
                idx[b, h, i, : len(sel)] = sel
                cnt[b, h, i] = len(sel)
    return idx, cnt


def mask_rows_ref(scores: np.ndarray, rows: Iterable[Tuple[int, int, int]], mode: int,
                  threshold: float, density: float, keep_sink: bool,
                  max_k: int) -> Dict[Tuple[int, int, int], List[int]]:
    """Selected lists of a few rows only (for the large workloads)."""
    scores = np.asarray(scores)
    out = {}
    for (b, h, i) in rows:
        b, h, i = int(b), int(h), int(i)
        out[(b, h, i)] = select_row(scores[b, h, i], i, mode, threshold, density,
                                    keep_sink, max_k)
    return out
