"""Seeded synthetic inputs for the block-sparse prefill path.

This module only draws random numbers and arranges them into tensors.  It
holds none of the arithmetic of the method itself (no mask selection, no
attention, no pooling), so that both the GPU path and the CPU oracle can be fed
from it without sharing any computation.

The shapes follow the attention layers the SeerAttention pages evaluate on
(Llama-3.1-8B: 32 query heads, 8 KV heads, head dim 128; Qwen2.5-32B: 40 query
heads, 8 KV heads), with the block size fixed at 64 (reproducibility summary of
"SeerAttention: Self-distilled Attention Gating for Efficient Long-context
Prefilling", Experiment Setup row).  The densities follow the model card's PG19
and RULER density tables, and the score structure (local window, attention
sink, vertical stripes) follows the attention patterns the rebuttal of
"SeerAttention: Learning Intrinsic Sparse Attention in Your LLMs" reports the
gate learning (answer to "Question 3 (What's the sparsity pattern)").  No
dataset, prompt or trained weight is used: every value is drawn from a seeded
NumPy PCG64 generator.

Seeds: ``seed = 1000 * workload_id + stream`` with stream 0 = Q, 1 = K, 2 = V,
3 = scores, 4 = stripe columns, 5 = sampled query blocks, 6 = block maps,
7 = gate weights.

Decode workloads (one new token per sequence over a KV cache) follow the
abstract of "SeerAttention-R: Sparse Attention Adaptation for Long Reasoning":
a 4K-token budget, blocks of 64 or 128 tokens and 90 % sparsity, here with
Llama-3.1-8B attention shapes.  Same seeding, streams 0-2 = q and the K/V cache,
3 = decode scores, 4 = stripe columns.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

BLOCK = 64

MODE_THRESHOLD = 0
MODE_TOPK = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, mask rule and score recipe."""

    wid: int
    name: str
    batch: int
    hq: int
    hkv: int
    head_dim: int
    seq: int
    kind: str  # "sparse" or "pooled"
    mode: int = MODE_TOPK
    density: float = 1.0
    threshold: float = 0.0
    keep_sink: bool = True
    scores: str = "uniform"  # "uniform" | "softmax_normal" | "local_stripe" | "none"
    qkv_scale: float = 1.0
    sample_qblocks: Optional[int] = None  # per head, for oracle checks at full size
    block: int = BLOCK  # tokens per block of the score grid and the index lists

    @property
    def nqb(self) -> int:
        return (self.seq + self.block - 1) // self.block

    @property
    def groups(self) -> int:
        return self.hq // self.hkv

    def seed(self, stream: int) -> int:
        return 1000 * self.wid + stream


# Tiny case: 2 query heads on 1 KV head, head dim 64, 512 tokens (8x8 blocks).
C1 = Workload(1, "tiny_gqa2_d64_t512_topk0.5", 1, 2, 1, 64, 512, "sparse",
              mode=MODE_TOPK, density=0.5, keep_sink=True, scores="uniform")
# Llama-3.1-8B attention shape at 8k tokens, threshold 2e-3 on softmaxed scores.
C2 = Workload(2, "llama3.1-8b_t8192_threshold2e-3", 1, 32, 8, 128, 8192, "sparse",
              mode=MODE_THRESHOLD, threshold=2e-3, keep_sink=False,
              scores="softmax_normal", qkv_scale=1.0 / math.sqrt(128.0))
# Llama-3.1-8B attention shape at 32k tokens, TopK density 0.1 (90 % sparsity).
C3 = Workload(3, "llama3.1-8b_t32768_topk0.1", 1, 32, 8, 128, 32768, "sparse",
              mode=MODE_TOPK, density=0.1, keep_sink=True, scores="local_stripe",
              sample_qblocks=8)
# Llama-3.1-8B attention shape at 128k tokens, TopK density 0.17.
C4 = Workload(4, "llama3.1-8b_t131072_topk0.17", 1, 32, 8, 128, 131072, "sparse",
              mode=MODE_TOPK, density=0.17, keep_sink=True, scores="local_stripe",
              sample_qblocks=64)
# Qwen2.5-32B attention shape at 32k tokens: dense causal pass with the pooled map.
C5 = Workload(5, "qwen2.5-32b_t32768_pooled_map", 1, 40, 8, 128, 32768, "pooled",
              scores="none", sample_qblocks=4)

WORKLOADS = {w.wid: w for w in (C1, C2, C3, C4, C5)}


def custom(wid: int, batch: int, hq: int, hkv: int, head_dim: int, seq: int, **kw) -> Workload:
    """A workload of arbitrary shape (tests use it for small and ragged cases)."""
    return Workload(wid, kw.pop("name", f"custom{wid}"), batch, hq, hkv, head_dim, seq,
                    kw.pop("kind", "sparse"), **kw)


def _normal_bf16(shape, seed: int, scale: float) -> torch.Tensor:
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    # Round-to-nearest-even to bf16 on the CPU; both sides see these exact bits.
    return torch.from_numpy(x).to(torch.bfloat16)


def make_qkv(w: Workload):
    """Q [B,Hq,T,D], K and V [B,Hkv,T,D] as bf16 CPU tensors (N(0,1) times qkv_scale)."""
    q = _normal_bf16((w.batch, w.hq, w.seq, w.head_dim), w.seed(0), w.qkv_scale)
    k = _normal_bf16((w.batch, w.hkv, w.seq, w.head_dim), w.seed(1), w.qkv_scale)
    v = _normal_bf16((w.batch, w.hkv, w.seq, w.head_dim), w.seed(2), w.qkv_scale)
    return q, k, v


def stripe_columns(w: Workload) -> np.ndarray:
    """Eight distinct KV-block columns per (batch, head) for the vertical-stripe pattern."""
    rng = np.random.Generator(np.random.PCG64(w.seed(4)))
    n = w.nqb
    cols = np.empty((w.batch, w.hq, min(8, n)), dtype=np.int64)
    for b in range(w.batch):
        for h in range(w.hq):
            cols[b, h] = rng.choice(n, size=min(8, n), replace=False)
    return cols


def make_scores(w: Workload) -> torch.Tensor:
    """Soft block scores [B,Hq,nQB,nKB] fp32 standing in for the AttnGate output.

    Only the causal part j <= i is meaningful; entries above the diagonal are 0.
    """
    n = w.nqb
    shape = (w.batch, w.hq, n, n)
    rng = np.random.Generator(np.random.PCG64(w.seed(3)))
    if w.scores == "uniform":
        s = rng.random(size=shape, dtype=np.float32)
    elif w.scores == "softmax_normal":
        # Gate-like rows: softmax over the causal blocks of N(0, std 2) logits,
        # evaluated in float64 and stored as fp32.
        logits = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(2.0)
        causal = np.tril(np.ones((n, n), dtype=bool))
        z = np.where(causal, logits.astype(np.float64), -np.inf)
        z -= z.max(axis=-1, keepdims=True)
        e = np.exp(z)
        s = (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)
    elif w.scores == "local_stripe":
        s = rng.standard_normal(size=shape, dtype=np.float32)
        ii = np.arange(n)[:, None]
        jj = np.arange(n)[None, :]
        s += np.float32(4.0) * (np.abs(ii - jj) <= 4).astype(np.float32)
        cols = stripe_columns(w)
        for b in range(w.batch):
            for h in range(w.hq):
                s[b, h][:, cols[b, h]] += np.float32(4.0)
    elif w.scores == "none":
        return torch.zeros((w.batch, w.hq, 0, 0), dtype=torch.float32)
    else:
        raise ValueError(f"unknown score recipe {w.scores!r}")
    s = np.ascontiguousarray(s, dtype=np.float32)
    s = np.where(np.tril(np.ones((n, n), dtype=bool)), s, np.float32(0.0)).astype(np.float32)
    return torch.from_numpy(np.ascontiguousarray(s))


def make_block_map(w: Workload, seed_stream: int = 6) -> torch.Tensor:
    """A stand-in for a max-pooled block map [B,Hq,nQB,nQB] fp32: U(0,1) on the
    causal entries j <= i (shifted away from 0) and large junk values above the
    diagonal, which consumers of such a map must never read."""
    n = w.nqb
    rng = np.random.Generator(np.random.PCG64(w.seed(seed_stream)))
    a = rng.random(size=(w.batch, w.hq, n, n), dtype=np.float32) + np.float32(1e-3)
    junk = np.float32(1e6) * (np.float32(1.0) + rng.random(size=a.shape, dtype=np.float32))
    causal = np.tril(np.ones((n, n), dtype=bool))
    return torch.from_numpy(np.ascontiguousarray(np.where(causal, a, junk).astype(np.float32)))


def make_gate_weights(w: Workload, dg: int, gain: float = 1.0, seed_stream: int = 7):
    """Random-init AttnGate linear weights: Wq [Hq, D, Dg] and Wk [Hkv, 2D, Dg],
    fp32, N(0, gain^2 / fan_in) (no trained gate weights are used anywhere)."""
    rng = np.random.Generator(np.random.PCG64(w.seed(seed_stream)))
    d = w.head_dim
    wq = (rng.standard_normal(size=(w.hq, d, dg), dtype=np.float32)
          * np.float32(gain / math.sqrt(d)))
    wk = (rng.standard_normal(size=(w.hkv, 2 * d, dg), dtype=np.float32)
          * np.float32(gain / math.sqrt(2 * d)))
    return torch.from_numpy(np.ascontiguousarray(wq)), torch.from_numpy(np.ascontiguousarray(wk))


def sample_qblocks(w: Workload, count: Optional[int] = None) -> np.ndarray:
    """Seeded sampled (b, h, i) query blocks, `count` per head, always including
    the first and the last query block of every head."""
    count = w.sample_qblocks if count is None else count
    rng = np.random.Generator(np.random.PCG64(w.seed(5)))
    out = []
    n = w.nqb
    for b in range(w.batch):
        for h in range(w.hq):
            k = min(count, n)
            picks = set([0, n - 1])
            if k > 2:
                picks.update(rng.choice(np.arange(1, n - 1), size=min(k - 2, max(n - 2, 0)),
                                        replace=False).tolist())
            for i in sorted(picks):
                out.append((b, h, i))
    return np.asarray(out, dtype=np.int64)



@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """One decode step: batch sequences with kv_lens cached tokens each (the last
    being the new token) in a [B, Hkv, tmax, D] cache; block lists per KV head
    (list_heads "kv") or per query head ("q")."""
    wid: int
    name: str
    batch: int
    hq: int
    hkv: int
    head_dim: int
    tmax: int
    kv_lens: tuple
    block: int = BLOCK
    budget_tokens: int = 4096
    list_heads: str = "kv"
    keep_sink: bool = True

    @property
    def nkb(self) -> int:
        return (self.tmax + self.block - 1) // self.block

    @property
    def k_blocks(self) -> int:
        return max(1, self.budget_tokens // self.block)

    @property
    def lh(self) -> int:
        return self.hkv if self.list_heads == "kv" else self.hq

    def seed(self, stream: int) -> int:
        return 1000 * self.wid + stream


# Eight sequences at 40k tokens (a 4K budget is 90 % sparsity), Llama-3.1-8B shape.
DEC1 = DecodeWorkload(11, "llama3.1-8b_decode_b8_kv40960_budget4096", 8, 32, 8, 128, 40960,
                      (40960,) * 8, block=64, budget_tokens=4096, list_heads="kv")
DEC2 = dataclasses.replace(DEC1, wid=12, name="llama3.1-8b_decode_b8_kv40960_budget4096_perhead",
                           list_heads="q")


def make_decode_inputs(dw: DecodeWorkload, tail_nan: bool = False):
    """q [B,Hq,D] and the K/V cache [B,Hkv,tmax,D], bf16 N(0,1) on the CPU.  With
    tail_nan the cache slots past each sequence's length hold NaN, which no
    consumer may read."""
    q = _normal_bf16((dw.batch, dw.hq, dw.head_dim), dw.seed(0), 1.0)
    k = _normal_bf16((dw.batch, dw.hkv, dw.tmax, dw.head_dim), dw.seed(1), 1.0)
    v = _normal_bf16((dw.batch, dw.hkv, dw.tmax, dw.head_dim), dw.seed(2), 1.0)
    if tail_nan:
        for b, n in enumerate(dw.kv_lens):
            k[b, :, n:] = float("nan")
            v[b, :, n:] = float("nan")
    kv_len = torch.tensor(dw.kv_lens, dtype=torch.int32)
    return q, k, v, kv_len


def make_decode_scores(dw: DecodeWorkload) -> torch.Tensor:
    """Decode block scores [B, H, nKB] fp32 (H = list heads): N(0,1) plus 4 on the
    last 4 blocks of the sequence (the local window) and on 8 stripe columns per
    head; entries past the sequence hold 1e6, which selection must never read."""
    lh, nkb = dw.lh, dw.nkb
    rng = np.random.Generator(np.random.PCG64(dw.seed(3)))
    srng = np.random.Generator(np.random.PCG64(dw.seed(4)))
    s = rng.standard_normal(size=(dw.batch, lh, nkb), dtype=np.float32)
    jj = np.arange(nkb)
    for b, n in enumerate(dw.kv_lens):
        nb = (n + dw.block - 1) // dw.block
        s[b] += np.float32(4.0) * ((jj >= nb - 4) & (jj < nb)).astype(np.float32)
        for h in range(lh):
            cols = srng.choice(max(nb, 1), size=min(8, max(nb, 1)), replace=False)
            s[b, h, cols] += np.float32(4.0)
        s[b, :, nb:] = np.float32(1e6)
    return torch.from_numpy(np.ascontiguousarray(s))
