"""The sparse pass at the largest sizes the library takes.

Two sequences of 262144 tokens (4096 query blocks, the longest list row the
mask build accepts), 64 query and 64 KV heads of dimension 128: each of Q, K, V
and O is 8 GiB, so head, row and tile offsets pass 2^31 elements and 2^32
bytes. Every one of the 524288 items gets a short well-formed list (block 0, two
spread earlier blocks and the diagonal block); Q, K and V are zero except seeded
random tiles under the sampled blocks, which the oracle then checks. For each
sampled block the oracle runs on a copy of just that head cut at the block's
end (rows past block i never enter its output), with the same list row.

Lists: rebuttal "SeerAttention: Learning Intrinsic Sparse Attention in Your
LLMs", "Weakness 2 (Memory complexity)" ([Seq/Block, TopK] index lists); the
block-causal attention those lists select: "SeerAttention: Self-distilled
Attention Gating for Efficient Long-context Prefilling", method section.
"""

import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_prefill_amd as seer
import oracle

pytestmark = pytest.mark.gpu

B, H, T, D = 2, 64, 262144, 128
NQB = T // 64
MAX_K = 4
O_TOL = 2e-2


def announce(msg):
    sys.__stderr__.write(f"\n[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def _lists():
    """Row (b, h, i): {0, a spread block, i // 2, i}, deduplicated and ascending."""
    i = np.arange(NQB, dtype=np.int64)[None, None, :]
    h = np.arange(H, dtype=np.int64)[None, :, None]
    b = np.arange(B, dtype=np.int64)[:, None, None]
    shape = (B, H, NQB)
    cols = [np.zeros(shape, np.int64), np.broadcast_to((i * (37 * h + 11) + 5 * b) % (i + 1), shape),
            np.broadcast_to(i // 2, shape), np.broadcast_to(i, shape)]
    arr = np.sort(np.stack(cols, -1), -1)
    big = np.int64(1 << 40)
    dup = np.zeros(arr.shape, bool)
    dup[..., 1:] = arr[..., 1:] == arr[..., :-1]
    arr = np.sort(np.where(dup, big, arr), -1)
    cnt = (arr != big).sum(-1).astype(np.int32)
    idx = np.where(arr == big, -1, arr).astype(np.int32)
    return idx, cnt


def _tile(seed, *key):
    rng = np.random.default_rng([seed, *key])
    return torch.from_numpy(rng.standard_normal((64, D), dtype=np.float32)).to(torch.bfloat16)


def test_sparse_prefill_max_size_offsets():
    announce(f"sparse prefill max size: B={B} H={H} T={T} D={D} (8 GiB per tensor)")
    assert torch.cuda.is_available()
    dev = torch.device("cuda:0")
    idx, cnt = _lists()
    rng = np.random.default_rng(9090)
    blocks = {(0, 0, 0), (1, H - 1, NQB - 1), (0, H - 1, NQB - 1), (1, 0, NQB - 1),
              (1, H - 1, 0), (1, H - 1, NQB // 2)}
    while len(blocks) < 24:
        blocks.add((int(rng.integers(0, B)), int(rng.integers(0, H)), int(rng.integers(0, NQB))))
    blocks = sorted(blocks)

    q = torch.zeros((B, H, T, D), dtype=torch.bfloat16, device=dev)
    k = torch.zeros_like(q)
    v = torch.zeros_like(q)
    filled = set()
    for (b, h, i) in blocks:
        q[b, h, 64 * i: 64 * i + 64] = _tile(1, b, h, i).to(dev)
        for j in idx[b, h, i, : cnt[b, h, i]]:
            if (b, h, int(j)) not in filled:
                filled.add((b, h, int(j)))
                k[b, h, 64 * j: 64 * j + 64] = _tile(2, b, h, int(j)).to(dev)
                v[b, h, 64 * j: 64 * j + 64] = _tile(3, b, h, int(j)).to(dev)

    o = seer.seer_sparse_prefill(q, k, v, torch.from_numpy(idx).to(dev),
                                 torch.from_numpy(cnt).to(dev))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all())

    worst = 0.0
    for (b, h, i) in blocks:
        n = 64 * (i + 1)  # the head cut at the end of block i
        qs = torch.zeros((1, 1, n, D), dtype=torch.bfloat16)
        ks = torch.zeros_like(qs)
        vs = torch.zeros_like(qs)
        qs[0, 0, 64 * i:] = _tile(1, b, h, i)
        for j in idx[b, h, i, : cnt[b, h, i]]:
            ks[0, 0, 64 * j: 64 * j + 64] = _tile(2, b, h, int(j))
            vs[0, 0, 64 * j: 64 * j + 64] = _tile(3, b, h, int(j))
        li = np.full((1, 1, i + 1, MAX_K), -1, np.int32)
        lc = np.zeros((1, 1, i + 1), np.int32)
        li[0, 0, i] = idx[b, h, i]
        lc[0, 0, i] = cnt[b, h, i]
        ref = oracle.sparse_attention_blocks_ref(qs, ks, vs, li, lc, None, [(0, 0, i)])[(0, 0, i)]
        got = o[b, h, 64 * i: 64 * i + 64].double().cpu().numpy()
        err = float(np.abs(got - ref).max())
        worst = max(worst, err)
        assert err <= O_TOL, f"block {(b, h, i)}: max-abs error {err}"
    announce(f"max size: worst max-abs error {worst:.3e} over {len(blocks)} blocks")
    del q, k, v, o
    torch.cuda.empty_cache()
