"""Pins for the decode oracles against things other than themselves: torch SDPA in
float64 with the block lists expanded to a boolean mask, closed forms (Q = 0,
one-hot logits), GQA list sharing, and for the decode selection an exhaustive
enumeration of top-k subsets on small rows with ties, NaN and signed zeros."""

import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import decode as od


def _cache(seed, b, hq, hkv, tmax, d):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(b, hq, d, generator=g).to(torch.bfloat16)
    k = torch.randn(b, hkv, tmax, d, generator=g).to(torch.bfloat16)
    v = torch.randn(b, hkv, tmax, d, generator=g).to(torch.bfloat16)
    return q, k, v


def _random_decode_lists(seed, kv_len, heads, block, max_k, junk=True):
    """Per (b, list head) a random set of valid blocks (any order), sometimes with
    entries outside [0, nb) that the definition skips, -1 padded."""
    rng = np.random.default_rng(seed)
    bsz = len(kv_len)
    idx = np.full((bsz, heads, max_k), -1, np.int32)
    cnt = np.zeros((bsz, heads), np.int32)
    for b in range(bsz):
        nb = od.decode_blocks(kv_len[b], block)
        for h in range(heads):
            m = int(rng.integers(0, min(nb, max_k - 1) + 1))
            sel = [int(x) for x in rng.choice(nb, size=m, replace=False)] if m else []
            if junk and len(sel) < max_k and rng.random() < 0.5:
                sel.append(nb + int(rng.integers(0, 3)))  # past the sequence: skipped
            rng.shuffle(sel)
            idx[b, h, : len(sel)] = sel
            cnt[b, h] = len(sel)
    return idx, cnt


def _sdpa_decode(q, k, v, kv_len, idx, cnt, scale, block):
    """Library reference: SDPA (float64, CPU) of each query over the whole cache with a
    boolean mask = listed blocks intersected with positions < kv_len.  Rows with no
    allowed key are zero by definition (SDPA would return NaN there)."""
    bsz, hq, d = q.shape
    hkv, tmax = k.shape[1], k.shape[2]
    grp = hq // hkv
    per_head = idx.shape[1] == hq
    out = torch.zeros(bsz, hq, d, dtype=torch.float64)
    pos = torch.arange(tmax)
    for b in range(bsz):
        for h in range(hq):
            lh = h if per_head else h // grp
            blk = torch.zeros(tmax, dtype=torch.bool)
            for j in idx[b, lh, : cnt[b, lh]]:
                if j >= 0:
                    blk |= (pos // block) == int(j)
            allow = blk & (pos < int(kv_len[b]))
            if not allow.any():
                continue
            o = F.scaled_dot_product_attention(
                q[b, h].double()[None, None, None, :], k[b, h // grp].double()[None, None],
                v[b, h // grp].double()[None, None], attn_mask=allow[None, None, None, :],
                scale=scale)
            out[b, h] = o[0, 0, 0]
    return out.numpy()


@pytest.mark.parametrize("block", [64, 128])
@pytest.mark.parametrize("shared", [False, True])
def test_decode_matches_sdpa_with_block_mask(block, shared):
    b, hq, hkv, tmax, d = 3, 4, 2, 700, 32
    q, k, v = _cache(10 + block + shared, b, hq, hkv, tmax, d)
    kv_len = np.array([700, 1, 333], np.int64)  # full, a single token, ragged
    heads = hkv if shared else hq
    idx, cnt = _random_decode_lists(20 + block, kv_len, heads, block, 8)
    scale = 0.3
    got = od.sparse_decode_ref(q, k, v, kv_len, idx, cnt, scale, block)
    want = _sdpa_decode(q, k, v, kv_len, idx, cnt, scale, block)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_decode_equals_last_prefill_row():
    """Decoding the token at position T - 1 with query block nQB - 1's list gives the
    last output row of the prefill definition (causality changes nothing there)."""
    b, hq, hkv, t, d = 1, 2, 1, 300, 16
    g = torch.Generator().manual_seed(3)
    qf = torch.randn(b, hq, t, d, generator=g).to(torch.bfloat16)
    kf = torch.randn(b, hkv, t, d, generator=g).to(torch.bfloat16)
    vf = torch.randn(b, hkv, t, d, generator=g).to(torch.bfloat16)
    nqb = (t + 63) // 64
    rng = np.random.default_rng(4)
    idx = np.full((b, hq, nqb, nqb), -1, np.int32)
    cnt = np.zeros((b, hq, nqb), np.int32)
    for h in range(hq):
        for i in range(nqb):
            sel = sorted({i} | set(int(x) for x in rng.choice(i + 1, size=min(2, i + 1),
                                                               replace=False)))
            idx[0, h, i, : len(sel)] = sel
            cnt[0, h, i] = len(sel)
    pre = oracle.sparse_attention_ref(qf, kf, vf, idx, cnt)
    dec = od.sparse_decode_ref(qf[:, :, t - 1], kf, vf, np.array([t]), idx[:, :, nqb - 1],
                               cnt[:, :, nqb - 1])
    np.testing.assert_allclose(dec, pre[:, :, t - 1], rtol=0, atol=1e-12)


def test_zero_query_is_mean_of_listed_values():
    b, hq, hkv, tmax, d, block = 2, 2, 1, 400, 8, 64
    _, k, v = _cache(5, b, hq, hkv, tmax, d)
    q = torch.zeros(b, hq, d, dtype=torch.bfloat16)
    kv_len = np.array([400, 130])
    idx, cnt = _random_decode_lists(6, kv_len, hq, block, 5, junk=True)
    got = od.sparse_decode_ref(q, k, v, kv_len, idx, cnt, None, block)
    vv = v.double().numpy()
    for bb in range(b):
        nb = od.decode_blocks(kv_len[bb], block)
        for h in range(hq):
            sel = {int(j) for j in idx[bb, h, : cnt[bb, h]] if 0 <= j < nb}
            keys = [c for c in range(int(kv_len[bb])) if c // block in sel]
            want = vv[bb, 0, keys].mean(axis=0) if keys else np.zeros(d)
            np.testing.assert_allclose(got[bb, h], want, rtol=0, atol=1e-12)


def test_one_hot_logit_limit_picks_that_value():
    """A key whose logit exceeds all others by far takes all the weight."""
    d, block, tmax = 4, 64, 200
    k = torch.zeros(1, 1, tmax, d)
    v = torch.arange(tmax * d, dtype=torch.float64).reshape(1, 1, tmax, d)
    k[0, 0, 150, 0] = 1.0
    q = torch.tensor([[[1.0, 0, 0, 0]]])
    idx = np.array([[[0, 2, -1]]], np.int32)
    cnt = np.array([[2]], np.int32)
    got = od.sparse_decode_ref(q, k, v, np.array([199]), idx, cnt, 1e4, block)
    np.testing.assert_allclose(got[0, 0], v[0, 0, 150].numpy(), rtol=0, atol=1e-9)
    # position 150 beyond kv_len: block 2 holds only 128 .. 149, whose logits tie
    got = od.sparse_decode_ref(q, k, v, np.array([150]), idx, cnt, 1e4, block)
    keys = list(range(0, 64)) + list(range(128, 150))
    np.testing.assert_allclose(got[0, 0], v[0, 0, keys].mean(axis=0).numpy(), rtol=0,
                               atol=1e-9)


def test_shared_lists_equal_repeated_per_head_lists():
    b, hq, hkv, tmax, d, block = 2, 6, 2, 500, 16, 128
    q, k, v = _cache(7, b, hq, hkv, tmax, d)
    kv_len = np.array([500, 257])
    idx, cnt = _random_decode_lists(8, kv_len, hkv, block, 4)
    shared = od.sparse_decode_ref(q, k, v, kv_len, idx, cnt, None, block)
    rep = od.sparse_decode_ref(q, k, v, kv_len, np.repeat(idx, hq // hkv, axis=1),
                               np.repeat(cnt, hq // hkv, axis=1), None, block)
    np.testing.assert_array_equal(shared, rep)


def _better(sc, a, b):
    fa = -math.inf if math.isnan(sc[a]) else float(sc[a])
    fb = -math.inf if math.isnan(sc[b]) else float(sc[b])
    return fa > fb or (fa == fb and a < b)


@pytest.mark.parametrize("seed", range(4))
def test_decode_topk_is_the_unique_exchange_optimal_subset(seed):
    """Every subset of the right size holding the forced blocks (last block, sink)
    is enumerated; exactly one may be exchange-optimal and it must be the oracle's."""
    rng = np.random.default_rng(seed)
    nkb, block = 9, 64
    s = rng.choice(np.array([0.1, 0.2, 0.2, 0.5, -0.0, 0.0, np.nan, 0.9], np.float32),
                   size=nkb).astype(np.float32)
    for kv_len in (1, 64, 65, 200, 576):
        nb = od.decode_blocks(kv_len, block)
        for sink in (False, True):
            forced = {nb - 1} | ({0} if sink else set())
            for kb in (1, 2, 4, 9):
                got = od.select_decode_row(s, kv_len, block, oracle.MODE_TOPK, 0.0, kb, sink, nkb)
                k = min(nb, max(len(forced), kb))
                free = [j for j in range(nb) if j not in forced]
                winners = []
                for extra in itertools.combinations(free, k - len(forced)):
                    ch = sorted(forced | set(extra))
                    out = [j for j in range(nb) if j not in ch]
                    if all(_better(s, a, o) for a in extra for o in out):
                        winners.append(ch)
                assert winners == [got], (seed, kv_len, sink, kb)


def test_decode_threshold_and_empty_rows():
    s = np.array([0.5, 0.1, 0.7, np.nan, 0.3, 0.9], np.float32)
    # kv_len 300 -> 5 blocks (0..4): forced {4}; passing >= 0.3: 0, 2 (4 is forced)
    assert od.select_decode_row(s, 300, 64, oracle.MODE_THRESHOLD, 0.3, 0, False, 6) == [0, 2, 4]
    # cut to max_k = 2: forced 4 plus the best passing block (2, score 0.7)
    assert od.select_decode_row(s, 300, 64, oracle.MODE_THRESHOLD, 0.3, 0, False, 2) == [2, 4]
    # block 5's score is never read: kv_len 300 has 5 blocks
    assert od.select_decode_row(s, 300, 64, oracle.MODE_TOPK, 0.0, 3, True, 6) == [0, 2, 4]
    assert od.select_decode_row(s, 0, 64, oracle.MODE_TOPK, 0.0, 3, True, 6) == []
    idx, cnt = od.build_mask_decode_ref(s[None, None], [0], 64, oracle.MODE_TOPK, 0.0, 3, True, 4)
    assert cnt.tolist() == [[0]] and idx.tolist() == [[[-1, -1, -1, -1]]]


def test_decode_row_equals_prefill_row_rule():
    """With kv_len = 64 (i + 1) the decode row is prefill row i's rule at a count
    that a density reproduces exactly (k / (i + 1) with i + 1 a power of two)."""
    rng = np.random.default_rng(11)
    for n in (1, 2, 4, 8, 16, 32):
        s = rng.random(n).astype(np.float32)
        for k in range(1, n + 1):
            dens = k / n
            for sink in (False, True):
                pre = oracle.select_row(s, n - 1, oracle.MODE_TOPK, 0.0, dens, sink, n)
                dec = od.select_decode_row(s, 64 * n, 64, oracle.MODE_TOPK, 0.0, k, sink, n)
                assert pre == dec, (n, k, sink)
