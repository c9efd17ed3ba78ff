"""Pins for the attention and pooled-map oracles against library routines
(torch scaled_dot_product_attention, torch softmax + max_pool2d in float64 on the
CPU), closed forms and limit cases."""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

BLOCK = 64


def _inputs(seed, b, hq, hkv, t, d, q_zero=False):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(b, hq, t, d, generator=g).to(torch.bfloat16)
    k = torch.randn(b, hkv, t, d, generator=g).to(torch.bfloat16)
    v = torch.randn(b, hkv, t, d, generator=g).to(torch.bfloat16)
    if q_zero:
        q = torch.zeros_like(q)
    return q, k, v


def _random_lists(seed, b, h, nqb, max_k, keep_diag=True):
    rng = np.random.default_rng(seed)
    idx = np.full((b, h, nqb, max_k), -1, np.int32)
    cnt = np.zeros((b, h, nqb), np.int32)
    for bb in range(b):
        for hh in range(h):
            for i in range(nqb):
                pool = [j for j in range(i + 1) if not (keep_diag and j == i)]
                m = int(rng.integers(0, min(len(pool), max_k - 1) + 1)) if pool else 0
                sel = list(rng.choice(pool, size=m, replace=False)) if m else []
                if keep_diag:
                    sel.append(i)
                rng.shuffle(sel)
                idx[bb, hh, i, : len(sel)] = sel
                cnt[bb, hh, i] = len(sel)
    return idx, cnt


def _sdpa_with_blocks(q, k, v, idx, cnt, scale, block=BLOCK):
    """Library reference: SDPA (float64, CPU) with the block list expanded to a
    boolean mask and intersected with causality; GQA by repeating KV heads."""
    b, hq, t, d = q.shape
    grp = hq // k.shape[1]
    kk = k.double().repeat_interleave(grp, dim=1)
    vv = v.double().repeat_interleave(grp, dim=1)
    nqb = (t + block - 1) // block
    allow = torch.zeros(b, hq, t, t, dtype=torch.bool)
    pos = torch.arange(t)
    causal = pos[None, :] <= pos[:, None]
    for bb in range(b):
        for hh in range(hq):
            bm = torch.zeros(nqb, nqb, dtype=torch.bool)
            for i in range(nqb):
                for j in idx[bb, hh, i, : cnt[bb, hh, i]]:
                    if 0 <= j <= i:
                        bm[i, j] = True
            allow[bb, hh] = bm.repeat_interleave(block, 0).repeat_interleave(block, 1)[:t, :t] & causal
    out = F.scaled_dot_product_attention(q.double(), kk, vv, attn_mask=allow, scale=scale)
    empty = ~allow.any(dim=-1)
    out[empty] = 0.0
    return out.numpy()


@pytest.mark.parametrize("t,block", [(200, 64), (256, 64), (300, 128), (256, 128)])
def test_density_one_equals_dense_causal_sdpa(t, block):
    b, hq, hkv, d = 1, 4, 2, 64
    q, k, v = _inputs(1, b, hq, hkv, t, d)
    nqb = (t + block - 1) // block
    idx = np.tile(np.arange(nqb, dtype=np.int32), (b, hq, nqb, 1))
    cnt = np.tile(np.arange(1, nqb + 1, dtype=np.int32), (b, hq, 1))
    o = oracle.sparse_attention_ref(q, k, v, idx, cnt, None, block)
    kk = k.double().repeat_interleave(hq // hkv, dim=1)
    vv = v.double().repeat_interleave(hq // hkv, dim=1)
    ref = F.scaled_dot_product_attention(q.double(), kk, vv, is_causal=True).numpy()
    np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)


@pytest.mark.parametrize("seed,block", [(2, 64), (3, 64), (4, 128), (5, 128)])
def test_block_mask_equals_sdpa_with_expanded_mask(seed, block):
    b, hq, hkv, t, d = 2, 4, 2, 300 if block == 64 else 700, 32
    q, k, v = _inputs(seed, b, hq, hkv, t, d)
    nqb = (t + block - 1) // block
    idx, cnt = _random_lists(seed, b, hq, nqb, nqb)
    scale = 0.3
    o = oracle.sparse_attention_ref(q, k, v, idx, cnt, scale, block)
    ref = _sdpa_with_blocks(q, k, v, idx, cnt, scale, block)
    np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)


def test_rows_without_diagonal_and_empty_rows_and_invalid_entries():
    b, hq, hkv, t, d = 1, 2, 1, 192, 16
    q, k, v = _inputs(5, b, hq, hkv, t, d)
    nqb = 3
    idx = np.full((b, hq, nqb, 4), -1, np.int32)
    cnt = np.zeros((b, hq, nqb), np.int32)
    idx[0, 0, 2, :3] = [0, 7, -3]     # only block 0 valid
    cnt[0, 0, 2] = 3
    idx[0, 1, 1, :2] = [5, 1]         # only the diagonal valid
    cnt[0, 1, 1] = 2
    o = oracle.sparse_attention_ref(q, k, v, idx, cnt, None)
    ref = _sdpa_with_blocks(q, k, v, idx, cnt, 1 / math.sqrt(d))
    np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)
    assert (o[0, 0, :128] == 0).all() and (o[0, 1, :64] == 0).all()


def test_gqa_equals_mha_with_repeated_kv():
    b, hq, hkv, t, d = 1, 6, 2, 130, 32
    q, k, v = _inputs(7, b, hq, hkv, t, d)
    nqb = 3
    idx, cnt = _random_lists(7, b, hq, nqb, nqb)
    o = oracle.sparse_attention_ref(q, k, v, idx, cnt, None)
    o_mha = oracle.sparse_attention_ref(q, k.repeat_interleave(3, 1), v.repeat_interleave(3, 1),
                                        idx, cnt, None)
    np.testing.assert_array_equal(o, o_mha)


def test_zero_query_gives_mean_of_allowed_values():
    b, hq, hkv, t, d = 1, 2, 1, 256, 8
    q, k, v = _inputs(9, b, hq, hkv, t, d, q_zero=True)
    nqb = 4
    idx, cnt = _random_lists(9, b, hq, nqb, nqb)
    o = oracle.sparse_attention_ref(q, k, v, idx, cnt, None)
    vv = v.double().numpy()
    for h in range(hq):
        for i in range(nqb):
            blocks = {int(j) for j in idx[0, h, i, : cnt[0, h, i]]}
            for r in range(64 * i, 64 * i + 64):
                keys = [c for c in range(r + 1) if c // 64 in blocks]
                np.testing.assert_allclose(o[0, h, r], vv[0, 0, keys].mean(axis=0), atol=1e-12)


def test_one_hot_limit():
    t, d = 128, 16
    q = torch.zeros(1, 1, t, d, dtype=torch.bfloat16)
    k = torch.zeros(1, 1, t, d, dtype=torch.bfloat16)
    v = torch.randn(1, 1, t, d, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    q[0, 0, 100, 0] = 64.0
    k[0, 0, 37, 0] = 64.0     # row 100 (block 1) sees key 37 (block 0) with logit 1024
    idx = np.array([[[[0, -1], [1, 0]]]], np.int32)
    cnt = np.array([[[1, 2]]], np.int32)
    o = oracle.sparse_attention_ref(q, k, v, idx, cnt, 1.0)
    np.testing.assert_allclose(o[0, 0, 100], v[0, 0, 37].double().numpy(), atol=1e-12)


def test_probability_rows_sum_to_one_and_respect_causality():
    rng = np.random.default_rng(11)
    qr = rng.standard_normal((64, 16))
    kk = rng.standard_normal((150, 16))
    rows = np.arange(64, 128)
    keys = np.arange(150)
    p = oracle.block_probs(qr, kk, rows, keys, 0.7)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-14)
    assert (p[keys[None, :] > rows[:, None]] == 0).all()


def test_list_order_does_not_matter():
    b, hq, hkv, t, d = 1, 1, 1, 320, 16
    q, k, v = _inputs(13, b, hq, hkv, t, d)
    idx = np.array([[[[0, -1, -1], [1, 0, -1], [2, 0, -1], [3, 1, 0], [4, 2, 0]]]], np.int32)
    cnt = np.array([[[1, 2, 2, 3, 3]]], np.int32)
    o1 = oracle.sparse_attention_ref(q, k, v, idx, cnt, None)
    o2 = oracle.sparse_attention_ref(q, k, v, np.sort(idx, axis=-1)[..., ::-1].copy(), cnt, None)
    np.testing.assert_array_equal(o1, o2)


# ---------------------------------------------------------------- pooled map


def _full_probs(q, k, scale):
    b, hq, t, d = q.shape
    grp = hq // k.shape[1]
    kk = k.double().repeat_interleave(grp, dim=1)
    s = scale * (q.double() @ kk.transpose(-1, -2))
    pos = torch.arange(t)
    s = s.masked_fill(pos[None, :] > pos[:, None], float("-inf"))
    return torch.softmax(s, dim=-1)


@pytest.mark.parametrize("t", [130, 256])
def test_pooled_map_equals_max_pool_of_full_probabilities(t):
    b, hq, hkv, d = 1, 4, 2, 32
    q, k, v = _inputs(21, b, hq, hkv, t, d)
    o, a = oracle.pooled_map_ref(q, k, v, None)
    p = _full_probs(q, k, 1 / math.sqrt(d))
    ref_a = F.max_pool2d(p, BLOCK, BLOCK, ceil_mode=True).numpy()
    nqb = ref_a.shape[-1]
    tri = np.tril(np.ones((nqb, nqb), bool))
    np.testing.assert_allclose(a[..., tri], ref_a[..., tri], atol=1e-14, rtol=0)
    assert (a[..., ~tri] == 0).all()
    assert (a[..., tri] > 0).all() and (a[..., tri] <= 1).all()
    assert (a[:, :, 0, 0] == 1.0).all()
    kk = k.double().repeat_interleave(2, dim=1)
    vv = v.double().repeat_interleave(2, dim=1)
    ref_o = F.scaled_dot_product_attention(q.double(), kk, vv, is_causal=True).numpy()
    np.testing.assert_allclose(o, ref_o, atol=1e-12, rtol=0)


def test_pooled_map_zero_query_closed_form():
    t, d = 320, 16
    q, k, v = _inputs(23, 1, 2, 1, t, d, q_zero=True)
    _, a = oracle.pooled_map_ref(q, k, v, None)
    for i in range(5):
        for j in range(5):
            want = 1.0 / (64 * i + 1) if j <= i else 0.0
            assert a[0, 0, i, j] == pytest.approx(want, abs=1e-15)


def test_pooled_map_bounds_every_probability_of_its_tile():
    t, d = 192, 16
    q, k, v = _inputs(25, 1, 1, 1, t, d)
    _, a = oracle.pooled_map_ref(q, k, v, 0.9)
    p = _full_probs(q, k, 0.9)[0, 0].numpy()
    for r in range(t):
        for c in range(r + 1):
            assert a[0, 0, r // 64, c // 64] >= p[r, c] * (1 - 1e-14)
