"""Pins for the AttnGate score oracle: pooling and linear against torch library
routines, RoPE against its explicit rotation and its relative-position property,
closed forms of the whole chain, causal softmax invariants and GQA."""

import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle


def _qk(seed, b, hq, hkv, t, d):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(b, hq, t, d, generator=g).to(torch.bfloat16)
    k = torch.randn(b, hkv, t, d, generator=g).to(torch.bfloat16)
    return q, k


def test_pooling_matches_torch_pooling_with_ceil_mode():
    q, k = _qk(1, 2, 3, 1, 200, 16)  # 200 = 3 full blocks + 8 tokens
    qp, kp = oracle.pool_qk(q, k)
    x = q.double().reshape(-1, 200, 16).transpose(1, 2)
    ref_q = F.avg_pool1d(x, 64, 64, ceil_mode=True).transpose(1, 2).reshape(2, 3, 4, 16)
    np.testing.assert_allclose(qp, ref_q.numpy(), rtol=0, atol=1e-14)
    y = k.double().reshape(-1, 200, 16).transpose(1, 2)
    kmax = F.max_pool1d(y, 64, 64, ceil_mode=True).transpose(1, 2).reshape(2, 1, 4, 16)
    kmin = -F.max_pool1d(-y, 64, 64, ceil_mode=True).transpose(1, 2).reshape(2, 1, 4, 16)
    np.testing.assert_array_equal(kp, np.concatenate([kmax.numpy(), kmin.numpy()], axis=-1))


def test_linear_matches_torch_linear():
    q, k = _qk(2, 1, 2, 1, 256, 8)
    rng = np.random.default_rng(3)
    wq = rng.standard_normal((2, 8, 6))
    wk = rng.standard_normal((1, 16, 6))
    qp, kp = oracle.pool_qk(q, k)
    qt, kt = oracle.gate_qk_ref(q, k, wq, wk)
    for h in range(2):
        lin = F.linear(torch.from_numpy(qp[0, h]), torch.from_numpy(wq[h]).T).numpy()
        np.testing.assert_allclose(qt[0, h], oracle.block_rope(lin), rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(qt[0, h, 0], lin[0], rtol=1e-13, atol=1e-14)  # position 0
    lin = F.linear(torch.from_numpy(kp[0, 0]), torch.from_numpy(wk[0]).T).numpy()
    np.testing.assert_allclose(kt[0, 0], oracle.block_rope(lin), rtol=1e-13, atol=1e-14)


def test_rope_explicit_rotation_norm_and_relative_positions():
    x = np.random.default_rng(4).standard_normal((3, 5, 8))
    r = oracle.block_rope(x)
    np.testing.assert_allclose(r[:, 0], x[:, 0], rtol=0, atol=0)              # position 0
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(x, axis=-1),
                               rtol=1e-14)
    # Dg = 2: one pair, frequency base^0 = 1, angle = position
    y = np.array([[[0.3, -1.2]] * 6])
    ry = oracle.block_rope(y)[0]
    for p in range(6):
        c, s = math.cos(p), math.sin(p)
        np.testing.assert_allclose(ry[p], [0.3 * c + 1.2 * s, -1.2 * c + 0.3 * s], rtol=1e-14)
    # <rope(a, i), rope(b, j)> depends on i - j only
    a = np.tile(np.random.default_rng(5).standard_normal(8), (7, 1))
    b = np.tile(np.random.default_rng(6).standard_normal(8), (7, 1))
    ra, rb = oracle.block_rope(a), oracle.block_rope(b)
    dots = ra @ rb.T
    for off in range(-6, 7):
        diag = np.diagonal(dots, off)
        np.testing.assert_allclose(diag, diag[0], rtol=1e-12, atol=1e-13)


def test_zero_query_weights_give_uniform_rows():
    q, k = _qk(7, 1, 4, 2, 300, 16)
    wq = np.zeros((4, 16, 8))
    wk = np.random.default_rng(8).standard_normal((2, 32, 8))
    s = oracle.gate_scores_ref(q, k, wq, wk)
    for i in range(5):
        np.testing.assert_allclose(s[..., i, : i + 1], 1.0 / (i + 1), rtol=1e-14)
        assert (s[..., i, i + 1:] == 0).all()


def test_constant_inputs_closed_form():
    # Every token of Q equal to u, of K equal to w: pooled Q = u, pooled K = [w | w].
    # Weights chosen so that Q~ = (a, 0) and K~ = (b, 0) (Dg = 2): with rotation angle
    # = block position, s_ij = scale * a * b * cos(i - j), then a causal softmax.
    d, t = 4, 64 * 6
    u = torch.tensor([1.0, 2.0, -1.0, 0.5]).to(torch.bfloat16)
    w = torch.tensor([0.25, -0.5, 1.0, 2.0]).to(torch.bfloat16)
    q = u.expand(1, 1, t, d).contiguous()
    k = w.expand(1, 1, t, d).contiguous()
    wq = np.zeros((1, d, 2)); wq[0, 0, 0] = 1.5                 # a = 1.5 * u[0] = 1.5
    wk = np.zeros((1, 2 * d, 2)); wk[0, 3, 0] = 1.0; wk[0, 7, 0] = 1.0  # b = w[3] + w[3] = 4
    s = oracle.gate_scores_ref(q, k, wq, wk, scale=0.7)[0, 0]
    a, bb = 1.5, 4.0
    for i in range(6):
        z = np.array([0.7 * a * bb * math.cos(i - j) for j in range(i + 1)])
        e = np.exp(z - z.max())
        np.testing.assert_allclose(s[i, : i + 1], e / e.sum(), rtol=1e-13)


def test_gqa_equals_mha_with_repeated_kv_and_weights():
    q, k = _qk(9, 2, 4, 2, 256, 8)
    rng = np.random.default_rng(10)
    wq = rng.standard_normal((4, 8, 4))
    wk = rng.standard_normal((2, 16, 4))
    s = oracle.gate_scores_ref(q, k, wq, wk)
    s_mha = oracle.gate_scores_ref(q, k.repeat_interleave(2, 1), wq, np.repeat(wk, 2, axis=0))
    np.testing.assert_allclose(s, s_mha, rtol=0, atol=0)
    np.testing.assert_allclose(s.sum(-1), 1.0, rtol=0, atol=1e-14)


def test_rope_rotate_half_pairing_dg4():
    # Dg = 4 with base 100: pairs (0, 2) at frequency 1 and (1, 3) at frequency 100^-0.5.
    x = np.array([[0.5, -1.0, 2.0, 0.25]] * 4)
    r = oracle.block_rope(x, base=100.0)
    for p in range(4):
        a0, a1 = p * 1.0, p * 0.1
        exp = [0.5 * math.cos(a0) - 2.0 * math.sin(a0),
               -1.0 * math.cos(a1) - 0.25 * math.sin(a1),
               2.0 * math.cos(a0) + 0.5 * math.sin(a0),
               0.25 * math.cos(a1) - 1.0 * math.sin(a1)]
        np.testing.assert_allclose(r[p], exp, rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------------ decode gate

def _gate_weights(seed, hq, hkv, d, dg):
    g = torch.Generator().manual_seed(seed)
    wq = torch.randn(hq, d, dg, generator=g, dtype=torch.float64) / math.sqrt(d)
    wk = torch.randn(hkv, 2 * d, dg, generator=g, dtype=torch.float64) / math.sqrt(2 * d)
    return wq.numpy(), wk.numpy()


import pytest  # noqa: E402


@pytest.mark.parametrize("block", [64, 128])
@pytest.mark.parametrize("t", [640, 700, 1])
def test_decode_gate_equals_last_prefill_row(block, t):
    """With every row of the last block equal to the new token's q, average pooling
    returns q itself, so the decode gate is the prefill gate's last row."""
    b, hq, hkv, d, dg = 2, 4, 2, 32, 16
    q_full, k_full = _qk(31 + t, b, hq, hkv, t, d)
    nb = (t + block - 1) // block
    qtok = q_full[:, :, t - 1]
    q_full[:, :, block * (nb - 1): t] = qtok[:, :, None, :]
    wq, wk = _gate_weights(32, hq, hkv, d, dg)
    tmax = t + 300  # cache slots past kv_len hold NaN: never read
    kc = torch.full((b, hkv, tmax, d), float("nan"), dtype=torch.bfloat16)
    kc[:, :, :t] = k_full
    got = oracle.decode_gate_scores_ref(qtok, kc, [t, t], wq, wk, block)
    want = oracle.gate_scores_ref(q_full, k_full, wq, wk, block=block)[:, :, nb - 1, :nb]
    np.testing.assert_allclose(got[:, :, :nb], want, rtol=0, atol=1e-12)
    assert (got[:, :, nb:] == 0).all()
    np.testing.assert_allclose(got.sum(axis=-1), 1.0, rtol=0, atol=1e-12)


def test_decode_gate_edges():
    b, hq, hkv, d, dg, tmax = 3, 2, 1, 16, 8, 500
    g = torch.Generator().manual_seed(40)
    q = torch.randn(b, hq, d, generator=g).to(torch.bfloat16)
    kc = torch.randn(b, hkv, tmax, d, generator=g).to(torch.bfloat16)
    wq, wk = _gate_weights(41, hq, hkv, d, dg)
    s = oracle.decode_gate_scores_ref(q, kc, [0, 65, 500], wq, wk, 64)
    assert s.shape == (3, 2, 8)
    assert (s[0] == 0).all()                       # an empty sequence has no blocks
    assert (s[1, :, 2:] == 0).all() and np.allclose(s[1].sum(-1), 1, atol=1e-12)
    # zero query weights: every block of the sequence gets 1 / nb
    z = oracle.decode_gate_scores_ref(q, kc, [0, 65, 500], np.zeros_like(wq), wk, 64)
    np.testing.assert_allclose(z[2], np.full((2, 8), 1 / 8), rtol=0, atol=1e-15)
    np.testing.assert_allclose(z[1, :, :2], 0.5, rtol=0, atol=1e-15)
    # the ragged last block pools only the token it has: its K~ row is that token's
    kp_last = np.concatenate([kc[1, 0, 64].double().numpy()] * 2)
    kt_last = oracle.rope_at(kp_last @ wk[0], 1)
    qt = oracle.rope_at(q[1, 0].double().numpy() @ wq[0], 1)
    kp0 = np.concatenate([kc[1, 0, :64].double().numpy().max(0),
                          kc[1, 0, :64].double().numpy().min(0)])
    kt0 = oracle.rope_at(kp0 @ wk[0], 0)
    sc = 1 / math.sqrt(dg)
    l0, l1 = sc * kt0 @ qt, sc * kt_last @ qt
    want = np.exp([l0, l1]) / np.exp([l0, l1]).sum()
    np.testing.assert_allclose(s[1, 0, :2], want, rtol=0, atol=1e-12)


def test_rope_at_is_block_rope_row():
    x = np.random.default_rng(5).standard_normal((3, 7, 12))
    full = oracle.block_rope(x)
    for i in range(7):
        np.testing.assert_allclose(oracle.rope_at(x[:, i], i), full[:, i], rtol=0, atol=1e-15)
