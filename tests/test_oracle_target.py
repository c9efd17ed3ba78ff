"""Pins for the distillation-target oracle (row normalisation + MSE): closed
forms, invariants and the chain from the pooled-map oracle on tiny inputs."""

import numpy as np
import torch

import oracle


def _random_map(seed, b, h, nqb):
    rng = np.random.default_rng(seed)
    a = rng.random((b, h, nqb, nqb)) + 1e-3
    return np.tril(a) * 0.5 + np.triu(rng.random((b, h, nqb, nqb)), 1) * 7.0  # junk above diag


def test_rows_sum_to_one_and_upper_triangle_zero():
    a = _random_map(1, 2, 3, 9)
    t, _, _ = oracle.pooled_target_ref(a)
    assert np.allclose(t.sum(axis=-1), 1.0, rtol=0, atol=1e-15)
    assert (np.triu(t, 1) == 0).all()
    causal = np.tril(np.ones((9, 9), dtype=bool))
    assert (t[..., causal] > 0).all()


def test_scale_invariance_per_row():
    # Scaling a row of the map by any positive factor leaves its target unchanged.
    a = _random_map(2, 1, 2, 7)
    f = np.random.default_rng(3).random((1, 2, 7, 1)) * 100 + 0.1
    t1, _, _ = oracle.pooled_target_ref(a)
    t2, _, _ = oracle.pooled_target_ref(a * f)
    assert np.allclose(t1, t2, rtol=1e-14, atol=0)


def test_zero_query_closed_form():
    # Q = 0: every causal probability in row block i is 1/(64 i + 1) (the oracle
    # pooled map is pinned to that separately), so the target row is uniform
    # 1/(i + 1); against a zero gate each row's SSE is (i + 1) / (i + 1)^2.
    nqb, d = 5, 64
    g = torch.Generator().manual_seed(4)
    q = torch.zeros(1, 2, 64 * nqb, d, dtype=torch.bfloat16)
    k = torch.randn(1, 1, 64 * nqb, d, generator=g).to(torch.bfloat16)
    v = torch.randn(1, 1, 64 * nqb, d, generator=g).to(torch.bfloat16)
    _, amap = oracle.pooled_map_ref(q, k, v)
    t, row_sse, loss = oracle.pooled_target_ref(amap, np.zeros_like(amap))
    for i in range(nqb):
        assert np.allclose(t[:, :, i, : i + 1], 1.0 / (i + 1), rtol=1e-13, atol=0)
        assert np.allclose(row_sse[:, :, i], 1.0 / (i + 1), rtol=1e-13, atol=0)
    n_causal = nqb * (nqb + 1) // 2
    assert abs(loss - sum(1.0 / (i + 1) for i in range(nqb)) / n_causal) < 1e-15


def test_mse_zero_against_itself_and_brute_force():
    a = _random_map(5, 2, 2, 6)
    t, _, _ = oracle.pooled_target_ref(a)
    _, row_sse, loss = oracle.pooled_target_ref(a, t)
    assert loss == 0.0 and (row_sse == 0).all()
    gate = np.random.default_rng(6).random(a.shape)
    _, row_sse, loss = oracle.pooled_target_ref(a, gate)
    # brute force over the causal entries with plain loops
    tot, cnt = 0.0, 0
    for b in range(2):
        for h in range(2):
            for i in range(6):
                s = 0.0
                for j in range(i + 1):
                    s += (gate[b, h, i, j] - t[b, h, i, j]) ** 2
                    cnt += 1
                assert abs(row_sse[b, h, i] - s) < 1e-15
                tot += s
    assert abs(loss - tot / cnt) < 1e-15


def test_gate_entries_above_diagonal_are_ignored():
    a = _random_map(7, 1, 1, 5)
    gate = np.random.default_rng(8).random(a.shape)
    _, r1, l1 = oracle.pooled_target_ref(a, gate)
    _, r2, l2 = oracle.pooled_target_ref(a, np.tril(gate) + np.triu(np.full_like(gate, 9.0), 1))
    assert (r1 == r2).all() and l1 == l2
