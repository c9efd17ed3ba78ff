"""GPU parity: the HIP library (through its C-ABI) against the fp64 CPU oracle on
the same seeded inputs.  Index lists must match bit for bit; O must be within
2e-2 max-abs and the pooled map within 1e-3 of the oracle."""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import block_sparse_attention_prefill_amd as seer
from block_sparse_attention_prefill_amd import workloads as wl

pytestmark = pytest.mark.gpu

O_TOL = 2e-2
A_TOL = 1e-3


def announce(msg):
    sys.__stderr__.write(f"\n[gpu-case] {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    seer.load()
    yield
    torch.cuda.synchronize()


def _dev(t):
    return t.to("cuda").contiguous()


def _oracle_max_k(w):
    if w.mode == wl.MODE_TOPK:
        return oracle.topk_count(w.nqb - 1, w.density, w.keep_sink)
    return w.nqb


def _gpu_mask(w, scores_cpu, max_k):
    idx, cnt = seer.seer_build_mask(_dev(scores_cpu), w.mode, w.threshold, w.density,
                                    w.keep_sink, max_k)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy()


# ------------------------------------------------------------------ masks


@pytest.mark.parametrize("wid", [1, 2, 3])
def test_mask_bitexact_full(wid):
    w = wl.WORKLOADS[wid]
    announce(f"mask full {w.name}")
    s = wl.make_scores(w)
    max_k = _oracle_max_k(w)
    assert seer.topk_budget(w.nqb, w.density, w.keep_sink) == max_k or w.mode != wl.MODE_TOPK
    gi, gc = _gpu_mask(w, s, max_k)
    ri, rc = oracle.build_mask_ref(s.numpy(), w.mode, w.threshold, w.density, w.keep_sink, max_k)
    np.testing.assert_array_equal(gc, rc)
    np.testing.assert_array_equal(gi, ri)
    if w.mode == wl.MODE_THRESHOLD:
        dens = gc.sum() / (w.hq * w.nqb * (w.nqb + 1) / 2)
        announce(f"threshold density {dens:.4f}")


def test_mask_bitexact_128k_sampled_rows():
    w = wl.C4
    announce(f"mask sampled {w.name}")
    s = wl.make_scores(w)
    max_k = _oracle_max_k(w)
    gi, gc = _gpu_mask(w, s, max_k)
    rows = wl.sample_qblocks(w)
    ref = oracle.mask_rows_ref(s.numpy(), rows, w.mode, w.threshold, w.density, w.keep_sink,
                               max_k)
    for (b, h, i), want in ref.items():
        assert gc[b, h, i] == len(want)
        assert gi[b, h, i, : len(want)].tolist() == want
        assert (gi[b, h, i, len(want):] == -1).all()
    # Every row's count is the TopK count, whatever row.
    ks = np.array([oracle.topk_count(i, w.density, w.keep_sink) for i in range(w.nqb)])
    assert (gc == ks[None, None, :]).all()
    assert gc.sum() // w.hq == 357715


def _edge_scores(seed, h, n, nkb):
    rng = np.random.default_rng(seed)
    vals = np.array([0.1, 0.2, 0.2, 0.5, -0.0, 0.0, np.nan, 0.9, -np.inf, np.inf, -3.0],
                    np.float32)
    s = rng.choice(vals, size=(1, h, n, nkb)).astype(np.float32)
    s[..., : n // 2, :] = rng.random((1, h, n // 2, nkb), dtype=np.float32)
    return torch.from_numpy(np.ascontiguousarray(s))


@pytest.mark.parametrize("mode,dens,thr,sink,max_k", [
    (wl.MODE_TOPK, 0.3, 0.0, True, None),
    (wl.MODE_TOPK, 0.05, 0.0, False, None),
    (wl.MODE_TOPK, 1.0, 0.0, True, None),
    (wl.MODE_THRESHOLD, 1.0, 0.15, True, 40),
    (wl.MODE_THRESHOLD, 1.0, 0.15, False, 3),   # capped rows
    (wl.MODE_THRESHOLD, 1.0, -1e30, True, 300),
])
def test_mask_edge_cases(mode, dens, thr, sink, max_k):
    announce(f"mask edge mode={mode} dens={dens} thr={thr} sink={sink} max_k={max_k}")
    n, nkb, h = 300, 304, 3   # row stride larger than nQB; rows span several 256-chunks
    s = _edge_scores(7, h, n, nkb)
    if max_k is None:
        max_k = oracle.topk_count(n - 1, dens, sink)
    w = wl.custom(90, 1, h, h, 64, n * 64, mode=mode, density=dens, threshold=thr,
                  keep_sink=sink)
    gi, gc = _gpu_mask(w, s, max_k)
    ri, rc = oracle.build_mask_ref(s.numpy()[..., :n], mode, thr, dens, sink, max_k)
    np.testing.assert_array_equal(gc, rc)
    np.testing.assert_array_equal(gi, ri)


@pytest.mark.parametrize("n", [3000, 4096])  # the longest rows: 64 key slots per lane
@pytest.mark.parametrize("mode,dens,thr,max_k", [(wl.MODE_TOPK, 0.05, 0.0, None),
                                                 (wl.MODE_THRESHOLD, 1.0, 0.15, 700)])
def test_mask_longest_rows_sampled(n, mode, dens, thr, max_k):
    announce(f"mask longest rows n={n} mode={mode}")
    s = _edge_scores(8 + n, 1, n, n)
    if max_k is None:
        max_k = oracle.topk_count(n - 1, dens, True)
    w = wl.custom(92, 1, 1, 1, 64, n * 64, mode=mode, density=dens, threshold=thr,
                  keep_sink=True)
    gi, gc = _gpu_mask(w, s, max_k)
    rows = [(0, 0, i) for i in sorted({0, 1, 2, 63, 64, 65, 1000, 2047, 2048, 2049, n - 2, n - 1})]
    rows += [(0, 0, int(i)) for i in np.random.default_rng(n).integers(0, n, 8)]
    ref = oracle.mask_rows_ref(s.numpy(), rows, mode, thr, dens, True, max_k)
    for (b, h, i), want in ref.items():
        assert gc[b, h, i] == len(want), (i, gc[b, h, i], len(want))
        assert gi[b, h, i, : len(want)].tolist() == want, i
        assert (gi[b, h, i, len(want):] == -1).all()
    if mode == wl.MODE_TOPK:
        ks = np.array([oracle.topk_count(i, dens, True) for i in range(n)])
        assert (gc[0, 0] == ks).all()


@pytest.mark.parametrize("case", ["c2_cut16", "c2_full", "c1_topk", "thr_sink_cut3"])
def test_build_mask_need_bitexact(case):
    """kv_need (blocks selected before the cut to max_k) and the lists, bit for bit
    against the oracle; a threshold row is cut exactly when kv_need > max_k."""
    if case.startswith("c2"):
        w = wl.C2
        max_k = 16 if case == "c2_cut16" else w.nqb
    elif case == "c1_topk":
        w = wl.C1
        max_k = _oracle_max_k(w)
    else:
        w = wl.custom(92, 2, 3, 1, 64, 64 * 37 + 5, mode=wl.MODE_THRESHOLD, threshold=0.01,
                      keep_sink=True, scores="softmax_normal")
        max_k = 3
    announce(f"mask need {case} {w.name} max_k={max_k}")
    s = wl.make_scores(w)
    idx, cnt, need = seer.seer_build_mask_need(_dev(s), w.mode, w.threshold, w.density,
                                               w.keep_sink, max_k)
    torch.cuda.synchronize()
    ri, rc, rn = oracle.build_mask_need_ref(s.numpy(), w.mode, w.threshold, w.density,
                                            w.keep_sink, max_k)
    assert np.array_equal(idx.cpu().numpy(), ri)
    assert np.array_equal(cnt.cpu().numpy(), rc)
    assert np.array_equal(need.cpu().numpy(), rn)
    cut = rn > max_k
    if case in ("c2_cut16", "thr_sink_cut3"):
        assert cut.any()
    if w.mode == wl.MODE_TOPK or case == "c2_full":
        assert not cut.any()
    # validation turns the cut rows into SEER_LIST_CAPACITY, and nothing else
    flags, rows = seer.seer_validate_lists(idx, cnt, need, row_flags=True)
    torch.cuda.synchronize()
    rf = rows.cpu().numpy()
    assert np.array_equal(rf == seer.SEER_LIST_CAPACITY, cut)
    assert np.array_equal(rf == 0, ~cut)
    f = int(flags.item())
    assert f == (seer.SEER_LIST_CAPACITY if cut.any() else 0)
    assert seer.list_flags_status(f) == (3 if cut.any() else 0)


@pytest.mark.parametrize("mode", ["sorted", "unsorted", "invalid", "dense", "repeats"])
def test_validate_lists_matches_oracle(mode):
    """Flag bits of every row, bit for bit against the oracle's list rules."""
    b, h, nqb = 2, 3, 150
    max_k = 40
    announce(f"validate lists {mode}")
    idx, cnt = _random_lists(7 * nqb + len(mode), b, h, nqb, max_k,
                             "invalid" if mode == "repeats" else mode)
    rng = np.random.default_rng(5)
    need = rng.integers(0, max_k + 3, size=(b, h, nqb)).astype(np.int32)
    if mode == "repeats":  # copy an entry over a later one in some rows (adjacent or not)
        for (bb, hh, i) in zip(*np.nonzero(cnt >= 3)):
            if rng.random() < 0.3:
                n = min(int(cnt[bb, hh, i]), max_k)
                x, y = sorted(rng.choice(n, size=2, replace=False))
                idx[bb, hh, i, y] = idx[bb, hh, i, x]
    flags, rows = seer.seer_validate_lists(_dev(torch.from_numpy(idx)),
                                           _dev(torch.from_numpy(cnt)),
                                           _dev(torch.from_numpy(need)), row_flags=True)
    torch.cuda.synchronize()
    rf, fall = oracle.validate_lists_ref(idx, cnt, need, max_k)
    assert np.array_equal(rows.cpu().numpy(), rf)
    assert int(flags.item()) == fall
    if mode == "repeats":
        assert fall & seer.SEER_LIST_REPEAT
    # without kv_need the capacity bit is never set
    flags2 = seer.seer_validate_lists(_dev(torch.from_numpy(idx)), _dev(torch.from_numpy(cnt)))
    torch.cuda.synchronize()
    assert int(flags2.item()) == fall & ~seer.SEER_LIST_CAPACITY


def test_mask_single_block():
    s = torch.full((2, 3, 1, 1), float("nan"))
    w = wl.custom(91, 2, 3, 3, 64, 64, density=0.1)
    gi, gc = _gpu_mask(w, s, 1)
    assert (gc == 1).all() and (gi == 0).all()


# ------------------------------------------------------------------ sparse prefill


def _run_sparse(q, k, v, idx, cnt, scale=None):
    o = seer.seer_sparse_prefill(_dev(q), _dev(k), _dev(v), _dev(idx), _dev(cnt), scale)
    torch.cuda.synchronize()
    return o.cpu()


def _check_blocks(o_gpu, ref, tol, label, block=64):
    worst = 0.0
    for (b, h, i), oi in ref.items():
        got = o_gpu[b, h, block * i: block * i + oi.shape[0]].double().numpy()
        err = float(np.abs(got - oi).max()) if oi.size else 0.0
        worst = max(worst, err)
        assert err <= tol, f"{label}: block {(b, h, i)} max-abs error {err}"
    announce(f"{label}: worst max-abs error {worst:.3e} over {len(ref)} blocks")
    return worst


@pytest.mark.parametrize("wid", [1, 2, 3])
def test_sparse_prefill_workloads(wid):
    w = wl.WORKLOADS[wid]
    announce(f"sparse prefill {w.name}")
    q, k, v = wl.make_qkv(w)
    s = wl.make_scores(w)
    max_k = _oracle_max_k(w)
    idx, cnt = oracle.build_mask_ref(s.numpy(), w.mode, w.threshold, w.density, w.keep_sink,
                                     max_k)
    o = _run_sparse(q, k, v, torch.from_numpy(idx), torch.from_numpy(cnt))
    assert torch.isfinite(o.float()).all()
    if wid == 1:
        blocks = [(0, h, i) for h in range(w.hq) for i in range(w.nqb)]
    else:
        blocks = wl.sample_qblocks(w, 8)
    ref = oracle.sparse_attention_blocks_ref(q, k, v, idx, cnt, None, blocks)
    _check_blocks(o, ref, O_TOL, w.name)


def _random_lists(seed, b, h, nqb, max_k, mode):
    rng = np.random.default_rng(seed)
    idx = np.full((b, h, nqb, max_k), -1, np.int32)
    cnt = np.zeros((b, h, nqb), np.int32)
    for bb in range(b):
        for hh in range(h):
            for i in range(nqb):
                hi = min(i + 1, max_k)
                if mode == "dense":  # mostly heavy rows, so that head pairs share a workgroup
                    m = int(rng.integers(max(0, (3 * hi) // 4), hi + 1))
                else:
                    m = int(rng.integers(0, hi + 1))
                sel = list(rng.choice(i + 1, size=m, replace=False)) if m else []
                if mode in ("unsorted", "dense"):
                    rng.shuffle(sel)
                else:
                    sel.sort()
                if mode == "invalid" and len(sel) < max_k:
                    sel.insert(int(rng.integers(0, len(sel) + 1)),
                               int(rng.choice([-5, i + 1, nqb + 3, 1 << 30])))
                idx[bb, hh, i, : len(sel)] = sel
                cnt[bb, hh, i] = len(sel)
                if mode == "invalid" and rng.random() < 0.2:
                    cnt[bb, hh, i] = max_k + 7   # more than max_k: read as max_k
    return idx, cnt


@pytest.mark.parametrize("b,hq,hkv,t,d,mode", [
    (1, 4, 2, 1000, 128, "sorted"),     # ragged last block, GQA 2
    (2, 6, 2, 320, 64, "unsorted"),     # batch 2, GQA 3, head dim 64
    (1, 3, 3, 200, 128, "invalid"),     # MHA, invalid entries, cnt > max_k, empty rows
    (1, 8, 1, 64, 128, "sorted"),       # a single block
    (1, 2, 1, 33, 64, "sorted"),        # shorter than one block
    (1, 8, 2, 900, 128, "dense"),       # GQA 4, heavy unsorted rows: paired and single items
    (2, 4, 1, 450, 64, "invalid"),      # GQA 4, invalid entries in paired rows
])
def test_sparse_prefill_shapes_and_lists(b, hq, hkv, t, d, mode):
    announce(f"sparse prefill custom b={b} hq={hq} hkv={hkv} t={t} d={d} lists={mode}")
    g = torch.Generator().manual_seed(t * 7 + d)
    q = torch.randn(b, hq, t, d, generator=g).to(torch.bfloat16)
    k = torch.randn(b, hkv, t, d, generator=g).to(torch.bfloat16)
    v = torch.randn(b, hkv, t, d, generator=g).to(torch.bfloat16)
    nqb = (t + 63) // 64
    max_k = nqb if mode == "dense" else max(1, min(nqb, 6))
    idx, cnt = _random_lists(t + d, b, hq, nqb, max_k, mode)
    scale = 0.2
    o = _run_sparse(q, k, v, torch.from_numpy(idx), torch.from_numpy(cnt), scale)
    ref = oracle.sparse_attention_ref(q, k, v, idx, cnt, scale)
    err = float(np.abs(o.double().numpy() - ref).max())
    announce(f"max-abs error {err:.3e}")
    assert err <= O_TOL


def _sweep_workload(seed):
    """A seeded random shape and mask rule (ragged T, GQA 1-5, D 64/128, 64- or
    128-token blocks, TopK or threshold, with or without the sink)."""
    rng = np.random.default_rng(5000 + seed)
    hkv = int(rng.integers(1, 4))
    g = int(rng.choice([1, 2, 4, 5]))
    topk = bool(rng.integers(0, 2))
    return wl.custom(
        200 + seed, int(rng.integers(1, 3)), hkv * g, hkv, int(rng.choice([64, 128])),
        int(rng.integers(1, 2600)), mode=wl.MODE_TOPK if topk else wl.MODE_THRESHOLD,
        density=float(rng.uniform(0.05, 0.6)), threshold=float(rng.uniform(0.02, 0.2)),
        keep_sink=bool(rng.integers(0, 2)),
        scores=str(rng.choice(["uniform", "local_stripe", "softmax_normal"])),
        qkv_scale=float(rng.choice([1.0, 0.25])), block=int(rng.choice([64, 128])))


@pytest.mark.parametrize("seed", range(8))
def test_mask_and_prefill_seeded_sweep(seed):
    """Seeded random shapes through the GPU mask build and the sparse pass: lists bit
    for bit against the oracle's, every query block's output against the oracle."""
    w = _sweep_workload(seed)
    announce(f"sweep {seed}: b={w.batch} hq={w.hq} hkv={w.hkv} d={w.head_dim} t={w.seq} "
             f"block={w.block} mode={w.mode} dens={w.density:.2f} thr={w.threshold:.3f} "
             f"sink={w.keep_sink} scores={w.scores}")
    q, k, v = wl.make_qkv(w)
    s = wl.make_scores(w)
    if w.mode == wl.MODE_TOPK:
        max_k = seer.topk_budget(w.nqb, w.density, w.keep_sink)
    else:
        max_k = max(2, w.nqb // 2)  # threshold rows longer than this keep their best
    idx, cnt = seer.seer_build_mask(_dev(s), w.mode, w.threshold, w.density, w.keep_sink, max_k)
    o = seer.seer_sparse_prefill_block(_dev(q), _dev(k), _dev(v), idx, cnt, w.block)
    torch.cuda.synchronize()
    o, idx, cnt = o.cpu(), idx.cpu().numpy(), cnt.cpu().numpy()
    ref_idx, ref_cnt = oracle.build_mask_ref(s.numpy(), w.mode, w.threshold, w.density,
                                             w.keep_sink, max_k)
    assert (cnt == ref_cnt).all() and (idx == ref_idx).all()
    blocks = [(b, h, i) for b in range(w.batch) for h in range(w.hq) for i in range(w.nqb)]
    ref = oracle.sparse_attention_blocks_ref(q, k, v, idx, cnt, None, blocks, w.block)
    _check_blocks(o, ref, O_TOL, f"sweep {seed}", w.block)


def test_sparse_density_one_matches_dense_causal():
    """Lists holding every causal block: the sparse kernel must reproduce dense
    causal attention (the oracle at density 1 is pinned to SDPA)."""
    announce("sparse prefill density 1")
    b, hq, hkv, t, d = 1, 4, 1, 777, 128
    g = torch.Generator().manual_seed(5)
    q = torch.randn(b, hq, t, d, generator=g).to(torch.bfloat16)
    k = torch.randn(b, hkv, t, d, generator=g).to(torch.bfloat16)
    v = torch.randn(b, hkv, t, d, generator=g).to(torch.bfloat16)
    nqb = (t + 63) // 64
    idx = np.tile(np.arange(nqb, dtype=np.int32), (b, hq, nqb, 1))
    cnt = np.tile(np.arange(1, nqb + 1, dtype=np.int32), (b, hq, 1))
    o = _run_sparse(q, k, v, torch.from_numpy(idx), torch.from_numpy(cnt))
    ref = oracle.sparse_attention_ref(q, k, v, idx, cnt, None)
    assert float(np.abs(o.double().numpy() - ref).max()) <= O_TOL


def _schedule_phases(ng, kv_bytes, active=64 * 1024 * 1024):
    """The phase count the schedule uses: doubling from 1 while a phase's K/V
    exceeds 64 MiB, each phase keeping an even share of the 8 XCDs."""
    p = 1
    if ng % 8:
        return p
    while kv_bytes / p > active and ng % (2 * p) == 0:
        gp = ng // (2 * p)
        if gp % 8 and 8 % gp:
            break
        p *= 2
    return p


@pytest.mark.parametrize("hq,hkv,t,mode,phases", [(32, 8, 4096, "sorted", 1),
                                                  (6, 2, 700, "dense", 1),
                                                  (4, 2, 900, "invalid", 1),
                                                  (3, 3, 1000, "invalid", 1),
                                                  (16, 8, 40000, "sorted", 2),
                                                  (8, 8, 140000, "invalid", 8),
                                                  # 9600 items in one group: the path that
                                                  # reads the lists again per pass
                                                  (16, 1, 38400, "invalid", 1)])
def test_sparse_schedule_work_list(hq, hkv, t, mode, phases):
    """The work list the schedule leaves in the workspace: KV group q = b * Hkv + g
    runs in phase q / GP (GP = NG / P groups per phase), and its rank-r item sits
    at position (q / GP) * GP * N + r * GP + q % GP (N = G * nQB); the group's
    column holds each of its items exactly once, longest list first, each with its
    first usable list position, that position's tile and the list length
    (bit-exact against a scan on the host)."""
    announce(f"schedule work list hq={hq} hkv={hkv} t={t} lists={mode} phases={phases}")
    b, d = 1, 64
    nqb = (t + 63) // 64
    G = hq // hkv
    max_k = nqb if mode == "dense" else max(1, min(nqb, 6))
    idx, cnt = _random_lists(hq * t, b, hq, nqb, max_k, mode)
    z = torch.zeros(b, hq, t, d, dtype=torch.bfloat16, device="cuda")
    zk = torch.zeros(b, hkv, t, d, dtype=torch.bfloat16, device="cuda")
    ws_bytes = seer.sparse_prefill_workspace_size(b, hq, hkv, t)
    ws = torch.empty(ws_bytes // 4, dtype=torch.int32, device="cuda")
    seer.seer_sparse_prefill(z, zk, zk, _dev(torch.from_numpy(idx)), _dev(torch.from_numpy(cnt)),
                             workspace=ws.view(torch.uint8))
    torch.cuda.synchronize()
    ng = b * hkv
    assert _schedule_phases(ng, 4.0 * b * hkv * t * d) == phases
    n_items = G * nqb
    gp = ng // phases
    work = ws.cpu().numpy()[: 4 * b * hq * nqb].reshape(-1, 4)
    flat_cnt = np.minimum(np.maximum(cnt.reshape(-1), 0), max_k)
    flat_idx = idx.reshape(-1, max_k)
    for grp in range(ng):
        bb, gg = divmod(grp, hkv)
        lo = (bb * hq + gg * G) * nqb
        rows = (grp // gp) * gp * n_items + np.arange(n_items) * gp + grp % gp
        col = work[rows, 0]
        assert sorted(col.tolist()) == list(range(lo, lo + n_items))
        costs = flat_cnt[col]
        assert (np.diff(costs) <= 0).all(), "items must be longest first"
        for item, pos, tile, n in work[rows]:
            i = item % nqb
            lst = flat_idx[item][: flat_cnt[item]]
            usable = [x for x, j in enumerate(lst) if 0 <= j <= i]
            assert n == flat_cnt[item]
            assert (pos, tile) == ((usable[0], lst[usable[0]]) if usable else (len(lst), -1))


@pytest.mark.parametrize("d", [128, 64])
def test_sparse_prefill_repeat_bitexact(d):
    """Repeated runs on the same inputs give bit-identical O.  A race on the
    K/V tiles in LDS can stay far inside the parity tolerance (a few outputs per
    million off by a few bf16 ulps), so it is checked for directly, at full
    workload size where many workgroups share each CU."""
    if d == 128:
        w = wl.C2
    else:
        w = wl.custom(31, 1, 16, 4, 64, 8192, mode=wl.MODE_TOPK, density=0.1, keep_sink=True,
                      scores="local_stripe")
    announce(f"sparse prefill repeat {w.name}")
    q, k, v = (_dev(t) for t in wl.make_qkv(w))
    max_k = seer.topk_budget(w.nqb, w.density, w.keep_sink) if w.mode == wl.MODE_TOPK else w.nqb
    idx, cnt = seer.seer_build_mask(_dev(wl.make_scores(w)), w.mode, w.threshold, w.density,
                                    w.keep_sink, max_k)
    first = seer.seer_sparse_prefill(q, k, v, idx, cnt).view(torch.int16).clone()
    for _ in range(3):
        again = seer.seer_sparse_prefill(q, k, v, idx, cnt).view(torch.int16)
        torch.cuda.synchronize()
        assert int((again != first).sum()) == 0


def test_pooled_map_repeat_bitexact():
    """Repeated pooled-map runs give bit-identical O and A."""
    w = wl.custom(32, 1, 32, 8, 128, 4096, kind="pooled", scores="none")
    announce(f"pooled map repeat {w.name}")
    q, k, v = (_dev(t) for t in wl.make_qkv(w))
    o0, a0 = seer.seer_pooled_attn_map(q, k, v)
    o0, a0 = o0.view(torch.int16).clone(), a0.clone()
    for _ in range(2):
        o, a = seer.seer_pooled_attn_map(q, k, v)
        torch.cuda.synchronize()
        assert int((o.view(torch.int16) != o0).sum()) == 0
        assert int((a != a0).sum()) == 0


# ------------------------------------------------------------------ 128-token blocks


def _run_sparse_block(q, k, v, idx, cnt, block, scale=None):
    o = seer.seer_sparse_prefill_block(_dev(q), _dev(k), _dev(v), _dev(idx), _dev(cnt), block,
                                       scale)
    torch.cuda.synchronize()
    return o.cpu()


@pytest.mark.parametrize("case", ["tiny", "llama8k"])
def test_sparse_prefill_block128_topk(case):
    """128-token blocks: mask built on the GPU from [B,H,T/128,T/128] scores
    (checked bit for bit against the oracle's lists), O against the oracle."""
    if case == "tiny":
        w = wl.custom(70, 1, 2, 1, 64, 512, mode=wl.MODE_TOPK, density=0.5, keep_sink=True,
                      scores="uniform", block=128)
    else:
        w = wl.custom(71, 1, 32, 8, 128, 8192, mode=wl.MODE_TOPK, density=0.1, keep_sink=True,
                      scores="local_stripe", block=128)
    announce(f"sparse prefill block 128 {w.name}")
    q, k, v = wl.make_qkv(w)
    s = wl.make_scores(w)
    max_k = seer.topk_budget(w.nqb, w.density, w.keep_sink)
    idx, cnt = seer.seer_build_mask(_dev(s), w.mode, w.threshold, w.density, w.keep_sink, max_k)
    o = seer.seer_sparse_prefill_block(_dev(q), _dev(k), _dev(v), idx, cnt, 128)
    torch.cuda.synchronize()
    o, idx, cnt = o.cpu(), idx.cpu().numpy(), cnt.cpu().numpy()
    ref_idx, ref_cnt = oracle.build_mask_ref(s.numpy(), w.mode, w.threshold, w.density,
                                             w.keep_sink, max_k)
    assert (idx == ref_idx).all() and (cnt == ref_cnt).all()
    if case == "tiny":
        blocks = [(0, h, i) for h in range(w.hq) for i in range(w.nqb)]
    else:
        blocks = wl.sample_qblocks(w, 4)
    ref = oracle.sparse_attention_blocks_ref(q, k, v, idx, cnt, None, blocks, 128)
    _check_blocks(o, ref, O_TOL, w.name, 128)


@pytest.mark.parametrize("b,hq,hkv,t,d,mode", [
    (1, 4, 2, 1000, 128, "unsorted"),   # ragged: the last 128-block holds one short tile
    (2, 6, 3, 700, 64, "invalid"),      # invalid entries, cnt > max_k, empty rows
    (1, 2, 1, 100, 128, "sorted"),      # one 128-block, two tiles
    (1, 4, 1, 777, 64, "dense"),        # heavy rows
])
def test_sparse_prefill_block128_lists(b, hq, hkv, t, d, mode):
    announce(f"sparse prefill block 128 custom b={b} hq={hq} hkv={hkv} t={t} d={d} lists={mode}")
    g = torch.Generator().manual_seed(t * 11 + d)
    q = torch.randn(b, hq, t, d, generator=g).to(torch.bfloat16)
    k = torch.randn(b, hkv, t, d, generator=g).to(torch.bfloat16)
    v = torch.randn(b, hkv, t, d, generator=g).to(torch.bfloat16)
    nb = (t + 127) // 128
    max_k = nb if mode == "dense" else max(1, min(nb, 4))
    idx, cnt = _random_lists(t + 3 * d, b, hq, nb, max_k, mode)
    o = _run_sparse_block(q, k, v, torch.from_numpy(idx), torch.from_numpy(cnt), 128, 0.2)
    ref = oracle.sparse_attention_ref(q, k, v, idx, cnt, 0.2, 128)
    err = float(np.abs(o.double().numpy() - ref).max())
    announce(f"max-abs error {err:.3e}")
    assert err <= O_TOL


def test_sparse_prefill_block128_density_one_and_repeat():
    """Every causal 128-block listed: dense causal attention (the oracle at
    density 1 is pinned to SDPA); repeated runs are bit-identical."""
    b, hq, hkv, t, d = 1, 4, 2, 1100, 128
    g = torch.Generator().manual_seed(9)
    q = torch.randn(b, hq, t, d, generator=g).to(torch.bfloat16)
    k = torch.randn(b, hkv, t, d, generator=g).to(torch.bfloat16)
    v = torch.randn(b, hkv, t, d, generator=g).to(torch.bfloat16)
    nb = (t + 127) // 128
    idx = np.tile(np.arange(nb, dtype=np.int32), (b, hq, nb, 1))
    cnt = np.tile(np.arange(1, nb + 1, dtype=np.int32), (b, hq, 1))
    o = _run_sparse_block(q, k, v, torch.from_numpy(idx), torch.from_numpy(cnt), 128)
    ref = oracle.sparse_attention_ref(q, k, v, idx, cnt, None, 128)
    assert float(np.abs(o.double().numpy() - ref).max()) <= O_TOL
    o2 = _run_sparse_block(q, k, v, torch.from_numpy(idx), torch.from_numpy(cnt), 128)
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))


# ------------------------------------------------------------------ pooled map


def _run_pooled(q, k, v, scale=None):
    o, a = seer.seer_pooled_attn_map(_dev(q), _dev(k), _dev(v), scale)
    torch.cuda.synchronize()
    return o.cpu(), a.cpu()


def test_pooled_map_tiny_full():
    w = wl.C1
    announce(f"pooled map {w.name}")
    q, k, v = wl.make_qkv(w)
    o, a = _run_pooled(q, k, v)
    ro, ra = oracle.pooled_map_ref(q, k, v, None)
    assert float(np.abs(o.double().numpy() - ro).max()) <= O_TOL
    assert float(np.abs(a.double().numpy() - ra).max()) <= A_TOL
    assert (a.numpy()[:, :, 0, 0] > 1 - A_TOL).all()


@pytest.mark.parametrize("b,hq,hkv,t,d", [
    (1, 4, 2, 1000, 128),
    (2, 3, 1, 130, 64),
    (1, 2, 2, 64, 128),
])
def test_pooled_map_shapes(b, hq, hkv, t, d):
    announce(f"pooled map custom b={b} hq={hq} hkv={hkv} t={t} d={d}")
    g = torch.Generator().manual_seed(t + d)
    q = (2.0 * torch.randn(b, hq, t, d, generator=g)).to(torch.bfloat16)
    k = torch.randn(b, hkv, t, d, generator=g).to(torch.bfloat16)
    v = torch.randn(b, hkv, t, d, generator=g).to(torch.bfloat16)
    o, a = _run_pooled(q, k, v, 0.15)
    ro, ra = oracle.pooled_map_ref(q, k, v, 0.15)
    eo = float(np.abs(o.double().numpy() - ro).max())
    ea = float(np.abs(a.double().numpy() - ra).max())
    announce(f"O err {eo:.3e}  A err {ea:.3e}")
    assert eo <= O_TOL and ea <= A_TOL


def test_pooled_map_zero_query_closed_form():
    announce("pooled map zero query")
    t, d = 512, 128
    q = torch.zeros(1, 2, t, d, dtype=torch.bfloat16)
    g = torch.Generator().manual_seed(3)
    k = torch.randn(1, 1, t, d, generator=g).to(torch.bfloat16)
    v = torch.randn(1, 1, t, d, generator=g).to(torch.bfloat16)
    _, a = _run_pooled(q, k, v)
    n = t // 64
    want = np.array([[1.0 / (64 * i + 1) if j <= i else 0.0 for j in range(n)] for i in range(n)])
    assert np.abs(a.numpy()[0] - want[None]).max() <= 1e-5


def test_pooled_map_qwen_32k_sampled():
    w = wl.C5
    announce(f"pooled map {w.name}")
    q, k, v = wl.make_qkv(w)
    o, a = _run_pooled(q, k, v)
    blocks = wl.sample_qblocks(w)
    ref = oracle.pooled_map_blocks_ref(q, k, v, None, blocks)
    worst_o = worst_a = 0.0
    an = a.numpy()
    for (b, h, i), (oi, ai) in ref.items():
        got = o[b, h, 64 * i: 64 * i + oi.shape[0]].double().numpy()
        worst_o = max(worst_o, float(np.abs(got - oi).max()))
        worst_a = max(worst_a, float(np.abs(an[b, h, i] - ai).max()))
    announce(f"{w.name}: O err {worst_o:.3e}  A err {worst_a:.3e}")
    assert worst_o <= O_TOL and worst_a <= A_TOL
    # Properties that hold for every row, sampled or not.
    tri = np.tril(np.ones((w.nqb, w.nqb), bool))
    assert (an[..., tri] > 0).all() and (an[..., tri] <= 1 + 1e-6).all()
    assert (an[..., ~tri] == 0).all()
    assert np.abs(an[:, :, 0, 0] - 1).max() <= 1e-6


# ------------------------------------------------------------------ distillation target

T_TOL = 1e-5      # target: fp32 row sums of <= 4096 terms in [0, 1], relative error << 1e-5
SSE_RTOL = 1e-4   # per-row squared error (fp32 sums of <= 4096 terms)
LOSS_RTOL = 1e-5  # loss: fp64 sum of the row errors


# nQB 8 .. 512: rows held in registers (2 chunks per lane); 1000, 2000: 4 and 8
# chunks per lane; 2052: the re-reading 16-byte form; 13: the 4-byte form.
@pytest.mark.parametrize("b,h,nqb", [(1, 2, 8), (2, 3, 13), (1, 40, 512), (1, 1, 1000),
                                     (1, 1, 2000), (1, 1, 2052)])
def test_pooled_target_random_maps(b, h, nqb):
    announce(f"pooled target b={b} h={h} nqb={nqb}")
    w = wl.custom(40 + nqb, b, h, 1, 64, 64 * nqb, scores="softmax_normal")
    amap = wl.make_block_map(w)
    gate = wl.make_scores(w)
    t, r, l = seer.seer_pooled_target_mse(_dev(amap), _dev(gate))
    torch.cuda.synchronize()
    rt, rr, rl = oracle.pooled_target_ref(amap.numpy(), gate.numpy())
    assert float(np.abs(t.cpu().double().numpy() - rt).max()) <= T_TOL
    assert np.allclose(r.cpu().double().numpy(), rr, rtol=SSE_RTOL, atol=1e-12)
    assert abs(float(l.cpu()) - rl) <= LOSS_RTOL * rl


@pytest.mark.parametrize("nqb", [37, 40])  # 4-byte and 16-byte row forms
def test_pooled_target_in_place_and_without_gate(nqb):
    w = wl.custom(60, 1, 4, 1, 64, 64 * nqb, scores="softmax_normal")
    amap = wl.make_block_map(w)
    rt, _, _ = oracle.pooled_target_ref(amap.numpy())
    a = _dev(amap)
    t, r, l = seer.seer_pooled_target_mse(a, None, target=a)
    torch.cuda.synchronize()
    assert r is None and l is None and t.data_ptr() == a.data_ptr()
    assert float(np.abs(a.cpu().double().numpy() - rt).max()) <= T_TOL


def test_pooled_target_unaligned_buffers():
    """nQB % 4 == 0 but buffers only 4-byte aligned: the 4-byte row form runs."""
    w = wl.custom(63, 1, 3, 1, 64, 64 * 24, scores="softmax_normal")
    amap, gate = wl.make_block_map(w), wl.make_scores(w)
    n = amap.numel()
    ab = torch.zeros(n + 1, dtype=torch.float32, device="cuda")
    gb = torch.zeros(n + 1, dtype=torch.float32, device="cuda")
    tb = torch.zeros(n + 1, dtype=torch.float32, device="cuda")
    a, g, t = (x[1:].view(amap.shape) for x in (ab, gb, tb))
    a.copy_(amap.cuda())
    g.copy_(gate.cuda())
    t_out, r, l = seer.seer_pooled_target_mse(a, g, target=t)
    torch.cuda.synchronize()
    rt, rr, rl = oracle.pooled_target_ref(amap.numpy(), gate.numpy())
    assert t_out.data_ptr() == t.data_ptr()
    assert float(np.abs(t.cpu().double().numpy() - rt).max()) <= T_TOL
    assert np.allclose(r.cpu().double().numpy(), rr, rtol=SSE_RTOL, atol=1e-12)
    assert abs(float(l.cpu()) - rl) <= LOSS_RTOL * rl
    assert float(tb[0]) == 0.0  # nothing written before the view


def test_pooled_target_chain_from_pooled_map():
    """GPU pooled map -> GPU target, against the oracle map -> oracle target."""
    w = wl.C1
    q, k, v = wl.make_qkv(w)
    _, amap = seer.seer_pooled_attn_map(_dev(q), _dev(k), _dev(v))
    gate = _dev(wl.make_scores(wl.custom(61, 1, w.hq, 1, 64, w.seq, scores="softmax_normal")))
    t, r, l = seer.seer_pooled_target_mse(amap, gate)
    torch.cuda.synchronize()
    _, ref_map = oracle.pooled_map_ref(q, k, v)
    rt, rr, rl = oracle.pooled_target_ref(ref_map, gate.cpu().numpy())
    # the map is within A_TOL of the oracle's; row normalisation can at most
    # double a relative error, and rows sum to 1, so 2 * A_TOL bounds the target
    assert float(np.abs(t.cpu().double().numpy() - rt).max()) <= 2 * A_TOL
    assert abs(float(l.cpu()) - rl) <= 4 * A_TOL


def test_pooled_target_repeat_bitexact():
    w = wl.custom(62, 1, 8, 1, 64, 64 * 300, scores="softmax_normal")
    amap, gate = _dev(wl.make_block_map(w)), _dev(wl.make_scores(w))
    t0, r0, l0 = (x.clone() for x in seer.seer_pooled_target_mse(amap, gate))
    for _ in range(2):
        t, r, l = seer.seer_pooled_target_mse(amap, gate)
        torch.cuda.synchronize()
        assert torch.equal(t, t0) and torch.equal(r, r0) and torch.equal(l, l0)


# ------------------------------------------------------------------ AttnGate scores

G_TOL = 1e-5  # scores in [0, 1]: fp32 pooling, projection and logits vs the fp64 oracle


def _gate_case(case):
    if case == "tiny":
        return wl.custom(80, 1, 2, 1, 64, 512), 32
    if case == "ragged":
        return wl.custom(81, 2, 4, 2, 128, 1000), 64
    if case == "d64":
        return wl.custom(82, 1, 6, 3, 64, 2000), 128
    if case == "far128k":  # block positions up to 2047: RoPE angles of ~2000 rad
        return wl.custom(86, 1, 2, 1, 64, 131072), 64
    if case == "rows4096":  # 4096 query blocks: rows longer than one workgroup's LDS holds
        return wl.custom(87, 1, 1, 1, 64, 262144), 32
    return wl.custom(83, 1, 32, 8, 128, 8192, qkv_scale=1.0 / math.sqrt(128.0)), 128


@pytest.mark.parametrize("case", ["tiny", "ragged", "d64", "far128k", "rows4096", "llama8k"])
def test_attn_gate_scores(case):
    w, dg = _gate_case(case)
    announce(f"attn gate scores {w.name} dg={dg}")
    q, k, _ = wl.make_qkv(w)
    wq, wk = wl.make_gate_weights(w, dg)
    s = seer.seer_attn_gate_scores(_dev(q), _dev(k), _dev(wq), _dev(wk))
    torch.cuda.synchronize()
    ref = oracle.gate_scores_ref(q, k, wq.numpy(), wk.numpy())
    err = float(np.abs(s.cpu().double().numpy() - ref).max())
    announce(f"max-abs error {err:.3e}")
    assert err <= G_TOL


def test_attn_gate_to_topk_lists():
    """Gate scores -> TopK on the GPU, against the oracle's scores -> TopK.  Lists
    must be equal wherever the oracle's selection boundary is wider than the score
    tolerance; elsewhere the GPU list must be a valid TopK within that tolerance."""
    # N(0, 1) inputs and gain-2 weights give peaked rows (about 3 % of them have
    # a selection boundary inside the score tolerance)
    w, dg = wl.custom(84, 1, 32, 8, 128, 8192), 128
    q, k, _ = wl.make_qkv(w)
    wq, wk = wl.make_gate_weights(w, dg, gain=2.0)
    density = 0.2
    max_k = seer.topk_budget(w.nqb, density, True)
    s = seer.seer_attn_gate_scores(_dev(q), _dev(k), _dev(wq), _dev(wk))
    idx, cnt = seer.seer_build_mask(s, wl.MODE_TOPK, 0.0, density, True, max_k)
    torch.cuda.synchronize()
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    ref = oracle.gate_scores_ref(q, k, wq.numpy(), wk.numpy())
    ridx, rcnt = oracle.build_mask_ref(ref.astype(np.float32), wl.MODE_TOPK, 0.0, density, True,
                                       max_k)
    assert (cnt == rcnt).all()
    exact = ambiguous = 0
    for b in range(w.batch):
        for h in range(w.hq):
            for i in range(w.nqb):
                got = idx[b, h, i, : cnt[b, h, i]].tolist()
                want = ridx[b, h, i, : rcnt[b, h, i]].tolist()
                forced = set(oracle.forced_blocks(i, True))
                others = sorted((j for j in range(i + 1) if j not in forced),
                                key=lambda j: (-ref[b, h, i, j], j))
                kk = len(want) - len(forced & set(want))
                if kk == 0 or kk == len(others):
                    assert got == want
                    exact += 1
                    continue
                gap = ref[b, h, i, others[kk - 1]] - ref[b, h, i, others[kk]]
                if gap > 2 * G_TOL:
                    assert got == want, (b, h, i)
                    exact += 1
                else:
                    ambiguous += 1
                    bound = ref[b, h, i, others[kk - 1]]
                    chosen = set(got) - forced
                    assert len(chosen) == kk and forced <= set(got)
                    assert all(ref[b, h, i, j] >= bound - 2 * G_TOL for j in chosen)
                    assert all(ref[b, h, i, j] <= bound + 2 * G_TOL
                               for j in others if j not in chosen)
    announce(f"gate -> TopK: {exact} rows exact, {ambiguous} rows within tolerance")
    assert exact > 0.9 * (exact + ambiguous)


@pytest.mark.parametrize("case", ["tiny", "ragged", "d64", "far128k", "rows4096", "llama8k"])
@pytest.mark.parametrize("mode", [wl.MODE_TOPK, wl.MODE_THRESHOLD])
def test_attn_gate_mask_equals_scores_then_mask(case, mode):
    """The fused call returns, bit for bit, the scores of seer_attn_gate_scores and
    the lists seer_build_mask makes from them, with and without a scores buffer, and
    with the logits produced in passes over tile rows."""
    w, dg = _gate_case(case)
    announce(f"attn gate mask {w.name} dg={dg} mode={mode}")
    q, k, _ = (_dev(t) for t in wl.make_qkv(w))
    wq, wk = (_dev(t) for t in wl.make_gate_weights(w, dg, gain=2.0))
    density, thr = 0.2, 0.02
    max_k = seer.topk_budget(w.nqb, density, True) if mode == wl.MODE_TOPK else w.nqb // 2 + 2
    s = seer.seer_attn_gate_scores(q, k, wq, wk)
    ri, rc = seer.seer_build_mask(s, mode, thr, density, True, max_k)
    gi, gc, gs = seer.seer_attn_gate_mask(q, k, wq, wk, mode, thr, density, True, max_k,
                                          return_scores=True)
    ni, nc, ns = seer.seer_attn_gate_mask(q, k, wq, wk, mode, thr, density, True, max_k)
    torch.cuda.synchronize()
    assert ns is None
    assert torch.equal(gs, s)
    assert torch.equal(gc, rc) and torch.equal(gi, ri)
    assert torch.equal(nc, rc) and torch.equal(ni, ri)
    # The logits in passes of 1 and 3 tile rows (64 query blocks each) from a
    # workspace sized for that: the same lists.
    for pt in (1, 3):
        pi, pc, _ = seer.seer_attn_gate_mask(q, k, wq, wk, mode, thr, density, True, max_k,
                                             pass_tiles=pt)
        torch.cuda.synchronize()
        assert torch.equal(pc, rc) and torch.equal(pi, ri), pt
    if mode == wl.MODE_THRESHOLD:
        announce(f"threshold lists: mean length {float(rc.float().mean()):.2f}, "
                 f"rows at max_k {int((rc == max_k).sum())}")


def test_attn_gate_repeat_bitexact():
    w, dg = _gate_case("ragged")
    q, k, _ = (_dev(t) for t in wl.make_qkv(w))
    wq, wk = (_dev(t) for t in wl.make_gate_weights(w, dg))
    s0 = seer.seer_attn_gate_scores(q, k, wq, wk).clone()
    for _ in range(2):
        s = seer.seer_attn_gate_scores(q, k, wq, wk)
        torch.cuda.synchronize()
        assert torch.equal(s, s0)



# ------------------------------------------------------------------ decode


def _decode_case(wid, batch, hq, hkv, tmax, d, kv_lens, block=64, list_heads="q",
                 budget_tokens=4096, keep_sink=True):
    return wl.DecodeWorkload(wid, f"decode{wid}", batch, hq, hkv, d, tmax, tuple(kv_lens),
                             block=block, budget_tokens=budget_tokens, list_heads=list_heads,
                             keep_sink=keep_sink)


def _decode_mask_scores(seed, dw, ties_nan=False):
    s = wl.make_decode_scores(dw)
    if ties_nan:
        rng = np.random.default_rng(seed)
        vals = np.array([0.1, 0.2, 0.2, 0.5, -0.0, 0.0, np.nan, 0.9], np.float32)
        s = torch.from_numpy(rng.choice(vals, size=tuple(s.shape)).astype(np.float32))
    return s


@pytest.mark.parametrize("block", [64, 128])
@pytest.mark.parametrize("mode,thr,kb,sink", [
    (wl.MODE_TOPK, 0.0, 3, True), (wl.MODE_TOPK, 0.0, 1, False), (wl.MODE_TOPK, 0.0, 64, True),
    (wl.MODE_THRESHOLD, 2.0, 0, True), (wl.MODE_THRESHOLD, 0.15, 0, False)])
@pytest.mark.parametrize("ties_nan", [False, True])
def test_decode_mask_bitexact(block, mode, thr, kb, sink, ties_nan):
    dw = _decode_case(70, 5, 4, 2, 2000, 64, (2000, 1, 0, 777, 129), block=block, keep_sink=sink)
    announce(f"decode mask block {block} mode {mode} thr {thr} kb {kb} sink {sink} "
             f"ties {ties_nan}")
    s = _decode_mask_scores(71, dw, ties_nan)
    nkb = s.shape[-1]
    max_k = nkb if mode == wl.MODE_THRESHOLD else max(2, min(nkb, kb))
    if mode == wl.MODE_THRESHOLD and thr == 2.0:
        max_k = 6  # lists longer than max_k keep the best-ranked passing blocks
    kv_len = torch.tensor(dw.kv_lens, dtype=torch.int32)
    gi, gc = seer.seer_build_mask_decode(_dev(s), _dev(kv_len), block, mode, thr, max(kb, 1),
                                         sink, max_k)
    torch.cuda.synchronize()
    ri, rc = oracle.build_mask_decode_ref(s.numpy(), dw.kv_lens, block, mode, thr, max(kb, 1),
                                          sink, max_k)
    np.testing.assert_array_equal(gc.cpu().numpy(), rc)
    np.testing.assert_array_equal(gi.cpu().numpy(), ri)


@pytest.mark.parametrize("mode,thr,kb", [(wl.MODE_TOPK, 0.0, 64), (wl.MODE_THRESHOLD, 2.0, 0)])
def test_decode_mask_longest_rows(mode, thr, kb):
    """nKB = 4096 (the limit): rows of 64 key slots per lane, full and ragged sequences."""
    dw = _decode_case(72, 3, 2, 1, 4096 * 64, 64, (4096 * 64, 100001, 64 * 4095 + 1))
    announce(f"decode mask longest rows mode {mode}")
    s = _decode_mask_scores(73, dw)
    assert s.shape[-1] == 4096
    max_k = 4096 if mode == wl.MODE_THRESHOLD else kb
    kv_len = torch.tensor(dw.kv_lens, dtype=torch.int32)
    gi, gc = seer.seer_build_mask_decode(_dev(s), _dev(kv_len), 64, mode, thr, max(kb, 1), True,
                                         max_k)
    torch.cuda.synchronize()
    ri, rc = oracle.build_mask_decode_ref(s.numpy(), dw.kv_lens, 64, mode, thr, max(kb, 1),
                                          True, max_k)
    np.testing.assert_array_equal(gc.cpu().numpy(), rc)
    np.testing.assert_array_equal(gi.cpu().numpy(), ri)


DEC_GATE_CASES = {
    # b, hq, hkv, d, tmax, kv_lens, block, dg
    "ragged_d64_b64": (3, 4, 2, 64, 700, (700, 1, 0), 64, 32),
    "gqa4_d128_b128": (2, 8, 2, 128, 1000, (1000, 450), 128, 64),
    "llama_40k": (2, 32, 8, 128, 40960, (40960, 12345), 64, 128),
    "rows_1500_d64_dg32": (2, 4, 1, 64, 96000, (96000, 50001), 64, 32),  # 32 key slots per lane
    "rows_3125_gqa4": (1, 8, 2, 128, 200000, (199999,), 64, 64),  # 64 key slots per lane
}


def _dec_gate_inputs(case):
    b, hq, hkv, d, tmax, lens, block, dg = DEC_GATE_CASES[case]
    g = torch.Generator().manual_seed(90 + tmax)
    q = torch.randn(b, hq, d, generator=g).to(torch.bfloat16)
    kc = torch.randn(b, hkv, tmax, d, generator=g).to(torch.bfloat16)
    w = wl.custom(95, b, hq, hkv, d, 64)
    wq, wk = wl.make_gate_weights(w, dg, gain=2.0)
    return q, kc, wq, wk, lens, block, tmax


@pytest.mark.parametrize("case", sorted(DEC_GATE_CASES))
def test_attn_gate_decode_scores(case):
    q, kc, wq, wk, lens, block, tmax = _dec_gate_inputs(case)
    announce(f"decode gate {case}")
    for bb, n in enumerate(lens):  # cache slots past each sequence: never read
        kc[bb, :, n:] = float("nan")
    kl = _dev(torch.tensor(lens, dtype=torch.int32))
    kg = seer.seer_attn_gate_decode_keys(_dev(kc), kl, _dev(wk), block)
    s = seer.seer_attn_gate_decode_scores(_dev(q), kg, kl, _dev(wq), tmax, block)
    torch.cuda.synchronize()
    ref = oracle.decode_gate_scores_ref(q, kc, lens, wq.numpy(), wk.numpy(), block)
    got = s.cpu().double().numpy()
    err = float(np.abs(got - ref).max())
    announce(f"max-abs error {err:.3e}")
    assert err <= G_TOL
    for bb, n in enumerate(lens):
        assert (got[bb, :, (n + block - 1) // block:] == 0).all()
    kg2 = seer.seer_attn_gate_decode_keys(_dev(kc), kl, _dev(wk), block)
    s2 = seer.seer_attn_gate_decode_scores(_dev(q), kg2, kl, _dev(wq), tmax, block)
    torch.cuda.synchronize()
    assert torch.equal(s, s2)


@pytest.mark.parametrize("case", ["ragged_d64_b64", "gqa4_d128_b128"])
def test_attn_gate_decode_last_block_updates(case):
    """Keys built once, then refreshed for the last block only as tokens are appended
    (across block boundaries): scores stay within tolerance of the oracle's."""
    q, kc, wq, wk, lens, block, tmax = _dec_gate_inputs(case)
    lens = [max(1, n - 70) for n in lens]
    kcd, wqd, wkd, qd = _dev(kc), _dev(wq), _dev(wk), _dev(q)
    kg = seer.seer_attn_gate_decode_keys(kcd, _dev(torch.tensor(lens, dtype=torch.int32)), wkd,
                                         block)
    worst = 0.0
    for step in range(70):
        lens = [min(n + 1, tmax) for n in lens]
        kl = _dev(torch.tensor(lens, dtype=torch.int32))
        seer.seer_attn_gate_decode_keys(kcd, kl, wkd, block, last_block_only=True, k_gate=kg)
        if step % 7 == 6:
            s = seer.seer_attn_gate_decode_scores(qd, kg, kl, wqd, tmax, block)
            torch.cuda.synchronize()
            ref = oracle.decode_gate_scores_ref(q, kc, lens, wq.numpy(), wk.numpy(), block)
            worst = max(worst, float(np.abs(s.cpu().double().numpy() - ref).max()))
    announce(f"incremental keys: worst max-abs error {worst:.3e}")
    assert worst <= G_TOL


def test_attn_gate_decode_matches_prefill_gate_last_row():
    """GPU decode gate against the GPU prefill gate when every row of the last block is
    the token's q (mean pooling then returns q): equal within the score tolerance."""
    b, hq, hkv, d, t, dg = 1, 8, 2, 128, 1000, 64
    g = torch.Generator().manual_seed(97)
    qf = torch.randn(b, hq, t, d, generator=g).to(torch.bfloat16)
    kf = torch.randn(b, hkv, t, d, generator=g).to(torch.bfloat16)
    nb = (t + 63) // 64
    qtok = qf[:, :, t - 1].clone()
    qf[:, :, 64 * (nb - 1):] = qtok[:, :, None, :]
    w = wl.custom(96, b, hq, hkv, d, t)
    wq, wk = (_dev(x) for x in wl.make_gate_weights(w, dg))
    pre = seer.seer_attn_gate_scores(_dev(qf), _dev(kf), wq, wk)
    kl = _dev(torch.tensor([t], dtype=torch.int32))
    kg = seer.seer_attn_gate_decode_keys(_dev(kf), kl, wk)
    dec = seer.seer_attn_gate_decode_scores(_dev(qtok), kg, kl, wq, t)
    torch.cuda.synchronize()
    err = float((pre[:, :, nb - 1, :].double() - dec.double()).abs().max())
    announce(f"decode vs prefill gate last row: {err:.3e}")
    assert err <= 2 * G_TOL


@pytest.mark.parametrize("case", sorted(DEC_GATE_CASES))
def test_attn_gate_decode_mask_equals_scores_then_mask(case):
    """One-pass decode gate lists equal seer_build_mask_decode on the scores call's
    rows, bit for bit (TopK and threshold, with and without the sink, a short max_k),
    and the optional score output equals the scores call's."""
    q, kc, wq, wk, lens, block, tmax = _dec_gate_inputs(case)
    announce(f"decode gate mask {case}")
    kl = _dev(torch.tensor(lens, dtype=torch.int32))
    qd, wqd = _dev(q), _dev(wq)
    kg = seer.seer_attn_gate_decode_keys(_dev(kc), kl, _dev(wk), block)
    ref_s = seer.seer_attn_gate_decode_scores(qd, kg, kl, wqd, tmax, block)
    nkb = (tmax + block - 1) // block
    rules = [(seer.SEER_MASK_TOPK, 0.0, 4, True, 8), (seer.SEER_MASK_TOPK, 0.0, 64, False, 64),
             (seer.SEER_MASK_THRESHOLD, 1.0 / nkb, 1, True, nkb),
             (seer.SEER_MASK_THRESHOLD, 1.0 / nkb, 1, False, 5)]
    for mode, tau, kb, sink, max_k in rules:
        max_k = min(max_k, nkb) if mode == seer.SEER_MASK_TOPK else max_k
        ri, rc = seer.seer_build_mask_decode(ref_s, kl, block, mode, tau, kb, sink, max_k)
        fi = torch.full_like(ri, -7)
        fc = torch.full_like(rc, -7)
        fi, fc, fs = seer.seer_attn_gate_decode_mask(qd, kg, kl, wqd, tmax, mode, tau, kb, sink,
                                                     max_k, block, return_scores=True,
                                                     kv_idx=fi, kv_cnt=fc)
        ni, nc, none = seer.seer_attn_gate_decode_mask(qd, kg, kl, wqd, tmax, mode, tau, kb,
                                                       sink, max_k, block)
        torch.cuda.synchronize()
        assert none is None
        assert torch.equal(fs, ref_s)
        assert torch.equal(fi, ri) and torch.equal(fc, rc), (mode, sink, max_k)
        assert torch.equal(ni, ri) and torch.equal(nc, rc)
        assert int(rc.min()) >= 0 and int(rc.max()) <= max_k


def _decode_lists(seed, dw, max_k, dense=False):
    """Random valid block sets per list head (any order), some with entries past
    the sequence that must be skipped; dense=True lists every block."""
    rng = np.random.default_rng(seed)
    lh = dw.lh
    idx = np.full((dw.batch, lh, max_k), -1, np.int32)
    cnt = np.zeros((dw.batch, lh), np.int32)
    for b, n in enumerate(dw.kv_lens):
        nb = (n + dw.block - 1) // dw.block
        for h in range(lh):
            if dense:
                sel = list(range(min(nb, max_k)))
            else:
                m = int(rng.integers(0, min(nb, max_k - 1) + 1)) if nb else 0
                sel = [int(x) for x in rng.choice(nb, size=m, replace=False)] if m else []
                if len(sel) < max_k and rng.random() < 0.3:
                    sel.append(nb + int(rng.integers(0, 4)))
            rng.shuffle(sel)
            idx[b, h, : len(sel)] = sel
            cnt[b, h] = len(sel)
    return idx, cnt


def _run_decode(dw, q, k, v, kv_len, idx, cnt, scale=None):
    o = seer.seer_sparse_decode(_dev(q), _dev(k), _dev(v), _dev(kv_len), _dev(torch.from_numpy(idx)),
                                _dev(torch.from_numpy(cnt)), dw.block, scale)
    torch.cuda.synchronize()
    return o


DECODE_CASES = {
    "gqa2_d128_b64_perhead": dict(batch=4, hq=4, hkv=2, tmax=700, d=128,
                                  kv_lens=(700, 1, 333, 0), block=64, list_heads="q", max_k=8),
    "gqa8_d64_b128_perhead": dict(batch=2, hq=8, hkv=1, tmax=1000, d=64, kv_lens=(1000, 450),
                                  block=128, list_heads="q", max_k=5),
    "gqa5_d128_b64_shared": dict(batch=2, hq=5, hkv=1, tmax=333, d=128, kv_lens=(333, 64),
                                 block=64, list_heads="kv", max_k=4),
    "mha_d64_b64": dict(batch=2, hq=2, hkv=2, tmax=257, d=64, kv_lens=(257, 200), block=64,
                        list_heads="q", max_k=5),
    "qwen_gqa5_d128_b128_perhead": dict(batch=1, hq=40, hkv=8, tmax=4096, d=128,
                                        kv_lens=(4001,), block=128, list_heads="q", max_k=12),
    "gqa4_d128_b64_dense_long": dict(batch=2, hq=8, hkv=2, tmax=5000, d=128,
                                     kv_lens=(5000, 3001), block=64, list_heads="q", max_k=79,
                                     dense=True),
}


@pytest.mark.parametrize("case", sorted(DECODE_CASES))
def test_sparse_decode_parity(case):
    c = dict(DECODE_CASES[case])
    max_k, dense = c.pop("max_k"), c.pop("dense", False)
    dw = _decode_case(80 + sorted(DECODE_CASES).index(case), **c)
    announce(f"decode {case}")
    q, k, v, kv_len = wl.make_decode_inputs(dw, tail_nan=True)
    idx, cnt = _decode_lists(dw.wid, dw, max_k, dense)
    scale = 1.0 / math.sqrt(dw.head_dim)
    got = _run_decode(dw, q, k, v, kv_len, idx, cnt, scale).float().cpu().numpy()
    ref = oracle.sparse_decode_ref(q, k, v, dw.kv_lens, idx, cnt, scale, dw.block)
    assert np.isfinite(got).all()
    err = np.abs(got - ref).max()
    announce(f"decode {case}: max err {err:.2e}")
    assert err <= O_TOL
    for b, n in enumerate(dw.kv_lens):
        if n == 0:
            assert (got[b] == 0).all()


def test_sparse_decode_workspace_reuse():
    """One workspace reused across decode calls of different shapes (per-head and
    per-KV-head lists, several chunks per KV group): every call equals the same call
    on a fresh workspace bit for bit (nothing from an earlier call leaks in)."""
    cases = [("gqa4_d128_long", dict(batch=3, hq=8, hkv=2, tmax=9000, d=128,
                                     kv_lens=(9000, 4000, 1), block=64, list_heads="q"), 60),
             ("gqa4_d128_kv", dict(batch=2, hq=8, hkv=2, tmax=9000, d=128,
                                   kv_lens=(8000, 9000), block=64, list_heads="kv"), 100),
             ("gqa2_d64_b128", dict(batch=1, hq=4, hkv=2, tmax=3000, d=64, kv_lens=(2999,),
                                    block=128, list_heads="q"), 20)]
    big = max(seer.sparse_decode_workspace_size(c["batch"], c["hq"], c["hkv"], c["tmax"], c["d"],
                                                c["hq"] if c["list_heads"] == "q" else c["hkv"],
                                                mk, c["block"]) for _, c, mk in cases)
    ws = torch.full((big,), 0x7F, dtype=torch.uint8, device="cuda")  # garbage to start from
    for rep in range(2):
        for n, (name, c, max_k) in enumerate(cases):
            announce(f"decode workspace reuse {name} rep {rep}")
            dw = _decode_case(120 + n, **c)
            q, k, v, kv_len = wl.make_decode_inputs(dw)
            idx, cnt = _decode_lists(dw.wid + rep, dw, max_k)
            args = (_dev(q), _dev(k), _dev(v), _dev(kv_len), _dev(torch.from_numpy(idx)),
                    _dev(torch.from_numpy(cnt)), dw.block)
            fresh = seer.seer_sparse_decode(*args)
            reused = seer.seer_sparse_decode(*args, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(fresh.view(torch.int16), reused.view(torch.int16)), name
            ref = oracle.sparse_decode_ref(q, k, v, dw.kv_lens, idx, cnt,
                                           1.0 / math.sqrt(dw.head_dim), dw.block)
            assert float(np.abs(reused.float().cpu().numpy() - ref).max()) <= O_TOL


@pytest.mark.parametrize("seed", range(6))
def test_decode_seeded_sweep(seed):
    """Seeded random decode steps (ragged lengths including empty and one-token
    sequences, GQA 1-8, D 64/128, 64- or 128-token blocks, lists per query head or
    per KV head, TopK budgets or thresholds): GPU lists from the decode scores bit
    for bit against the oracle's, outputs against the oracle."""
    rng = np.random.default_rng(7000 + seed)
    hkv = int(rng.integers(1, 4))
    g = int(rng.choice([1, 2, 4, 5, 8]))
    b = int(rng.integers(1, 5))
    tmax = int(rng.integers(1, 3000))
    lens = [int(x) for x in rng.integers(0, tmax + 1, size=b)]
    lens[0] = tmax
    if b > 1:
        lens[1] = int(rng.choice([0, 1, tmax]))
    block = int(rng.choice([64, 128]))
    dw = _decode_case(300 + seed, b, hkv * g, hkv, tmax, int(rng.choice([64, 128])), lens,
                      block=block, list_heads=str(rng.choice(["q", "kv"])),
                      budget_tokens=block * int(rng.integers(1, 12)),
                      keep_sink=bool(rng.integers(0, 2)))
    mode = wl.MODE_TOPK if rng.integers(0, 2) else wl.MODE_THRESHOLD
    announce(f"decode sweep {seed}: b={b} hq={dw.hq} hkv={hkv} d={dw.head_dim} tmax={tmax} "
             f"lens={lens} block={block} lists={dw.list_heads} mode={mode} "
             f"budget={dw.budget_tokens} sink={dw.keep_sink}")
    q, k, v, kv_len = wl.make_decode_inputs(dw, tail_nan=True)
    s = wl.make_decode_scores(dw)
    thr = 2.0
    max_k = min(dw.nkb, max(dw.k_blocks, 2)) if mode == wl.MODE_TOPK else max(2, dw.nkb // 3)
    gi, gc = seer.seer_build_mask_decode(_dev(s), _dev(kv_len), block, mode, thr, dw.k_blocks,
                                         dw.keep_sink, max_k)
    ri, rc = oracle.build_mask_decode_ref(s.numpy(), lens, block, mode, thr, dw.k_blocks,
                                          dw.keep_sink, max_k)
    gi, gc = gi.cpu().numpy(), gc.cpu().numpy()
    assert (gc == rc).all() and (gi == ri).all()
    scale = 1.0 / math.sqrt(dw.head_dim)
    got = _run_decode(dw, q, k, v, kv_len, gi, gc, scale).float().cpu().numpy()
    ref = oracle.sparse_decode_ref(q, k, v, lens, gi, gc, scale, block)
    assert np.isfinite(got).all()
    err = float(np.abs(got - ref).max())
    announce(f"decode sweep {seed}: max err {err:.2e}")
    assert err <= O_TOL


def test_sparse_decode_shared_equals_repeated_per_head_lists():
    """Ascending shared lists and the same lists repeated per query head go through
    the direct and the union path; both visit the same tiles in the same order (at
    these sizes both grids are under one workgroup per CU, so both take the smallest
    chunk of blocks per workgroup)."""
    dw = _decode_case(90, 3, 8, 2, 3000, 128, (3000, 1234, 65), list_heads="kv")
    q, k, v, kv_len = wl.make_decode_inputs(dw)
    idx, cnt = _decode_lists(91, dw, 20)
    for b in range(dw.batch):
        for h in range(dw.lh):
            row = sorted(int(j) for j in idx[b, h, : cnt[b, h]]
                         if 0 <= j < (dw.kv_lens[b] + 63) // 64)
            idx[b, h] = -1
            idx[b, h, : len(row)] = row
            cnt[b, h] = len(row)
    shared = _run_decode(dw, q, k, v, kv_len, idx, cnt)
    g = dw.hq // dw.hkv
    per = _run_decode(dw, q, k, v, kv_len, np.ascontiguousarray(np.repeat(idx, g, axis=1)),
                      np.ascontiguousarray(np.repeat(cnt, g, axis=1)))
    assert torch.equal(shared, per)


@pytest.mark.parametrize("dw", [wl.DEC1, wl.DEC2], ids=lambda d: d.name)
def test_sparse_decode_bench_workload(dw):
    """The benchmarked decode step at full size: GPU lists from the decode scores,
    bit-exact against the oracle's; outputs of two sampled sequences (all heads)
    against the oracle."""
    announce(f"decode bench workload {dw.name}")
    q, k, v, kv_len = wl.make_decode_inputs(dw)
    s = wl.make_decode_scores(dw)
    max_k = min(dw.nkb, max(dw.k_blocks, 2))
    gi, gc = seer.seer_build_mask_decode(_dev(s), _dev(kv_len), dw.block, wl.MODE_TOPK, 0.0,
                                         dw.k_blocks, dw.keep_sink, max_k)
    ri, rc = oracle.build_mask_decode_ref(s.numpy(), dw.kv_lens, dw.block, wl.MODE_TOPK, 0.0,
                                          dw.k_blocks, dw.keep_sink, max_k)
    np.testing.assert_array_equal(gc.cpu().numpy(), rc)
    np.testing.assert_array_equal(gi.cpu().numpy(), ri)
    o = seer.seer_sparse_decode(_dev(q), _dev(k), _dev(v), _dev(kv_len), gi, gc, dw.block)
    torch.cuda.synchronize()
    got = o.float().cpu().numpy()
    assert np.isfinite(got).all()
    for b in (0, dw.batch - 1):
        ref = oracle.sparse_decode_ref(q[b:b + 1], k[b:b + 1], v[b:b + 1], [dw.kv_lens[b]],
                                       ri[b:b + 1], rc[b:b + 1], None, dw.block)
        err = np.abs(got[b:b + 1] - ref).max()
        announce(f"decode {dw.name} seq {b}: max err {err:.2e}")
        assert err <= O_TOL


def test_sparse_decode_repeat_bitexact():
    dw = _decode_case(92, 2, 32, 8, 8192, 128, (8192, 5000), list_heads="q")
    q, k, v, kv_len = wl.make_decode_inputs(dw)
    idx, cnt = _decode_lists(93, dw, 40)
    a = _run_decode(dw, q, k, v, kv_len, idx, cnt)
    b = _run_decode(dw, q, k, v, kv_len, idx, cnt)
    assert torch.equal(a, b)


def test_sparse_decode_kv_len_clamped():
    """kv_len values above Tmax act as Tmax and negative ones as 0 (the call's
    documented clamping): compared with the oracle on the clamped lengths."""
    dw = _decode_case(94, 3, 4, 2, 640, 128, (640, 0, 300), list_heads="q")
    q, k, v, _ = wl.make_decode_inputs(dw)
    idx, cnt = _decode_lists(95, dw, 6)
    given = torch.tensor([640 + 100, -5, 300], dtype=torch.int32)
    got = _run_decode(dw, q, k, v, given, idx, cnt).float().cpu().numpy()
    ref = oracle.sparse_decode_ref(q, k, v, [640, 0, 300], idx, cnt, None, dw.block)
    assert np.abs(got - ref).max() <= O_TOL
    assert (got[1] == 0).all()
