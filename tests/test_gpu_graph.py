"""The mask build and the no-allocation sparse prefill captured in a HIP graph
(the callers that entry point is for): every replay, with new inputs written in
place in between and eager work and a synchronisation before it, must give lists
and outputs bit-identical to the same calls made eagerly.  The library issues no
memset and allocates nothing, so its launches are all a capture records."""

import pytest
import torch

import block_sparse_attention_prefill_amd as seer
from block_sparse_attention_prefill_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _inputs(w, seed_shift):
    """Seeded inputs of workload w, drawn from a shifted workload id so that each
    replay sees different values of the same shapes."""
    ws = wl.custom(w.wid + seed_shift, w.batch, w.hq, w.hkv, w.head_dim, w.seq, mode=w.mode,
                   density=w.density, threshold=w.threshold, keep_sink=w.keep_sink,
                   scores=w.scores)
    q, k, v = (t.to("cuda") for t in wl.make_qkv(ws))
    return q, k, v, wl.make_scores(ws).to("cuda")


@pytest.mark.parametrize("mode", [wl.MODE_TOPK, wl.MODE_THRESHOLD])
def test_graph_replays_match_eager(mode):
    assert torch.cuda.is_available()
    seer.load()
    # Llama-like group of 4 query heads on 2 KV heads, ragged T, head dim 128
    w = wl.custom(61, 1, 8, 2, 128, 2048 + 37, mode=mode, density=0.3, threshold=2e-3,
                  keep_sink=True,
                  scores="local_stripe" if mode == wl.MODE_TOPK else "softmax_normal")
    nb = w.nqb
    max_k = seer.topk_budget(nb, w.density, w.keep_sink) if mode == wl.MODE_TOPK else nb
    q, k, v, s = _inputs(w, 0)
    idx = torch.empty((w.batch, w.hq, nb, max_k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((w.batch, w.hq, nb), dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)

    def step():
        seer.seer_build_mask(s, mode, w.threshold, w.density, w.keep_sink, max_k, kv_idx=idx,
                             kv_cnt=cnt)
        seer.seer_sparse_prefill_noalloc(q, k, v, idx, cnt, out=out)

    # eager calls first: the scratch address lookup happens outside the capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for r in range(3):
        nq, nk, nv, ns = _inputs(w, 100 + r)
        q.copy_(nq)
        k.copy_(nk)
        v.copy_(nv)
        s.copy_(ns)
        out.fill_(float("nan"))
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        # the eager reference on the same inputs, into buffers of its own
        ref_idx, ref_cnt = seer.seer_build_mask(ns, mode, w.threshold, w.density, w.keep_sink,
                                                max_k)
        ref_out = seer.seer_sparse_prefill(nq, nk, nv, ref_idx, ref_cnt)
        torch.cuda.synchronize()
        assert torch.equal(cnt, ref_cnt), f"replay {r}: counts"
        assert torch.equal(idx, ref_idx), f"replay {r}: lists"
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"replay {r}: O"
        assert int(ref_cnt.sum()) > nb * w.hq  # more than the diagonal alone
