"""The no-allocation prefill entry point (static scratch instead of a caller
workspace) against seer_sparse_prefill with a workspace: the same kernels, so
the outputs must be bit-identical, on two calls in a row (the second smaller),
with the library's scratch keeping the first call's contents in between."""

import numpy as np
import pytest
import torch

import oracle
import block_sparse_attention_prefill_amd as seer
from block_sparse_attention_prefill_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _case(w):
    q, k, v = (t.to("cuda") for t in wl.make_qkv(w))
    s = wl.make_scores(w).to("cuda")
    max_k = seer.topk_budget(w.nqb, w.density, w.keep_sink) if w.mode == wl.MODE_TOPK else w.nqb
    idx, cnt = seer.seer_build_mask(s, w.mode, w.threshold, w.density, w.keep_sink, max_k)
    return q, k, v, idx, cnt


def test_noalloc_matches_workspace_call_twice():
    assert torch.cuda.is_available()
    seer.load()
    big = wl.C2  # Llama 32/8/128, 8192 tokens, threshold lists (4096 items)
    small = wl.custom(41, 1, 4, 2, 64, 1000, mode=wl.MODE_TOPK, density=0.3, keep_sink=True,
                      scores="local_stripe")  # ragged, head dim 64, 64 items
    outs = []
    for w in (big, small):
        q, k, v, idx, cnt = _case(w)
        ref = seer.seer_sparse_prefill(q, k, v, idx, cnt)
        got = torch.full_like(q, float("nan"))
        seer.seer_sparse_prefill_noalloc(q, k, v, idx, cnt, out=got)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), w.name
        outs.append((w, q, k, v, idx, cnt, got))
    # the smaller call's output also against the oracle (the parity bar)
    w, q, k, v, idx, cnt, got = outs[1]
    ro = oracle.sparse_attention_ref(q.cpu(), k.cpu(), v.cpu(), idx.cpu().numpy(),
                                     cnt.cpu().numpy(), None)
    assert float(np.abs(got.cpu().double().numpy() - ro).max()) <= 2e-2


def test_noalloc_rejects_sizes_beyond_scratch():
    seer.load()
    fake = 1 << 12
    lib = seer.load()
    # 8 x 64 heads x 1024 blocks = 524288 items > 262144: refused before any launch
    st = lib.seer_sparse_prefill_noalloc(fake, fake, fake, 8, 64, 8, 65536, 128, 0.1, fake, fake,
                                         4, fake, None)
    assert st == 4  # SEER_ERR_WORKSPACE
