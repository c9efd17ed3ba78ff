"""Argument checks of the Python binding that need a GPU to reach: a caller's
workspace must be contiguous device memory of the current device (the library
itself can only check its size and alignment), and the call is refused before
anything is launched."""

import pytest
import torch

import block_sparse_attention_prefill_amd as seer
from block_sparse_attention_prefill_amd import workloads as wl

pytestmark = pytest.mark.gpu


def test_caller_workspace_must_be_device_memory():
    seer.load()
    w = wl.custom(51, 1, 4, 2, 64, 300, mode=wl.MODE_TOPK, density=0.5, keep_sink=True,
                  scores="uniform")
    q, k, v = (t.to("cuda") for t in wl.make_qkv(w))
    s = wl.make_scores(w).to("cuda")
    max_k = seer.topk_budget(w.nqb, w.density, w.keep_sink)
    idx, cnt = seer.seer_build_mask(s, w.mode, w.threshold, w.density, w.keep_sink, max_k)
    need = seer.sparse_prefill_workspace_size(w.batch, w.hq, w.hkv, w.seq)
    with pytest.raises(ValueError, match="workspace must be a GPU tensor"):
        seer.seer_sparse_prefill(q, k, v, idx, cnt, workspace=torch.empty(need, dtype=torch.uint8))
    strided = torch.empty(2 * need, dtype=torch.uint8, device="cuda")[::2]
    with pytest.raises(ValueError, match="contiguous"):
        seer.seer_sparse_prefill(q, k, v, idx, cnt, workspace=strided)
    # a proper caller workspace gives the same output as the binding's own
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    a = seer.seer_sparse_prefill(q, k, v, idx, cnt, workspace=ws)
    b = seer.seer_sparse_prefill(q, k, v, idx, cnt)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
