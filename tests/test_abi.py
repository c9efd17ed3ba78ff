"""CPU-side checks of the C-ABI: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any launch."""

import ctypes
import os
import re

import pytest

import block_sparse_attention_prefill_amd as seer
from block_sparse_attention_prefill_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "seer.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(seer_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared() == sorted(binding.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = seer.load()
    for name in _declared():
        assert hasattr(lib, name), name
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_status_strings_and_version():
    lib = seer.load()
    assert lib.seer_status_string(0) == b"SEER_OK"
    assert lib.seer_status_string(3) == b"SEER_ERR_CAPACITY"
    assert lib.seer_status_string(99) == b"SEER_ERR_UNKNOWN"
    assert seer.version() >= 100


def test_topk_budget_host_helper():
    assert seer.topk_budget(512, 0.1, True) == 52
    assert seer.topk_budget(2048, 0.17, True) == 349
    assert seer.topk_budget(8, 0.5, True) == 4
    assert seer.topk_budget(1, 0.01, True) == 1
    assert seer.topk_budget(8, 0.0, True) == -1
    assert seer.topk_budget(8, 1.5, True) == -1


def test_workspace_sizes():
    assert seer.sparse_prefill_workspace_size(1, 32, 8, 32768) >= 32 * 512 * 4
    assert seer.sparse_prefill_workspace_size(1, 32, 7, 32768) == 0  # Hq % Hkv != 0
    # 64 fp32 per causal tile: 40 heads * 512*513/2 tiles at 32k tokens.
    assert seer.pooled_attn_map_workspace_size(1, 40, 32768) >= 40 * (512 * 513 // 2) * 64 * 4
    assert seer.pooled_attn_map_workspace_size(1, 0, 64) == 0
    # gate: Q~, K~, tile partials, pooled Q and K (fp32)
    nqb, nt = 512, 8
    floats = (32 + 8) * nqb * 128 + 2 * 32 * nqb * nt + (32 + 2 * 8) * nqb * 128
    assert seer.attn_gate_workspace_size(1, 32, 8, 32768, 128) >= floats * 4
    assert seer.attn_gate_workspace_size(1, 32, 7, 32768, 128) == 0  # Hq % Hkv != 0
    # fused gate + mask: the same, plus the logits map when no scores buffer is given
    with_s = seer.attn_gate_mask_workspace_size(1, 32, 8, 32768, 128, True)
    without = seer.attn_gate_mask_workspace_size(1, 32, 8, 32768, 128, False)
    assert with_s == seer.attn_gate_workspace_size(1, 32, 8, 32768, 128)
    assert without == with_s + 32 * 512 * 512 * 4
    assert seer.attn_gate_mask_workspace_size(1, 32, 7, 32768, 128, True) == 0
    # passes of tile rows: one row of tiles is 64 logit rows of nQB per head
    one = seer.attn_gate_mask_pass_workspace_size(1, 32, 8, 32768, 128, 1)
    assert one == with_s + 32 * 64 * 512 * 4
    assert seer.attn_gate_mask_pass_workspace_size(1, 32, 8, 32768, 128, 3) == \
        with_s + 32 * 192 * 512 * 4
    assert seer.attn_gate_mask_pass_workspace_size(1, 32, 8, 32768, 128, 8) == without
    assert seer.attn_gate_mask_pass_workspace_size(1, 32, 8, 32768, 128, 1000) == without
    assert seer.attn_gate_mask_pass_workspace_size(1, 32, 8, 32768, 128, 0) == 0
    # a ragged T: the last tile row holds fewer than 64 rows
    assert seer.attn_gate_mask_pass_workspace_size(1, 4, 2, 64 * 100, 64, 2) == \
        seer.attn_gate_mask_workspace_size(1, 4, 2, 64 * 100, 64, False)


FAKE = 1 << 20  # never dereferenced: every call below fails its host checks first


@pytest.mark.parametrize("args,status", [
    # mode
    ((FAKE, 1, 1, 4, 4, 7, 0.0, 0.5, 1, FAKE, FAKE, 4, None), 1),
    # nKB < nQB
    ((FAKE, 1, 1, 4, 3, 1, 0.0, 0.5, 1, FAKE, FAKE, 4, None), 1),
    # density out of range
    ((FAKE, 1, 1, 4, 4, 1, 0.0, 0.0, 1, FAKE, FAKE, 4, None), 1),
    # threshold not finite
    ((FAKE, 1, 1, 4, 4, 0, float("nan"), 0.5, 1, FAKE, FAKE, 4, None), 1),
    # max_k below the TopK budget (4 blocks at density 1 need 4)
    ((FAKE, 1, 1, 4, 4, 1, 0.0, 1.0, 1, FAKE, FAKE, 3, None), 3),
    # max_k cannot hold diagonal + sink
    ((FAKE, 1, 1, 4, 4, 0, 0.1, 0.5, 1, FAKE, FAKE, 1, None), 3),
    # null output
    ((FAKE, 1, 1, 4, 4, 1, 0.0, 0.5, 1, None, FAKE, 4, None), 1),
    # row longer than SEER_MAX_QUERY_BLOCKS
    ((FAKE, 1, 1, 4097, 4097, 1, 0.0, 0.5, 1, FAKE, FAKE, 4097, None), 2),
])
def test_build_mask_rejects_on_host(args, status):
    assert seer.load().seer_build_mask(*args) == status


def test_build_mask_need_rejects_on_host():
    lib = seer.load()
    ok = (FAKE, 1, 1, 4, 4, 1, 0.0, 0.5, 1, FAKE, FAKE, FAKE, 4, None)
    bad = [((1,), None),            # null kv_need
           ((5,), 7),               # mode
           ((4,), 3),               # nKB < nQB
           ((7,), 0.0),             # density out of range
           ((12,), 1)]              # max_k below the TopK budget (ceil(0.5 * 4) = 2 + sink)
    for (pos,), val in bad:
        a = list(ok)
        if pos == 1:
            a[11] = None
            want = 1
        else:
            a[pos] = val
            want = 3 if pos == 12 else 1
        assert lib.seer_build_mask_need(*a) == want, (pos, val)
    a = list(ok)
    a[3], a[4], a[12] = 4097, 4097, 4097
    assert lib.seer_build_mask_need(*a) == 2
    a = list(ok)
    a[1] = 0
    a[11] = None
    assert lib.seer_build_mask_need(*a) == 0  # nothing to do: nothing needed, nothing launched


def test_validate_lists_rejects_on_host():
    lib = seer.load()
    v = lambda *a: lib.seer_validate_lists(*a)
    assert v(FAKE, FAKE, None, -1, 1, 4, 4, None, FAKE, None) == 1
    assert v(FAKE, FAKE, None, 1, 1, -4, 4, None, FAKE, None) == 1
    assert v(FAKE, FAKE, None, 1, 1, 4, 0, None, FAKE, None) == 1      # max_k < 1
    assert v(FAKE, FAKE, None, 1, 1, 4, 4, None, None, None) == 1      # no flags output
    assert v(None, FAKE, None, 1, 1, 4, 4, None, FAKE, None) == 1
    assert v(FAKE, None, None, 1, 1, 4, 4, None, FAKE, None) == 1
    assert v(FAKE, FAKE, None, 1 << 20, 1 << 10, 1 << 10, 4, None, FAKE, None) == 2


def test_list_flags_status_host_helper():
    st = seer.list_flags_status
    assert st(0) == 0
    assert st(seer.SEER_LIST_UNSORTED | seer.SEER_LIST_BAD_ENTRY | seer.SEER_LIST_BAD_COUNT) == 0
    assert st(seer.SEER_LIST_REPEAT) == 1
    assert st(seer.SEER_LIST_CAPACITY | seer.SEER_LIST_REPEAT) == 3
    assert st(seer.SEER_LIST_CAPACITY) == 3


def _prefill(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, B=1, Hq=4, Hkv=2, T=128, D=128, scale=0.1, idx=FAKE,
             cnt=FAKE, max_k=2, o=FAKE, ws=FAKE, wsb=1 << 20, stream=None)
    a.update(kw)
    return seer.load().seer_sparse_prefill(*a.values())


def test_sparse_prefill_rejects_on_host():
    assert _prefill(D=96) == 2
    assert _prefill(Hkv=3) == 1
    assert _prefill(scale=0.0) == 1
    assert _prefill(scale=float("inf")) == 1
    assert _prefill(q=None) == 1
    assert _prefill(q=FAKE + 8) == 1          # misaligned
    assert _prefill(max_k=0) == 1
    assert _prefill(ws=None) == 4
    assert _prefill(wsb=16) == 4
    assert _prefill(ws=FAKE + 16) == 4        # workspace not 256-byte aligned
    assert _prefill(T=0) == 0                 # nothing to do, nothing launched
    assert _prefill(B=0) == 0


def test_pooled_map_rejects_on_host():
    lib = seer.load()
    ok = (FAKE, FAKE, FAKE, 1, 4, 2, 128, 128, 0.1, FAKE, FAKE, FAKE, 1 << 20, None)
    bad_d = ok[:7] + (80,) + ok[8:]
    assert lib.seer_pooled_attn_map(*bad_d) == 2
    no_map = ok[:10] + (None,) + ok[11:]
    assert lib.seer_pooled_attn_map(*no_map) == 1
    small_ws = ok[:12] + (64,) + ok[13:]
    assert lib.seer_pooled_attn_map(*small_ws) == 4


def test_pooled_target_rejects_on_host():
    lib = seer.load()
    ok = (FAKE, FAKE, 1, 2, 8, FAKE, FAKE, FAKE, None)
    assert lib.seer_pooled_target_mse(*((None,) + ok[1:])) == 1          # no map
    assert lib.seer_pooled_target_mse(*(ok[:5] + (None,) + ok[6:])) == 1  # no target
    assert lib.seer_pooled_target_mse(*(ok[:1] + (None,) + ok[2:])) == 1  # loss without gate
    assert lib.seer_pooled_target_mse(*(ok[:6] + (None,) + ok[7:])) == 1  # loss without row_sse
    assert lib.seer_pooled_target_mse(FAKE, FAKE, -1, 2, 8, FAKE, FAKE, FAKE, None) == 1
    assert lib.seer_pooled_target_mse(FAKE, FAKE, 0, 2, 8, FAKE, FAKE, FAKE, None) == 0  # empty


def test_sparse_prefill_block_rejects_on_host():
    lib = seer.load()
    a = [FAKE, FAKE, FAKE, 1, 4, 2, 128, 128, 0.1, 128, FAKE, FAKE, 2, FAKE, FAKE, 1 << 20, None]
    for bad_block in (32, 96, 256, 0):
        a2 = list(a)
        a2[9] = bad_block
        assert lib.seer_sparse_prefill_block(*a2) == 2
    a2 = list(a)
    a2[7] = 80          # head dim
    assert lib.seer_sparse_prefill_block(*a2) == 2
    a2 = list(a)
    a2[14] = None       # workspace
    assert lib.seer_sparse_prefill_block(*a2) == 4


def test_attn_gate_rejects_on_host():
    lib = seer.load()
    a = [FAKE, FAKE, 1, 4, 2, 256, 128, FAKE, FAKE, 64, 0.125, 10000.0, FAKE, FAKE, 1 << 20, None]
    def call(**kw):
        b = list(a)
        for i, v in kw.items():
            b[int(i[1:])] = v
        return lib.seer_attn_gate_scores(*b)
    assert call(p6=96) == 2            # head dim
    assert call(p9=48) == 2            # gate dim
    assert call(p4=3) == 1             # Hq % Hkv
    assert call(p10=0.0) == 1          # scale
    assert call(p11=1.0) == 1          # rope base
    assert call(p7=None) == 1          # weights
    assert call(p13=None) == 4         # workspace
    assert call(p2=0) == 0             # empty
    assert seer.load().seer_attn_gate_workspace_size(1, 4, 2, 256, 64) >= (4 + 2) * 4 * 64 * 4



def test_attn_gate_mask_rejects_on_host():
    lib = seer.load()
    # q, k, B, Hq, Hkv, T, D, wq, wk, Dg, scale, rope_base, mode, threshold, density,
    # keep_sink, kv_idx, kv_cnt, max_k, scores, workspace, workspace_bytes, stream.
    # The base call fails only on its 16-byte workspace, so nothing ever launches.
    a = [FAKE, FAKE, 1, 4, 2, 256, 128, FAKE, FAKE, 64, 0.125, 10000.0, 1, 0.0, 0.5, 1, FAKE,
         FAKE, 3, FAKE, FAKE, 16, None]
    def call(**kw):
        b = list(a)
        for i, v in kw.items():
            b[int(i[1:])] = v
        return lib.seer_attn_gate_mask(*b)
    assert call() == 4                 # workspace too small
    assert call(p6=96) == 2            # head dim
    assert call(p9=48) == 2            # gate dim
    assert call(p4=3) == 1             # Hq % Hkv
    assert call(p10=0.0) == 1          # scale
    assert call(p12=5) == 1            # mode
    assert call(p14=0.0) == 1          # density
    assert call(p12=0, p13=float("inf")) == 1  # threshold
    assert call(p18=0) == 3            # max_k < 1
    assert call(p18=1) == 3            # under the TopK budget (2 of 4 blocks)
    assert call(p12=0, p15=1, p18=1) == 3  # threshold with sink needs 2 slots
    assert call(p5=64 * 4097) == 2     # more than SEER_MAX_QUERY_BLOCKS blocks
    assert call(p16=None) == 1         # lists
    assert call(p7=None) == 1          # weights
    assert call(p2=0) == 0             # empty
    # without scores the workspace must hold at least one tile row of logits
    gate = seer.attn_gate_workspace_size(1, 4, 2, 256, 64)
    one = seer.attn_gate_mask_pass_workspace_size(1, 4, 2, 256, 64, 1)
    assert one > gate
    assert call(p19=None, p21=gate) == 4
    assert call(p19=None, p21=one - 1) == 4
    assert call(p21=gate - 1) == 4     # with scores the gate's own part is the minimum


def test_attn_gate_decode_rejects_on_host():
    lib = seer.load()
    # scores call: q, k_gate, kv_len, B, Hq, Hkv, Tmax, D, wq, Dg, scale, rope_base, block,
    # scores, stream.  No call here passes every check, so nothing ever launches.
    a = [FAKE, FAKE, FAKE, 2, 4, 2, 700, 128, FAKE, 64, 0.125, 10000.0, 64, None, None]
    def call(**kw):
        b = list(a)
        for i, v in kw.items():
            b[int(i[1:])] = v
        return lib.seer_attn_gate_decode_scores(*b)
    assert call() == 1                 # scores
    assert call(p7=96) == 2            # head dim
    assert call(p9=48) == 2            # gate dim
    assert call(p12=32) == 2           # block
    assert call(p4=3) == 1             # Hq % Hkv
    assert call(p6=0) == 1             # Tmax
    assert call(p6=64 * 4097) == 2     # more than SEER_MAX_QUERY_BLOCKS blocks
    assert call(p10=-1.0) == 1         # scale
    assert call(p11=0.5) == 1          # rope base
    assert call(p13=FAKE, p2=None) == 1  # kv_len
    assert call(p13=FAKE, p1=None) == 1  # k_gate
    assert call(p3=0) == 0             # empty batch
    # keys call: k_cache, kv_len, B, Hkv, Tmax, D, wk, Dg, rope_base, block, last_only,
    # k_gate, workspace, workspace_bytes, stream.  The all-block base call fails only
    # on its 16-byte workspace; every last-block call here lacks k_gate.
    k = [FAKE, FAKE, 2, 2, 700, 128, FAKE, 64, 10000.0, 64, 0, FAKE, FAKE, 16, None]
    def kcall(**kw):
        b = list(k)
        for i, v in kw.items():
            b[int(i[1:])] = v
        return lib.seer_attn_gate_decode_keys(*b)
    assert kcall() == 4                # workspace too small for the all-block pass
    assert kcall(p5=96) == 2 and kcall(p7=48) == 2 and kcall(p9=256) == 2
    assert kcall(p8=1.0) == 1 and kcall(p11=None) == 1 and kcall(p0=None) == 1
    assert kcall(p10=1, p11=None) == 1  # last block only still needs k_gate
    assert kcall(p2=0) == 0
    ws = lib.seer_attn_gate_decode_keys_workspace_size
    assert ws(8, 8, 40960, 128, 64) >= 8 * 8 * 640 * 256 * 4
    assert ws(8, 8, 40960, 128, 128) < ws(8, 8, 40960, 128, 64)
    assert ws(8, 8, 0, 128, 64) == 0


def test_attn_gate_decode_mask_rejects_on_host():
    lib = seer.load()
    # q, k_gate, kv_len, B, Hq, Hkv, Tmax, D, wq, Dg, scale, rope_base, block, mode,
    # threshold, k_blocks, keep_sink, kv_idx, kv_cnt, max_k, scores, stream (nKB = 11).
    # The base call lacks kv_cnt, and every call that supplies it lacks another pointer.
    a = [FAKE, FAKE, FAKE, 2, 4, 2, 700, 128, FAKE, 64, 0.125, 10000.0, 64, 1, 0.0, 4, 1,
         FAKE, None, 16, None, None]
    def call(**kw):
        b = list(a)
        for i, v in kw.items():
            b[int(i[1:])] = v
        return lib.seer_attn_gate_decode_mask(*b)
    assert call() == 1                 # kv_cnt
    assert call(p7=96) == 2            # head dim
    assert call(p9=48) == 2            # gate dim
    assert call(p12=32) == 2           # block
    assert call(p6=64 * 4097) == 2     # more than SEER_MAX_QUERY_BLOCKS blocks
    assert call(p4=3) == 1             # Hq % Hkv
    assert call(p10=-1.0) == 1         # scale
    assert call(p11=0.5) == 1          # rope base
    assert call(p13=7) == 1            # mode
    assert call(p15=0) == 1            # TopK budget
    assert call(p19=3) == 3            # max_k below the budget
    assert call(p15=40, p19=10) == 3   # budget capped at nKB = 11
    assert call(p15=40, p19=11) == 1   # enough room: fails on kv_cnt
    assert call(p13=0, p14=float("nan")) == 1  # threshold
    assert call(p13=0, p19=1) == 3     # sink + last block need 2
    assert call(p19=0) == 3
    assert call(p19=1 << 30) == 2      # B * Hq * max_k over int32
    assert call(p18=FAKE, p0=None) == 1 and call(p18=FAKE, p1=None) == 1
    assert call(p18=FAKE, p2=None) == 1 and call(p18=FAKE, p8=None) == 1
    assert call(p18=FAKE, p17=None) == 1
    assert call(p18=FAKE, p1=FAKE + 4) == 1     # k_gate not 16-byte aligned
    assert call(p3=0) == 0             # empty batch


def test_build_mask_decode_rejects_on_host():
    lib = seer.load()
    # scores, kv_len, B, H, nKB, block, mode, threshold, k_blocks, keep_sink, idx, cnt, max_k
    a = [FAKE, FAKE, 2, 8, 640, 64, 1, 0.0, 64, 1, FAKE, FAKE, 64, None]
    def call(**kw):
        b = list(a)
        for i, v in kw.items():
            b[int(i[1:])] = v
        return lib.seer_build_mask_decode(*b)
    assert call(p5=96) == 2            # block size
    assert call(p4=4097) == 2          # row longer than the mask kernel takes
    assert call(p6=7) == 1             # mode
    assert call(p8=0) == 1             # TopK budget
    assert call(p12=63) == 3           # max_k below the budget
    assert call(p4=40, p12=39) == 3    # budget capped at nKB = 40
    assert call(p6=0, p7=float("inf")) == 1   # threshold
    assert call(p6=0, p12=1) == 3      # sink + last block need 2
    assert call(p0=None) == 1 and call(p1=None) == 1
    assert call(p2=-1) == 1
    assert call(p2=0) == 0             # empty


def test_sparse_decode_rejects_on_host():
    lib = seer.load()
    # q, k, v, kv_len, B, Hq, Hkv, Tmax, D, scale, block, idx, cnt, list_heads, max_k, o, ws, bytes, s
    a = [FAKE, FAKE, FAKE, FAKE, 2, 32, 8, 4096, 128, 0.088, 64, FAKE, FAKE, 8, 64, FAKE, FAKE,
         1 << 30, None]
    def call(**kw):
        b = list(a)
        for i, v in kw.items():
            b[int(i[1:])] = v
        return lib.seer_sparse_decode(*b)
    assert call(p8=96) == 2            # head dim
    assert call(p10=32) == 2           # block size
    assert call(p5=72) == 2            # 9 query heads per KV head
    assert call(p5=30) == 1            # Hq % Hkv
    assert call(p13=16) == 1           # list heads neither Hq nor Hkv
    assert call(p7=0) == 1             # empty cache capacity
    assert call(p7=64 * 32769) == 2    # more blocks than the union flags hold
    assert call(p9=0.0) == 1 and call(p9=float("nan")) == 1
    assert call(p14=0) == 1            # max_k
    assert call(p3=None) == 1 and call(p15=None) == 1
    assert call(p16=None) == 4         # workspace
    assert call(p17=1024) == 4         # workspace too small
    assert call(p4=0) == 0             # empty batch
    ws = lib.seer_sparse_decode_workspace_size
    assert ws(2, 32, 8, 4096, 128, 8, 64, 64) > 0
    assert ws(2, 32, 8, 4096, 128, 32, 64, 64) > ws(2, 32, 8, 4096, 128, 8, 64, 64)
    assert ws(2, 32, 8, 4096, 128, 16, 64, 64) == 0
    assert ws(2, 32, 8, 0, 128, 8, 64, 64) == 0


def test_decode_workspace_follows_chunk_rule():
    """The decode workspace holds one partial per chunk of listed blocks; a chunk is
    the largest of 1024, 512, 256, 128 tokens that still gives each of the 256 CUs a
    workgroup (B * Hkv * chunks >= 256), else 128 tokens."""
    a256 = lambda x: (x + 255) // 256 * 256
    def expect(b, hq, hkv, tmax, d, lh, max_k, bs):
        g, groups, nbmax = hq // hkv, b * hkv, (tmax + bs - 1) // bs
        union = lh == hq and g > 1
        umax = min(g * max_k, nbmax) if union else max_k
        for tok in (1024, 512, 256, 128):
            chunk = max(1, tok // bs)
            nsplit = max(1, (umax + chunk - 1) // chunk)
            if groups * nsplit >= 256:
                break
        off = a256(groups * umax * 4) + a256(groups * 4) if union else 0
        return off + a256(groups * nsplit * g * 2 * 4) + a256(groups * nsplit * g * d * 4) + 256
    for args in [(8, 32, 8, 40960, 128, 8, 64, 64),    # 1024-token chunks, 256 workgroups
                 (8, 32, 8, 40960, 128, 32, 64, 64),   # union of per-head lists
                 (1, 32, 8, 40960, 128, 8, 64, 64),    # small grid: 128-token chunks
                 (2, 8, 2, 3000, 64, 8, 20, 128),      # 128-token blocks
                 (4, 32, 8, 16384, 128, 8, 32, 64)]:   # 256-token chunks
        assert seer.sparse_decode_workspace_size(*args) == expect(*args), args
